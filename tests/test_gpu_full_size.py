"""Full-size workloads in the launch configuration the benchmark times (block index,
reorder with XCD slicing, attention through the permutation, G, W, Top-p), with
sampled outputs checked row by row against the fp64 oracle and whole-output
properties checked everywhere."""

import numpy as np
import pytest
import torch

import cache_aware_query_amd as caq
import oracle
import synth
from cache_aware_query_amd.pipeline import HotPath
from helpers import assert_attention_close, banner, gpu, np64

pytestmark = pytest.mark.gpu


def _run_full(name):
    dev = gpu()
    banner(f"full-size {name}: generating")
    w = synth.make_workload(name, device=dev)
    H, mb = w.mask.shape[0], w.mask.shape[1]
    nnz = int(w.mask.sum())
    _, _, wave = caq.schedule_info(0, w.head_dim)
    params = caq.ReorderParams(wave=wave, n_slices=8, skip_mode=caq.WA_SKIP_NEVER)
    hp = HotPath(H, w.seq_len, w.head_dim, w.block, dev, capacity=nnz, reorder=params, gsrs_p=0.9)
    banner(f"full-size {name}: H={H} MB={mb} nnz={nnz} wave={wave}")
    hp.step(w.q, w.k, w.v, w.mask, w.x0)
    torch.cuda.synchronize()
    return w, hp


def _sample_rows(w, rng, n_heads=4, n_blocks=3):
    H, mb = w.mask.shape[0], w.mask.shape[1]
    L, b = w.seq_len, w.block
    heads = sorted(set([0, H - 1] + rng.choice(H, size=n_heads, replace=False).tolist()))
    out = []
    for h in heads:
        blocks = sorted(set([mb - 1] + rng.choice(mb, size=n_blocks, replace=False).tolist()))
        for u in blocks:
            r0, r1 = u * b, min((u + 1) * b, L)
            rows = np.unique(np.concatenate([[r0, r1 - 1], rng.integers(r0, r1, size=6)]))
            out.append((h, u, rows))
    return out


@pytest.mark.parametrize("name", ["wan75k", "hunyuan119k"])
def test_full_size_attention_sampled(name):
    w, hp = _run_full(name)
    rng = np.random.default_rng(7)
    o = hp.o
    lse = hp.lse
    assert not torch.isnan(o[:, : w.seq_len]).any()
    assert not torch.isnan(lse[:, : w.seq_len]).any()
    perm = hp.perm.cpu().numpy()
    for h in range(perm.shape[0]):
        assert sorted(perm[h].tolist()) == list(range(perm.shape[1]))
    for h, u, rows in _sample_rows(w, rng):
        qh, kh, vh = (np64(t[h]) for t in (w.q, w.k, w.v))
        o_ref, l_ref = oracle.masked_attention_rows(qh, kh, vh, w.mask[h].cpu().numpy(), rows,
                                                    w.seq_len, w.block, w.scale)
        assert_attention_close(np64(o[h])[rows], lse[h].cpu().numpy().astype(np.float64)[rows],
                               o_ref, l_ref, f"{name} h={h} u={u}")
    stats = hp.stats.cpu().numpy()
    print(f"{name}: density per head {np.round(stats[:, 1], 4).tolist()}")


def test_full_size_gsrs_dense_pass_sampled():
    w, hp = _run_full("gsrs75k")
    rng = np.random.default_rng(9)
    H, mb = w.mask.shape[0], w.mask.shape[1]
    L, b = w.seq_len, w.block
    rp = hp.row_ptr.cpu().numpy()
    wts = hp.w.cpu().numpy().astype(np.float64)
    # every row of W sums to one over the dense candidate set
    sums = wts[: rp[-1]].reshape(H * mb, mb).sum(1)
    np.testing.assert_allclose(sums, 1.0, atol=1e-4)
    sel = hp.next_mask.cpu().numpy()
    assert 0 < sel.sum() < H * mb * mb
    for h in sorted(set([0, H - 1, int(rng.integers(H))])):
        for u in sorted(set([mb - 1, int(rng.integers(mb))])):
            sub = np.zeros((1, mb, mb), dtype=np.uint8)
            sub[0, u] = 1
            srp, sci, _, _, _ = oracle.block_index(sub)
            q, k = np64(w.q[h:h + 1]), np64(w.k[h:h + 1])
            g_ref, lse_ref = oracle.block_lse(q, k, srp, sci, L, b, w.scale)
            w_ref = oracle.block_importance(g_ref, lse_ref, srp, L, b)
            nrows = min(b, L - u * b)
            lo = rp[h * mb + u]
            g_gpu = hp.g[lo:lo + mb, :nrows].cpu().numpy().astype(np.float64)
            np.testing.assert_allclose(g_gpu, g_ref[:, :nrows], atol=5e-3, rtol=0)
            np.testing.assert_allclose(wts[lo:lo + mb], w_ref, atol=2e-4, rtol=1e-3)
            banner(f"gsrs75k h={h} u={u} kept {int(sel[h, u].sum())} of {mb}")


def _row_csr(cols, mb):
    """One-row CSR of the given block ids (ascending) for the oracle's per-row calls."""
    sub = np.zeros((1, 1, mb), dtype=np.uint8)
    sub[0, 0, cols] = 1
    rp, ci, _, _, _ = oracle.block_index(sub)
    return rp, ci


def test_full_size_gsrs_search_step_sampled():
    """The GSRS search step at full size, in the configuration the bench times (the
    calibrated reorder), checked on sampled query blocks: S1 is Top-p at 0.9 of the
    dense pass's W (bit-exact); the pass over S1 gives W within tolerance of the
    oracle's over the same candidates; S2 is Top-p at 0.8 of that W (bit-exact) and
    lies inside S1 everywhere; the pass over S2 matches the oracle's attention."""
    from cache_aware_query_amd.pipeline import GsrsSearch
    dev = gpu()
    banner("full-size gsrs75k search step: generating")
    w = synth.make_workload("gsrs75k", device=dev)
    H, mb = w.mask.shape[0], w.mask.shape[1]
    L, b, d = w.seq_len, w.block, w.head_dim
    n_xcd, _, wave = caq.schedule_info(0, d)
    params = caq.ReorderParams.calibrated(wave=wave, n_slices=n_xcd, iters=5)
    gs = GsrsSearch(H, L, d, b, dev, reorder=params, p1=0.9, p2=0.8)
    banner(f"full-size gsrs75k search step: H={H} MB={mb}")
    gs.step(w.q, w.k, w.v, w.x0)
    torch.cuda.synchronize()
    m1, m2 = gs.mask1.cpu().numpy(), gs.mask2.cpu().numpy()
    assert not (m2 > m1).any(), "S2 must lie inside S1"
    rp_d, rp_1 = gs.dense.row_ptr.cpu().numpy(), gs.s1.row_ptr.cpu().numpy()
    rng = np.random.default_rng(13)
    for h in sorted(set([0, H - 1, int(rng.integers(H))])):
        qh, kh, vh = (np64(t[h:h + 1]) for t in (w.q, w.k, w.v))
        for u in sorted(set([mb - 1, int(rng.integers(mb)), int(rng.integers(mb))])):
            r = h * mb + u
            # S1: Top-p of the dense pass's W, every block a candidate
            w_d = gs.dense.w[rp_d[r]:rp_d[r + 1]].cpu().numpy()
            rp, ci = _row_csr(np.arange(mb), mb)
            np.testing.assert_array_equal(m1[h, u], oracle.topp_select(w_d, rp, ci, 1, 1, mb,
                                                                       0.9)[0, 0])
            # the pass over S1: W over the S1 candidates
            cols1 = np.flatnonzero(m1[h, u])
            w_1 = gs.s1.w[rp_1[r]:rp_1[r + 1]].cpu().numpy()
            assert w_1.size == cols1.size
            rp, ci = _row_csr(cols1, mb)
            sub = np.zeros((1, mb, mb), dtype=np.uint8)
            sub[0, u, cols1] = 1
            srp, sci, _, _, _ = oracle.block_index(sub)
            g_ref, lse_ref = oracle.block_lse(qh, kh, srp, sci, L, b, w.scale)
            w_ref = oracle.block_importance(g_ref, lse_ref, srp, L, b)
            np.testing.assert_allclose(w_1.astype(np.float64), w_ref, atol=2e-4, rtol=1e-3,
                                       err_msg=f"W over S1 h={h} u={u}")
            # S2: Top-p at 0.8 of the GPU's W over S1
            np.testing.assert_array_equal(m2[h, u], oracle.topp_select(w_1, rp, ci, 1, 1, mb,
                                                                       0.8)[0, 0])
            # the pass over S2
            r0, r1 = u * b, min((u + 1) * b, L)
            rows = np.unique(np.concatenate([[r0, r1 - 1], rng.integers(r0, r1, size=6)]))
            o_ref, l_ref = oracle.masked_attention_rows(qh[0], kh[0], vh[0], m2[h], rows, L, b,
                                                        w.scale)
            assert_attention_close(np64(gs.s2.o[h])[rows],
                                   gs.s2.lse[h].cpu().numpy().astype(np.float64)[rows],
                                   o_ref, l_ref, f"S2 pass h={h} u={u}")
            banner(f"gsrs75k search h={h} u={u}: S1 {cols1.size}, S2 {int(m2[h, u].sum())} of {mb}")


def test_more_blocks_than_the_staged_list_cap():
    """2,100 query blocks (block 64): the attention kernel reads its lists from global
    memory, the reorder gathers through the transposed lists and sorts 4,096 keys."""
    dev = gpu()
    L, b, d, mb = 2100 * 64, 64, 64, 2100
    banner(f"large MB: L={L} b={b} d={d} MB={mb}")
    w = synth.random_tiny_case(71, heads=1, seq_len=L, head_dim=d, block=b, density=0.002,
                               empty_rows=(5,))
    assert mb == w.mask.shape[1] and caq.reorder_needs_csc(mb, mb)
    q, k, v, mask, x0 = (t.to(dev) for t in (w.q, w.k, w.v, w.mask, w.x0))
    idx = caq.build_block_index(mask)
    params = caq.ReorderParams(wave=64, n_slices=8, iters=5, skip_mode=caq.WA_SKIP_NEVER)
    ro = caq.reorder_rows(idx, x0, b, d, params)
    o, lse, _ = caq.sparse_attn_fwd(q, k, v, L, b, idx.row_ptr, idx.col_idx, perm=ro.perm,
                                    perm_slices=ro.n_slices)
    o_id, lse_id, _ = caq.sparse_attn_fwd(q, k, v, L, b, idx.row_ptr, idx.col_idx)
    torch.cuda.synchronize()
    perm = ro.perm.cpu().numpy()[0]
    assert sorted(perm.tolist()) == list(range(mb))
    assert torch.equal(o, o_id) and torch.equal(lse, lse_id)
    # sampled rows against the oracle (the empty block 5 included)
    qn, kn, vn = np64(w.q)[0], np64(w.k)[0], np64(w.v)[0]
    m = w.mask.cpu().numpy()[0]
    rng = np.random.default_rng(3)
    for u in sorted(set([0, 5, mb - 1] + rng.choice(mb, size=6, replace=False).tolist())):
        rows = np.arange(u * b, min((u + 1) * b, L))[::9]
        o_ref, l_ref = oracle.masked_attention_rows(qn, kn, vn, m, rows, L, b, w.scale)
        assert_attention_close(np64(o[0, rows]), lse[0, rows].cpu().numpy().astype(np.float64),
                               o_ref, l_ref, f"row block {u}")


def test_the_largest_supported_mask():
    """WA_MAX_BLOCKS = 4,096 query and key blocks (block 64, ragged last block): the
    reorder's statistics, angles and permutation against the oracle, the attention's
    global-list path on sampled rows, and the MinHash order bit for bit."""
    dev = gpu()
    mb, b, d = 4096, 64, 64
    L = mb * b - 17
    banner(f"largest mask: L={L} b={b} d={d} MB={mb}")
    w = synth.random_tiny_case(83, heads=1, seq_len=L, head_dim=d, block=b, density=0.001,
                               empty_rows=(7,))
    assert w.mask.shape[1] == mb and caq.reorder_needs_csc(mb, mb)
    q, k, v, mask, x0 = (t.to(dev) for t in (w.q, w.k, w.v, w.mask, w.x0))
    idx = caq.build_block_index(mask)
    params = caq.ReorderParams(wave=64, n_slices=8, iters=5, skip_mode=caq.WA_SKIP_NEVER)
    ro = caq.reorder_rows(idx, x0, b, d, params)
    o, lse, _ = caq.sparse_attn_fwd(q, k, v, L, b, idx.row_ptr, idx.col_idx, perm=ro.perm,
                                    perm_slices=ro.n_slices)
    a_mh, b_mh = synth.minhash_params(2)
    perm_mh, _ = caq.minhash_order(idx, a_mh, b_mh, 64, 8)
    torch.cuda.synchronize()
    m_all = w.mask.cpu().numpy()
    op = oracle.ReorderParams(wave=64, n_slices=8, iters=5, skip_mode=oracle.reorder.SKIP_NEVER)
    perm_o, _, _, ang_o, st_o = oracle.reorder_rows(m_all, w.x0.cpu().numpy().astype(np.float64),
                                                    b, d, op)
    np.testing.assert_array_equal(ro.stats.cpu().numpy(), st_o)
    ang_g = ro.angles.cpu().numpy()[0]
    both = np.isfinite(ang_o[0])
    np.testing.assert_allclose(ang_g[both], ang_o[0][both], atol=1e-9, rtol=0)
    assert sorted(ro.perm.cpu().numpy()[0].tolist()) == list(range(mb))
    np.testing.assert_array_equal(perm_mh.cpu().numpy(),
                                  oracle.minhash_order(m_all, a_mh, b_mh, 64, 8)[0])
    qn, kn, vn = np64(w.q)[0], np64(w.k)[0], np64(w.v)[0]
    m = m_all[0]
    for u in (0, 7, 2048, mb - 1):
        rows = np.arange(u * b, min((u + 1) * b, L))[::5]
        o_ref, l_ref = oracle.masked_attention_rows(qn, kn, vn, m, rows, L, b, w.scale)
        assert_attention_close(np64(o[0, rows]), lse[0, rows].cpu().numpy().astype(np.float64),
                               o_ref, l_ref, f"row block {u}")


def test_long_sequence_sampled():
    # The 363,600-token shape (2,841 blocks per side) on 4 of its 40 heads: the reorder
    # takes the transposed-list form, the attention reads its lists from global memory
    # (more than 2,048 blocks), and Top-p sorts rows of hundreds of keys in registers.
    dev = gpu()
    banner("long sequence: generating wan364k, 4 heads")
    w = synth.make_workload("wan364k", device=dev, heads=4)
    H, mb = w.mask.shape[0], w.mask.shape[1]
    nnz = int(w.mask.sum())
    _, _, wave = caq.schedule_info(0, w.head_dim)
    params = caq.ReorderParams(wave=wave, n_slices=8, skip_mode=caq.WA_SKIP_NEVER)
    hp = HotPath(H, w.seq_len, w.head_dim, w.block, dev, capacity=nnz, reorder=params, gsrs_p=0.9)
    assert hp.with_csc
    banner(f"long sequence: H={H} MB={mb} nnz={nnz}")
    hp.step(w.q, w.k, w.v, w.mask, w.x0)
    torch.cuda.synchronize()
    perm = hp.perm.cpu().numpy()
    for h in range(H):
        assert sorted(perm[h].tolist()) == list(range(mb))
    assert not torch.isnan(hp.o[:, : w.seq_len]).any()
    rp = hp.row_ptr.cpu().numpy()
    ci = hp.col_idx.cpu().numpy()
    wts = hp.w.cpu().numpy()
    sel = hp.next_mask.cpu().numpy()
    mask = w.mask.cpu().numpy()
    rng = np.random.default_rng(11)
    samples = _sample_rows(w, rng, n_heads=2, n_blocks=3)
    cached = {}
    for h, u, rows in samples:
        if h not in cached:
            cached.clear()
            cached[h] = tuple(np64(t[h]) for t in (w.q, w.k, w.v))
        qh, kh, vh = cached[h]
        o_ref, l_ref = oracle.masked_attention_rows(qh, kh, vh, mask[h], rows, w.seq_len,
                                                    w.block, w.scale)
        assert_attention_close(np64(hp.o[h])[rows],
                               hp.lse[h].cpu().numpy().astype(np.float64)[rows], o_ref, l_ref,
                               f"wan364k h={h} u={u}")
        # Top-p of this row from the same W, bit for bit
        lo, hi = int(rp[h * mb + u]), int(rp[h * mb + u + 1])
        assert abs(float(wts[lo:hi].astype(np.float64).sum()) - 1.0) < 1e-4
        ref = oracle.topp_select(wts[lo:hi], np.array([0, hi - lo]), ci[lo:hi], 1, 1, mb, 0.9)
        np.testing.assert_array_equal(sel[h, u], ref[0, 0], err_msg=f"top-p h={h} u={u}")
    lengths = np.diff(rp)
    print(f"wan364k: longest row {lengths.max()} blocks, mean {lengths.mean():.1f}")
