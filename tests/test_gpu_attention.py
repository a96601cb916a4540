"""wa_sparse_attn_fwd against the fp64 oracle (element by element), plus the
invariants the pages fix: the output does not depend on the execution order of
query blocks, an all-ones mask is dense attention, a fully masked query block
gives O = 0 and LSE = -inf."""

import numpy as np
import pytest
import torch

import cache_aware_query_amd as caq
import oracle
import synth
from helpers import assert_attention_close, banner, gpu, np64

pytestmark = pytest.mark.gpu


def _run(w, perm=None, schedule=caq.WA_SCHED_XCD_SLICED, with_g=False):
    dev = gpu()
    q, k, v, mask = (t.to(dev) for t in (w.q, w.k, w.v, w.mask))
    idx = caq.build_block_index(mask)
    p = None if perm is None else perm.to(dev)
    # a free permutation: the slice count of the schedule it runs under is the device's
    n_xcd = caq.schedule_info(0, w.head_dim)[0]
    o, lse, g = caq.sparse_attn_fwd(q, k, v, w.seq_len, w.block, idx.row_ptr, idx.col_idx,
                                    perm=p, schedule=schedule, with_g=with_g,
                                    perm_slices=None if p is None else n_xcd)
    torch.cuda.synchronize()
    return o, lse, g, idx


def _oracle(w):
    return oracle.masked_attention(np64(w.q), np64(w.k), np64(w.v), w.mask.cpu().numpy(),
                                   w.seq_len, w.block, w.scale)


def _compare(w, o, lse, what):
    o_ref, lse_ref = _oracle(w)
    L = w.seq_len
    assert_attention_close(np64(o)[:, :L], lse.cpu().numpy().astype(np.float64)[:, :L],
                           o_ref[:, :L], lse_ref[:, :L], what)


CASES = [
    ("tiny", {}),
    ("layer16k", {"heads": 3}),
]


@pytest.mark.parametrize("name,over", CASES)
@pytest.mark.parametrize("schedule", [caq.WA_SCHED_NATURAL, caq.WA_SCHED_XCD_SLICED])
def test_attention_matches_oracle_on_workloads(name, over, schedule):
    w = synth.make_workload(name, **over)
    banner(f"attention {name} {over} schedule={schedule}")
    o, lse, _, _ = _run(w, schedule=schedule)
    _compare(w, o, lse, f"{name} schedule={schedule}")


@pytest.mark.parametrize("seq_len,head_dim,block,density", [
    (1000, 128, 128, 0.5),    # ragged tail: 8 blocks, the last with 104 tokens
    (1100, 64, 128, 0.4),     # d = 64
    (700, 128, 64, 0.35),     # block 64, d 128, ragged
    (257, 64, 64, 0.7),       # one valid token in the last block
    (128, 128, 128, 1.0),     # a single block
])
def test_attention_ragged_and_shapes(seq_len, head_dim, block, density):
    w = synth.random_tiny_case(seq_len + head_dim, heads=2, seq_len=seq_len, head_dim=head_dim,
                               block=block, density=density, empty_rows=(1,))
    banner(f"attention random L={seq_len} d={head_dim} b={block} rho={density}")
    o, lse, _, _ = _run(w)
    _compare(w, o, lse, f"L={seq_len} d={head_dim} b={block}")


def test_all_ones_mask_is_dense_attention():
    dev = gpu()
    w = synth.random_tiny_case(7, heads=2, seq_len=640, head_dim=128, block=128, density=1.0)
    banner("attention all-ones mask vs dense")
    o, lse, _, _ = _run(w)
    q, k, v = (np64(t)[:, :640] for t in (w.q, w.k, w.v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
    np.testing.assert_allclose(np64(o)[:, :640], ref, atol=2e-2, rtol=2e-2)
    assert dev.type == "cuda"


def test_output_is_independent_of_execution_order():
    w = synth.random_tiny_case(11, heads=3, seq_len=2000, head_dim=128, block=128, density=0.4,
                               empty_rows=(4,))
    mb = w.mask.shape[1]
    banner("attention permutation invariance")
    o0, l0, g0, _ = _run(w, schedule=caq.WA_SCHED_NATURAL, with_g=True)
    gen = torch.Generator().manual_seed(5)
    perm = torch.stack([torch.randperm(mb, generator=gen) for _ in range(3)]).to(torch.int32)
    for sched in (caq.WA_SCHED_NATURAL, caq.WA_SCHED_XCD_SLICED, caq.WA_SCHED_HEADS_INTERLEAVED,
                  caq.WA_SCHED_DEFAULT):
        o1, l1, g1, _ = _run(w, perm=perm, schedule=sched, with_g=True)
        assert torch.equal(o0, o1) and torch.equal(l0, l1) and torch.equal(g0, g1)
    # repeated runs are bitwise identical
    o2, l2, g2, _ = _run(w, schedule=caq.WA_SCHED_NATURAL, with_g=True)
    assert torch.equal(o0, o2) and torch.equal(l0, l2) and torch.equal(g0, g2)
    # without G the exponentials use the running max instead of the block max:
    # the same result up to rounding, and itself order independent
    o3, l3, _, _ = _run(w, schedule=caq.WA_SCHED_NATURAL)
    o4, l4, _, _ = _run(w, perm=perm, schedule=caq.WA_SCHED_XCD_SLICED)
    assert torch.equal(o3, o4) and torch.equal(l3, l4)
    torch.testing.assert_close(o3.float(), o0.float(), atol=2e-2, rtol=2e-2)
    torch.testing.assert_close(l3, l0, atol=1e-4, rtol=0)


def test_fully_masked_block_gives_zero_and_neg_inf():
    w = synth.make_workload("tiny")
    banner("attention fully masked block")
    o, lse, _, _ = _run(w)
    b = w.block
    assert torch.all(o[0, 7 * b:8 * b] == 0)
    assert torch.all(torch.isneginf(lse[0, 7 * b:8 * b]))
    assert torch.all(torch.isfinite(lse[0, :7 * b]))


def _diag(w, with_g=False):
    dev = gpu()
    q, k, v, mask = (t.to(dev) for t in (w.q, w.k, w.v, w.mask))
    idx = caq.build_block_index(mask)
    ent = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=dev)
    dist = torch.empty_like(ent)
    o, lse, _ = caq.sparse_attn_fwd(q, k, v, w.seq_len, w.block, idx.row_ptr, idx.col_idx,
                                    with_g=with_g, entropy_out=ent, distance_out=dist)
    o2, lse2, _ = caq.sparse_attn_fwd(q, k, v, w.seq_len, w.block, idx.row_ptr, idx.col_idx,
                                      with_g=with_g)
    # each output alone equals the same output of the joint call
    ent1 = torch.empty_like(ent)
    dist1 = torch.empty_like(ent)
    caq.sparse_attn_fwd(q, k, v, w.seq_len, w.block, idx.row_ptr, idx.col_idx, with_g=with_g,
                        entropy_out=ent1)
    caq.sparse_attn_fwd(q, k, v, w.seq_len, w.block, idx.row_ptr, idx.col_idx, with_g=with_g,
                        distance_out=dist1)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    L = w.seq_len
    assert torch.equal(ent1[:, :L], ent[:, :L]) and torch.equal(dist1[:, :L], dist[:, :L])
    return (ent.cpu().numpy().astype(np.float64)[:, :L],
            dist.cpu().numpy().astype(np.float64)[:, :L])


@pytest.mark.parametrize("with_g", [False, True])
@pytest.mark.parametrize("shape", [(128, 128), (64, 64)])
def test_diagnostics_match_oracle(shape, with_g):
    """Row entropy (LSE - E[z]) and mean attention distance from the same pass against
    the explicit softmax statistics; O and LSE are unchanged by asking for them."""
    d, b = shape
    w = synth.random_tiny_case(41 + d, heads=2, seq_len=900, head_dim=d, block=b, density=0.4,
                               empty_rows=(2,))
    banner(f"attention diagnostics d={d} b={b} with_g={with_g}")
    ent, dist = _diag(w, with_g)
    L = w.seq_len
    m = w.mask.cpu().numpy()
    ref_e = oracle.attention_entropy(np64(w.q), np64(w.k), m, L, w.block, w.scale)[:, :L]
    ref_d = oracle.attention_distance(np64(w.q), np64(w.k), m, L, w.block, w.scale)[:, :L]
    assert np.all(np.isfinite(ent)) and np.all(np.isfinite(dist))
    np.testing.assert_allclose(ent, ref_e, rtol=0, atol=2e-2)
    # P is rounded to bf16 (relative error <= 2^-9 per weight) and normalised by the sum
    # of the rounded weights, so |D~ - D| <= 2^-9 * max_j |j - i| / (1 - 2^-9) < 2^-8 * L.
    # Independent roundings average out, so the mean error is far smaller; a key index
    # off by one would move every row by about one token.
    err = np.abs(dist - ref_d)
    assert err.max() < 2.0 ** -8 * L, err.max()
    assert err.mean() < 2.0 ** -4, err.mean()
    assert np.all(ent[:, 2 * b:3 * b] == 0.0) and np.all(dist[:, 2 * b:3 * b] == 0.0)


@pytest.mark.parametrize("shape", [(128, 128), (64, 64)])
def test_distance_with_uniform_attention(shape):
    """Zero queries: every allowed key has weight exactly 1 in bf16, so the mean attention
    distance is the plain mean of |i - j| over the allowed keys (fp32 sums only) and the
    entropy is ln(#keys)."""
    d, b = shape
    w = synth.random_tiny_case(57 + d, heads=2, seq_len=1000, head_dim=d, block=b, density=0.5,
                               empty_rows=(1,))
    w.q.zero_()
    banner(f"attention distance, uniform weights d={d} b={b}")
    ent, dist = _diag(w)
    L = w.seq_len
    m = w.mask.cpu().numpy()
    for h in range(m.shape[0]):
        for i in range(L):
            keys = np.concatenate([np.arange(vb * b, min((vb + 1) * b, L))
                                   for vb in np.nonzero(m[h, i // b])[0]] or [np.zeros(0, int)])
            if keys.size == 0:
                assert dist[h, i] == 0.0 and ent[h, i] == 0.0
                continue
            assert abs(dist[h, i] - np.abs(keys - i).mean()) < 1e-2
            assert abs(ent[h, i] - np.log(keys.size)) < 1e-3


@pytest.mark.parametrize("skip_mode,expect", [(caq.WA_SKIP_ALWAYS, caq.WA_SCHED_DEFAULT),
                                              (caq.WA_SKIP_NEVER, caq.WA_SCHED_XCD_SLICED)])
def test_auto_schedule_follows_the_skip_flags(skip_mode, expect):
    """WA_SCHED_AUTO runs the default path when every head kept its order and the
    XCD-sliced schedule otherwise; the output is the same either way."""
    dev = gpu()
    w = synth.random_tiny_case(23, heads=3, seq_len=1500, head_dim=128, block=128, density=0.4,
                               empty_rows=(2,))
    banner(f"attention AUTO schedule skip_mode={skip_mode}")
    q, k, v, mask, x0 = (t.to(dev) for t in (w.q, w.k, w.v, w.mask, w.x0))
    idx = caq.build_block_index(mask)
    n_xcd = caq.schedule_info(0, w.head_dim)[0]
    ro = caq.reorder_rows(idx, x0, w.block, w.head_dim,
                          caq.ReorderParams(wave=8, n_slices=n_xcd, skip_mode=skip_mode))
    ws = torch.empty(caq.sparse_attn_workspace_size(3, w.seq_len, 128, 128), dtype=torch.uint8,
                     device=dev)
    caq.attn_schedule_select(ro.skipped, ws)
    o, lse, g = caq.sparse_attn_fwd(q, k, v, w.seq_len, w.block, idx.row_ptr, idx.col_idx,
                                    perm=ro.perm, schedule=caq.WA_SCHED_AUTO, with_g=True,
                                    workspace=ws, perm_slices=ro.n_slices)
    o2, lse2, g2 = caq.sparse_attn_fwd(q, k, v, w.seq_len, w.block, idx.row_ptr, idx.col_idx,
                                       perm=ro.perm, schedule=expect, with_g=True,
                                       perm_slices=ro.n_slices)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == expect
    assert torch.equal(o, o2) and torch.equal(lse, lse2) and torch.equal(g, g2)
    _compare(w, o, lse, f"AUTO skip_mode={skip_mode}")


def _csr_from_lists(lists):
    """row_ptr, col_idx (int32) of per-row id lists, in row order."""
    row_ptr = np.zeros(len(lists) + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum([len(x) for x in lists])
    col_idx = np.array([v for x in lists for v in x] or [0], dtype=np.int32)
    return row_ptr, col_idx


@pytest.mark.parametrize("with_g", [False, True])
def test_list_entries_outside_the_key_blocks(with_g):
    """CSR entries outside [0, MB) evaluate no key: a row holding only such ids gets
    O = 0 and LSE = -inf (no NaN), a row mixing them with real ids equals the row
    of the real ids alone, their G is -inf and their block weight 0."""
    dev = gpu()
    w = synth.random_tiny_case(31, heads=1, seq_len=1000, head_dim=128, block=128, density=0.5,
                               empty_rows=())
    mb = w.mask.shape[1]
    banner(f"attention with list entries outside [0, {mb}) with_g={with_g}")
    m = w.mask.cpu().numpy()[0].astype(bool)
    bad = [-1, mb, mb + 5, -(2 ** 31)]
    lists = []
    for u in range(mb):
        real = np.flatnonzero(m[u]).tolist()
        if u == 2:
            lists.append(bad[:3])                   # only ids that name no block
        elif u == 5:
            lists.append([bad[0]] + real + [bad[1], bad[3]])  # mixed
        else:
            lists.append(real)
    rp, ci = _csr_from_lists(lists)
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    row_ptr, col_idx = torch.from_numpy(rp).to(dev), torch.from_numpy(ci).to(dev)
    o, lse, g = caq.sparse_attn_fwd(q, k, v, w.seq_len, w.block, row_ptr, col_idx,
                                    schedule=caq.WA_SCHED_NATURAL, with_g=with_g)
    torch.cuda.synchronize()
    m_ref = m.copy()
    m_ref[2] = False
    L, b = w.seq_len, w.block
    o_ref, lse_ref = oracle.masked_attention(np64(w.q), np64(w.k), np64(w.v), m_ref[None], L, b,
                                             w.scale)
    assert_attention_close(np64(o)[:, :L], lse.cpu().numpy().astype(np.float64)[:, :L],
                           o_ref[:, :L], lse_ref[:, :L], "entries outside [0, MB)")
    assert torch.all(o[0, 2 * b:3 * b] == 0)
    if with_g:
        gn = g.cpu().numpy()
        ids = ci[: rp[-1]]
        outside = (ids < 0) | (ids >= mb)
        assert np.all(np.isneginf(gn[outside]))
        wts = caq.block_importance(g, lse, row_ptr, L, b).cpu().numpy()
        assert np.all(wts[outside] == 0)
        # each row with real keys still sums to 1 over its real entries
        for u in range(mb):
            if u != 2:
                assert abs(wts[rp[u]:rp[u + 1]].sum() - 1.0) < 1e-3


def test_row_longer_than_the_staged_list():
    """A (malformed) row listing one block 2,100 times: past the 2,048 entries staged
    in LDS the kernel reads the list from global memory.  Every key of the block then
    counts 2,100 times: O equals the single-block row and LSE rises by ln 2,100."""
    dev = gpu()
    w = synth.random_tiny_case(37, heads=1, seq_len=16 * 128, head_dim=128, block=128,
                               density=0.3, empty_rows=())
    mb = w.mask.shape[1]
    banner("attention row of 2,100 entries (staged list cap 2,048)")
    reps, u_long, v_long = 2100, 6, 3
    m = w.mask.cpu().numpy()[0].astype(bool)
    lists = [np.flatnonzero(m[u]).tolist() for u in range(mb)]
    lists[u_long] = [v_long] * reps
    rp, ci = _csr_from_lists(lists)
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    row_ptr, col_idx = torch.from_numpy(rp).to(dev), torch.from_numpy(ci).to(dev)
    o, lse, _ = caq.sparse_attn_fwd(q, k, v, w.seq_len, w.block, row_ptr, col_idx,
                                    schedule=caq.WA_SCHED_NATURAL)
    torch.cuda.synchronize()
    m_ref = m.copy()
    m_ref[u_long] = False
    m_ref[u_long, v_long] = True
    L, b = w.seq_len, w.block
    o_ref, lse_ref = oracle.masked_attention(np64(w.q), np64(w.k), np64(w.v), m_ref[None], L, b,
                                             w.scale)
    lse_ref = lse_ref.copy()
    lse_ref[0, u_long * b:(u_long + 1) * b] += np.log(reps)
    assert_attention_close(np64(o)[:, :L], lse.cpu().numpy().astype(np.float64)[:, :L],
                           o_ref[:, :L], lse_ref[:, :L], "row of 2,100 entries")


def test_host_skipped_path_runs_the_default_path():
    """A HotPath whose shape cannot pass the adaptive skip's work rule launches no
    reorder and runs the default path: bitwise the plain call."""
    from cache_aware_query_amd.pipeline import HotPath

    dev = gpu()
    w = synth.make_workload("layer16k", device="cuda", heads=4)
    H, mb = w.mask.shape[0], w.mask.shape[1]
    nnz = int(w.mask.sum())
    banner("host-skipped HotPath layer16k heads=4")
    params = caq.ReorderParams(wave=64, n_slices=caq.schedule_info(0, 128)[0],
                               skip_mode=caq.WA_SKIP_ADAPTIVE, flops_min=2.2e11)
    hp = HotPath(H, w.seq_len, w.head_dim, w.block, dev, capacity=nnz, reorder=params,
                 schedule=caq.WA_SCHED_AUTO, gsrs_p=None)
    assert hp.host_skip
    hp.build_index(w.mask)
    hp.reorder_rows(w.x0)
    hp.attention(w.q, w.k, w.v)
    o, lse, _ = caq.sparse_attn_fwd(w.q, w.k, w.v, w.seq_len, w.block, hp.row_ptr, hp.col_idx,
                                    schedule=caq.WA_SCHED_DEFAULT)
    torch.cuda.synchronize()
    assert torch.equal(hp.o, o) and torch.equal(hp.lse, lse)
