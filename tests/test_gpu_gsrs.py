"""GSRS stage on the GPU against the oracle: Phase-1 G, Phase-2 W, Top-p.

G and W are compared with tolerances (fp32 against fp64); the Top-p kept sets
are compared bit for bit for the same W, which both sides get from the seeded
generator."""

import math

import numpy as np
import pytest
import torch

import cache_aware_query_amd as caq
import oracle
import synth
from cache_aware_query_amd.pipeline import GsrsSchedule
from helpers import banner, gpu, np64

pytestmark = pytest.mark.gpu


def _g_and_w(w):
    dev = gpu()
    q, k, v, mask = (t.to(dev) for t in (w.q, w.k, w.v, w.mask))
    idx = caq.build_block_index(mask)
    o, lse, g = caq.sparse_attn_fwd(q, k, v, w.seq_len, w.block, idx.row_ptr, idx.col_idx,
                                    with_g=True)
    wts = caq.block_importance(g, lse, idx.row_ptr, w.seq_len, w.block)
    torch.cuda.synchronize()
    return idx, lse, g, wts


@pytest.mark.parametrize("case", ["tiny", "ragged128", "ragged64"])
def test_block_lse_and_importance_match_oracle(case):
    if case == "tiny":
        w = synth.make_workload("tiny")
    elif case == "ragged128":
        w = synth.random_tiny_case(21, heads=2, seq_len=1000, head_dim=128, block=128,
                                   density=0.5, empty_rows=(2,))
    else:
        w = synth.random_tiny_case(22, heads=2, seq_len=700, head_dim=64, block=64, density=0.4,
                                   empty_rows=(0,))
    banner(f"gsrs G/W {case}")
    idx, lse, g, wts = _g_and_w(w)
    rp, ci, _, _, _ = oracle.block_index(w.mask.numpy())
    nnz = int(rp[-1])
    g_ref, lse_ref = oracle.block_lse(np64(w.q), np64(w.k), rp, ci, w.seq_len, w.block, w.scale)
    w_ref = oracle.block_importance(g_ref, lse_ref, rp, w.seq_len, w.block)
    g_gpu = g.cpu().numpy()[:nnz].astype(np.float64)
    w_gpu = wts.cpu().numpy()[:nnz].astype(np.float64)
    H, mb = w.mask.shape[0], w.mask.shape[1]
    L, b = w.seq_len, w.block
    for r in range(H * mb):
        u = r % mb
        nrows = min(b, L - u * b)
        lo, hi = rp[r], rp[r + 1]
        if hi == lo:
            continue
        gg, gr = g_gpu[lo:hi, :nrows], g_ref[lo:hi, :nrows]
        assert not np.isnan(gg).any()
        np.testing.assert_allclose(gg, gr, atol=5e-3, rtol=0)
        np.testing.assert_allclose(w_gpu[lo:hi], w_ref[lo:hi], atol=2e-4, rtol=1e-3)
        assert abs(w_gpu[lo:hi].sum() - 1.0) < 1e-4


def _random_weights(rng, row_ptr):
    """Per-row fp32 weights with ties, one-hot rows, uniform rows and zero rows."""
    nnz = int(row_ptr[-1])
    w = np.zeros(nnz, dtype=np.float32)
    for r in range(len(row_ptr) - 1):
        lo, hi = row_ptr[r], row_ptr[r + 1]
        n = hi - lo
        if n == 0:
            continue
        kind = r % 5
        if kind == 0:
            x = rng.random(n)
        elif kind == 1:
            x = rng.integers(1, 4, size=n).astype(float)       # many ties
        elif kind == 2:
            x = np.zeros(n)
            x[rng.integers(0, n)] = 1.0                        # one-hot
        elif kind == 3:
            x = np.ones(n)                                     # uniform
        else:
            x = rng.random(n) ** 8                             # peaked
        w[lo:hi] = (x / x.sum()).astype(np.float32)
    return w


@pytest.mark.parametrize("p", [0.5, 0.8, 0.9, 0.95, 1.0])
def test_topp_is_bit_exact_for_a_given_w(p):
    dev = gpu()
    rng = np.random.default_rng(31)
    H, mb, nb = 3, 120, 150
    mask = (rng.random((H, mb, nb)) < 0.5).astype(np.uint8)
    mask[:, 5] = 0
    mask[:, 7] = 1          # full rows (150 candidates)
    mask[0, 9] = 0
    mask[0, 9, :100] = 1    # 100 uniform weights (the fp64 accumulation trap)
    rp, ci, _, _, _ = oracle.block_index(mask)
    w = _random_weights(rng, rp)
    w[rp[9]:rp[10]] = np.float32(0.01)
    banner(f"topp p={p}")
    sel = caq.topp_select(torch.from_numpy(w).to(dev), torch.from_numpy(rp.astype(np.int32)).to(dev),
                          torch.from_numpy(ci.astype(np.int32)).to(dev), H, mb, nb, p)
    torch.cuda.synchronize()
    ref = oracle.topp_select(w, rp, ci, H, mb, nb, p)
    np.testing.assert_array_equal(sel.cpu().numpy(), ref)
    if p == 0.9:
        assert int(ref[0, 9].sum()) == 91


@pytest.mark.parametrize("p", [0.5, 0.9, 1.0])
def test_topp_rows_of_every_length_class(p):
    # Rows of 0..1,500 candidates: each side of every register-sort size (64, 128, 256,
    # 512 and 1,024 keys) and rows longer than 1,024, which take the LDS sort.
    dev = gpu()
    rng = np.random.default_rng(37)
    lengths = [0, 1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 512, 513, 700, 1023,
               1024, 1025, 1200, 1500]
    H, nb = 2, 1500
    mb = len(lengths)
    mask = np.zeros((H, mb, nb), dtype=np.uint8)
    for h in range(H):
        for u, n in enumerate(lengths):
            mask[h, u, rng.choice(nb, size=n, replace=False)] = 1
    rp, ci, _, _, _ = oracle.block_index(mask)
    w = _random_weights(rng, rp)
    banner(f"topp length classes p={p}")
    sel = caq.topp_select(torch.from_numpy(w).to(dev), torch.from_numpy(rp.astype(np.int32)).to(dev),
                          torch.from_numpy(ci.astype(np.int32)).to(dev), H, mb, nb, p)
    torch.cuda.synchronize()
    ref = oracle.topp_select(w, rp, ci, H, mb, nb, p)
    np.testing.assert_array_equal(sel.cpu().numpy(), ref)


def test_gsrs_search_pipeline_growing_sparsity():
    """Dense pass -> W -> Top-p(0.9) = S1; pass over S1 -> W over S1 -> Top-p(0.8) = S2."""
    dev = gpu()
    w = synth.make_workload("gsrs75k", device="cuda", heads=2, grid=(3, 45, 80))
    H, mb = w.mask.shape[0], w.mask.shape[1]
    banner(f"gsrs pipeline H={H} MB={mb}")
    idx, lse, g, wts = _g_and_w(w)
    s1 = caq.topp_select(wts, idx.row_ptr, idx.col_idx, H, mb, mb, 0.9)
    idx1 = caq.build_block_index(s1)
    o1, lse1, g1 = caq.sparse_attn_fwd(w.q.to(dev), w.k.to(dev), w.v.to(dev), w.seq_len, w.block,
                                       idx1.row_ptr, idx1.col_idx, with_g=True)
    w1 = caq.block_importance(g1, lse1, idx1.row_ptr, w.seq_len, w.block)
    s2 = caq.topp_select(w1, idx1.row_ptr, idx1.col_idx, H, mb, mb, 0.8)
    torch.cuda.synchronize()
    s1n, s2n = s1.cpu().numpy(), s2.cpu().numpy()
    assert np.all(s2n <= s1n)
    assert 0 < s2n.sum() < s1n.sum() < H * mb * mb
    # every non-empty row of W over S1 sums to one
    rp1 = idx1.row_ptr.cpu().numpy()
    wn = w1.cpu().numpy().astype(np.float64)
    sums = np.add.reduceat(wn[: rp1[-1]], rp1[:-1][np.diff(rp1) > 0])
    np.testing.assert_allclose(sums, 1.0, atol=1e-4)
    # the oracle's S1 from its own W agrees except at cumulative-sum near-ties
    q, k = np64(w.q), np64(w.k)
    rp, ci, _, _, _ = oracle.block_index(w.mask.cpu().numpy())
    g_ref, lse_ref = oracle.block_lse(q, k, rp, ci, w.seq_len, w.block, w.scale)
    w_ref = oracle.block_importance(g_ref, lse_ref, rp, w.seq_len, w.block).astype(np.float32)
    s1_ref = oracle.topp_select(w_ref, rp, ci, H, mb, mb, 0.9)
    diff = np.sum(s1_ref != s1n)
    assert diff <= max(2, 0.002 * s1_ref.sum()), diff
    # Step 5 (the pass restricted to S1, GSRS reduced search): the index of S1 is the
    # oracle's, G1 and W1 over S1 match the oracle's block LSE and block importance
    # over the same candidate set, and S2 is exactly the oracle's Top-p(0.8) of the
    # GPU's W1.
    rp1, ci1, _, _, _ = oracle.block_index(s1n)
    nnz1 = int(rp1[-1])
    np.testing.assert_array_equal(idx1.row_ptr.cpu().numpy(), rp1)
    np.testing.assert_array_equal(idx1.col_idx.cpu().numpy()[:nnz1], ci1)
    g1_ref, lse1_ref = oracle.block_lse(q, k, rp1, ci1, w.seq_len, w.block, w.scale)
    w1_ref = oracle.block_importance(g1_ref, lse1_ref, rp1, w.seq_len, w.block)
    g1n = g1.cpu().numpy()[:nnz1].astype(np.float64)
    L, b = w.seq_len, w.block
    for r in range(H * mb):
        u = r % mb
        nrows = min(b, L - u * b)
        lo, hi = rp1[r], rp1[r + 1]
        if hi > lo:
            np.testing.assert_allclose(g1n[lo:hi, :nrows], g1_ref[lo:hi, :nrows], atol=5e-3,
                                       rtol=0)
    fin = np.isfinite(lse1_ref[:, :L])
    np.testing.assert_allclose(lse1.cpu().numpy()[:, :L][fin], lse1_ref[:, :L][fin], atol=5e-3,
                               rtol=0)
    np.testing.assert_allclose(wn[:nnz1], w1_ref, atol=2e-4, rtol=1e-3)
    s2_ref = oracle.topp_select(w1.cpu().numpy()[:nnz1], rp1, ci1, H, mb, mb, 0.8)
    np.testing.assert_array_equal(s2n, s2_ref)


def test_gsrs_search_class_matches_the_explicit_chain():
    """The benchmark's GsrsSearch (buffers allocated once, reordered sparse passes)
    selects the same S1 and S2 as the explicit chain of library calls."""
    from cache_aware_query_amd.pipeline import GsrsSearch

    dev = gpu()
    w = synth.make_workload("gsrs75k", device="cuda", heads=2, grid=(3, 45, 80))
    H, mb = w.mask.shape[0], w.mask.shape[1]
    banner(f"gsrs search class H={H} MB={mb}")
    params = caq.ReorderParams(wave=64, n_slices=8, iters=5, skip_mode=caq.WA_SKIP_NEVER)
    gs = GsrsSearch(H, w.seq_len, w.head_dim, w.block, dev, reorder=params)
    gs.step(w.q, w.k, w.v, w.x0)
    _, _, _, wts = _g_and_w(w)
    idx = caq.build_block_index(w.mask.to(dev))
    s1 = caq.topp_select(wts, idx.row_ptr, idx.col_idx, H, mb, mb, 0.9)
    idx1 = caq.build_block_index(s1)
    _, lse1, g1 = caq.sparse_attn_fwd(w.q, w.k, w.v, w.seq_len, w.block, idx1.row_ptr,
                                      idx1.col_idx, with_g=True)
    w1 = caq.block_importance(g1, lse1, idx1.row_ptr, w.seq_len, w.block)
    s2 = caq.topp_select(w1, idx1.row_ptr, idx1.col_idx, H, mb, mb, 0.8)
    torch.cuda.synchronize()
    assert torch.equal(gs.mask1, s1)
    # Reordering changes which workgroup runs a query block, not its arithmetic, so
    # S1's reordered pass gives the same G and LSE and the same second selection.
    assert torch.equal(gs.mask2, s2)
    assert int((gs.mask2.to(torch.int16) > gs.mask1.to(torch.int16)).sum()) == 0
    n = gs.selected_pairs()
    assert n[0] == H * mb * mb and n[1] == int(s1.sum()) and n[2] == int(gs.mask2.sum())


def test_gsrs_schedule_reduced_search_and_mask_reuse():
    """Warmup, a full first search, reduced searches inside S1, mask reuse between."""
    from cache_aware_query_amd.pipeline import GsrsSchedule

    dev = gpu()
    w = synth.make_workload("gsrs75k", device="cuda", heads=2, grid=(3, 45, 80))
    H, mb = w.mask.shape[0], w.mask.shape[1]
    banner(f"gsrs schedule H={H} MB={mb}")
    search = (2, 4, 6)
    states = synth.drift_states(w, len(search) + 1)
    params = caq.ReorderParams(wave=64, n_slices=8, iters=5, skip_mode=caq.WA_SKIP_NEVER)
    gs = GsrsSchedule(H, w.seq_len, w.head_dim, w.block, dev, reorder=params, steps=8,
                      search_steps=search, thresholds=(0.95, 0.9, 0.8))

    def inputs(t):
        q, k, v = states[sum(1 for s in search if t >= s)]
        return q, k, v, w.x0

    masks = {}

    def on_step(t, kind):
        if kind == "search":
            masks[t] = gs.mask.clone()

    gs.run(inputs, on_step)
    torch.cuda.synchronize()
    assert gs.kinds == ["warmup", "warmup", "search", "reuse", "search", "reuse", "search",
                        "reuse"]
    s1 = gs.s1.to(torch.int16)
    assert 0 < int(s1.sum()) < H * mb * mb
    for t, m in masks.items():
        assert int((m.to(torch.int16) > s1).sum()) == 0, t   # every mask lies inside S1
        assert int(m.sum()) > 0
    # The last step reuses the last search's mask: same output as a plain pass.
    q, k, v, _ = inputs(7)
    idx = caq.build_block_index(masks[6])
    o, lse, _ = caq.sparse_attn_fwd(q, k, v, w.seq_len, w.block, idx.row_ptr, idx.col_idx)
    torch.cuda.synchronize()
    assert torch.equal(o, gs.sparse.o) and torch.equal(lse, gs.sparse.lse)


@pytest.mark.parametrize("case", ["ragged128", "ragged64"])
def test_mask_recall_matches_oracle(case):
    """Recall of a mask from the block weights of a full pass, against the full softmax."""
    dev = gpu()
    if case == "ragged128":
        w = synth.random_tiny_case(31, heads=2, seq_len=1000, head_dim=128, block=128,
                                   density=0.4)
    else:
        w = synth.random_tiny_case(32, heads=2, seq_len=700, head_dim=64, block=64, density=0.3)
    H, mb = w.mask.shape[0], w.mask.shape[1]
    banner(f"mask recall {case}")
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    ones = torch.ones(H, mb, mb, dtype=torch.uint8, device=dev)
    idx = caq.build_block_index(ones)
    _, lse, g = caq.sparse_attn_fwd(q, k, v, w.seq_len, w.block, idx.row_ptr, idx.col_idx,
                                    with_g=True)
    wts = caq.block_importance(g, lse, idx.row_ptr, w.seq_len, w.block)
    rec = caq.mask_recall(wts, idx.row_ptr, idx.col_idx, w.mask.to(dev))
    rec_all = caq.mask_recall(wts, idx.row_ptr, idx.col_idx, ones)
    torch.cuda.synchronize()
    ref = oracle.mask_recall(np64(w.q), np64(w.k), w.mask.cpu().numpy(), w.seq_len, w.block,
                             w.scale)
    np.testing.assert_allclose(rec.cpu().numpy(), ref, rtol=0, atol=2e-4)
    np.testing.assert_allclose(rec_all.cpu().numpy(), 1.0, rtol=0, atol=2e-4)


def test_schedule_diagnostics_match_plain_schedule():
    """A schedule with diagnostics gives the same outputs and masks as without, and its
    per-step entropy and distance are finite and non-negative."""
    dev = gpu()
    w = synth.random_tiny_case(31, heads=2, seq_len=1200, head_dim=64, block=64, density=1.0,
                               device=dev)
    banner("GSRS schedule with diagnostics")
    p = caq.ReorderParams(wave=8, n_slices=8, skip_mode=caq.WA_SKIP_NEVER)
    kw = dict(steps=6, search_steps=(2, 4), thresholds=(0.9, 0.8))
    a = GsrsSchedule(2, w.seq_len, 64, 64, dev, reorder=p, **kw)
    b = GsrsSchedule(2, w.seq_len, 64, 64, dev, reorder=p, diagnostics=True, **kw)
    inputs = lambda t: (w.q, w.k, w.v, w.x0)  # noqa: E731
    a.run(inputs)
    b.run(inputs)
    torch.cuda.synchronize()
    assert torch.equal(a.mask, b.mask) and torch.equal(a.s1, b.s1)
    assert torch.equal(a.sparse.o, b.sparse.o) and torch.equal(a.sparse.lse, b.sparse.lse)
    assert [k for _, k, _, _ in b.trace] == b.kinds
    for _, _, e, dist in b.trace:
        assert math.isfinite(float(e)) and float(e) >= 0.0
        assert math.isfinite(float(dist)) and float(dist) >= 0.0


def test_gsrs_schedule_matches_the_oracle_step_by_step():
    """GsrsSchedule against oracle.gsrs_schedule on drifting inputs: the same kind of
    step, the same mask at every step (Top-p of each search decided on the GPU's W, so
    the sets compare bit for bit), W at every search within the dense-pass tolerance
    of the oracle's W over the same candidates, and the last step's O and LSE against
    the oracle's attention under the last mask."""
    w = synth.make_workload("gsrs75k", device="cuda", heads=2, grid=(2, 45, 80))
    _schedule_vs_oracle(w, (2, 4, 6), (0.95, 0.9, 0.8), 8)


def _schedule_vs_oracle(w, search, thresholds, steps):
    dev = gpu()
    H, mb = w.mask.shape[0], w.mask.shape[1]
    banner(f"gsrs schedule vs oracle H={H} MB={mb} steps={steps} searches={search} "
           f"p={thresholds}")
    states = synth.drift_states(w, len(search) + 1)
    n_xcd = caq.schedule_info(0, w.head_dim)[0]
    params = caq.ReorderParams(wave=64, n_slices=n_xcd, iters=5, skip_mode=caq.WA_SKIP_NEVER)
    gs = GsrsSchedule(H, w.seq_len, w.head_dim, w.block, dev, reorder=params, steps=steps,
                      search_steps=search, thresholds=thresholds)

    def state(t):
        return states[sum(1 for s_ in search if t >= s_)]

    masks, w_gpu = [], {}

    def on_step(t, kind):
        masks.append(gs.mask.clone())
        if kind == "search":
            path = gs.full if t == search[0] else gs.search
            nnz = int(path.row_ptr[-1].item())
            w_gpu[t] = path.w[:nnz].clone()

    gs.run(lambda t: (*state(t)[:3], w.x0), on_step)
    torch.cuda.synchronize()
    qk = {}

    def qk_at(t):
        i = sum(1 for s_ in search if t >= s_)
        if i not in qk:
            qk[i] = (np64(states[i][0]), np64(states[i][1]))
        return qk[i]

    wsel = {t: v.cpu().numpy() for t, v in w_gpu.items()}
    kinds, masks_ref, w_ref = oracle.gsrs_schedule(steps, search, thresholds, qk_at,
                                                   w.seq_len, w.block, w.scale, w_select=wsel)
    assert gs.kinds == kinds
    for t in range(steps):
        if kinds[t] == "warmup":
            continue  # the warmup runs the dense pass; the schedule keeps no mask then
        np.testing.assert_array_equal(masks[t].cpu().numpy(), masks_ref[t], err_msg=f"step {t}")
    for t in search:
        np.testing.assert_allclose(wsel[t].astype(np.float64), w_ref[t], atol=2e-4, rtol=1e-3,
                                   err_msg=f"W at step {t}")
    # the last step: attention under the last mask with that step's inputs
    q, k, v = (np64(x) for x in state(steps - 1)[:3])
    L = w.seq_len
    o_ref, lse_ref = oracle.masked_attention(q, k, v, masks_ref[-1], L, w.block, w.scale)
    from helpers import assert_attention_close
    assert_attention_close(np64(gs.sparse.o)[:, :L], gs.sparse.lse.cpu().numpy().astype(np.float64)[:, :L],
                           o_ref[:, :L], lse_ref[:, :L], "last schedule step")


@pytest.mark.parametrize("seed", range(8))
def test_gsrs_schedule_random_sweep(seed):
    """Seeded random schedules against oracle.gsrs_schedule: grid, head count, step
    count, search steps (a first search at step 0, no warmup, included) and thresholds."""
    rng = np.random.default_rng(9300 + seed)
    grid = [(1, 20, 40), (2, 30, 40), (3, 24, 40), (2, 45, 80)][int(rng.integers(0, 4))]
    steps = int(rng.integers(2, 10))
    # searches before the last step, so that the last step reuses a mask (the step whose
    # output is compared with the oracle's attention)
    n_search = int(rng.integers(1, min(4, steps - 1) + 1))
    search = tuple(sorted(int(x) for x in rng.choice(steps - 1, size=n_search, replace=False)))
    thresholds = tuple(round(float(x), 3) for x in rng.uniform(0.5, 0.99, size=n_search))
    w = synth.make_workload("gsrs75k", device="cuda", heads=int(rng.integers(1, 3)), grid=grid)
    _schedule_vs_oracle(w, search, thresholds, steps)


@pytest.mark.parametrize("seed", range(48))
def test_topp_random_sweep(seed):
    """Seeded random shapes (rows of up to 1,600 candidates: every register-sort size and
    the LDS sort), densities, thresholds p in (0, 1] and weights with ties, one-hot,
    uniform and peaked rows: the kept sets bit-exact for the same W."""
    dev = gpu()
    rng = np.random.default_rng(9700 + seed)
    H = int(rng.integers(1, 4))
    mb = int(rng.integers(1, 40))
    nb = int(rng.choice([int(rng.integers(1, 70)), int(rng.integers(70, 600)),
                         int(rng.integers(600, 1600))]))
    dens = float(rng.choice([0.02, 0.2, 0.6, 1.0]))
    p = float(rng.choice([float(rng.uniform(0.05, 1.0)), 1.0, 0.9]))
    mask = (rng.random((H, mb, nb)) < dens).astype(np.uint8)
    mask[0, 0, 0] = 1  # at least one candidate, so that the index arrays are not empty
    rp, ci, _, _, _ = oracle.block_index(mask)
    w = _random_weights(rng, rp)
    banner(f"topp sweep seed={seed} H={H} MB={mb} NB={nb} density={dens} p={p}")
    sel = caq.topp_select(torch.from_numpy(w).to(dev), torch.from_numpy(rp.astype(np.int32)).to(dev),
                          torch.from_numpy(ci.astype(np.int32)).to(dev), H, mb, nb, p)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sel.cpu().numpy(), oracle.topp_select(w, rp, ci, H, mb, nb, p))
