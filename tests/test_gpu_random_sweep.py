"""A seeded sweep of small random cases through the whole path, each against the oracle.

Every case draws its block size, head dimension, block count, ragged tail, density,
head count, diagonal and empty rows from its seed, then checks:

- the CSR of the mask, bit for bit;
- O and LSE (the attention parity tolerances) and the block LSE G;
- the block weights W, and each query block's weights summing to 1;
- the Top-p sets for the GPU's own W, bit for bit;
- the reorder's permutations (each a permutation of the head's query blocks);
- O, LSE and G under those permutations, bitwise the same as in the original order;
- the explicit path (Q blocks and mask rows gathered into the new order, O and LSE
  scattered back), bitwise the same as the fused path;
- the row entropy and mean attention distance of the diagnostics pass, with O and LSE
  unchanged by asking for them.
"""

import numpy as np
import pytest
import torch

import cache_aware_query_amd as caq
import oracle
import synth
from helpers import assert_attention_close, banner, gpu, np64

pytestmark = pytest.mark.gpu

SEEDS = list(range(64))


def _case(seed):
    rng = np.random.default_rng(7000 + seed)
    block = int(rng.choice([64, 128]))
    head_dim = int(rng.choice([64, 128]))
    nb = int(rng.integers(1, 25))
    tail = int(rng.integers(1, block + 1))  # tokens in the last block
    seq_len = (nb - 1) * block + tail
    density = float(rng.choice([0.03, 0.1, 0.3, 0.6, 1.0]))
    heads = int(rng.integers(1, 4))
    diagonal = bool(rng.random() < 0.7)
    n_empty = min(nb, int(rng.integers(0, 3)))
    empty = tuple(int(x) for x in rng.choice(nb, size=n_empty, replace=False))
    p = float(rng.choice([0.5, 0.8, 0.9, 0.95]))
    w = synth.random_tiny_case(500 + seed, heads=heads, seq_len=seq_len, head_dim=head_dim,
                               block=block, density=density, diagonal=diagonal,
                               empty_rows=empty)
    return w, p


@pytest.mark.parametrize("seed", SEEDS)
def test_random_case_through_the_path(seed):
    w, p = _case(seed)
    H, mb, nb = w.mask.shape
    L, b, d = w.seq_len, w.block, w.head_dim
    banner(f"sweep seed={seed} H={H} L={L} d={d} b={b} MB={mb} nnz={int(w.mask.sum())} p={p}")
    dev = gpu()
    q, k, v, mask = (t.to(dev) for t in (w.q, w.k, w.v, w.mask))

    # CSR, bit for bit
    idx = caq.build_block_index(mask)
    rp, ci, _, _, _ = oracle.block_index(w.mask.numpy())
    nnz = int(rp[-1])
    np.testing.assert_array_equal(idx.row_ptr.cpu().numpy(), rp)
    np.testing.assert_array_equal(idx.col_idx.cpu().numpy()[:nnz], ci)

    # attention with G, against the oracle
    o, lse, g = caq.sparse_attn_fwd(q, k, v, L, b, idx.row_ptr, idx.col_idx, with_g=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.masked_attention(np64(w.q), np64(w.k), np64(w.v), w.mask.numpy(),
                                             L, b, w.scale)
    assert_attention_close(np64(o)[:, :L], lse.cpu().numpy().astype(np.float64)[:, :L],
                           o_ref[:, :L], lse_ref[:, :L], f"seed {seed}")
    g_ref, lse_g = oracle.block_lse(np64(w.q), np64(w.k), rp, ci, L, b, w.scale)
    g_gpu = g.cpu().numpy()[:nnz].astype(np.float64)
    for r in range(H * mb):
        lo, hi = rp[r], rp[r + 1]
        rows = min(b, L - (r % mb) * b)
        if hi > lo:
            np.testing.assert_allclose(g_gpu[lo:hi, :rows], g_ref[lo:hi, :rows], atol=5e-3,
                                       rtol=0, err_msg=f"seed {seed} G row {r}")

    # W, and Top-p decided on the GPU's W by both sides
    wts = caq.block_importance(g, lse, idx.row_ptr, L, b)
    torch.cuda.synchronize()
    w_gpu = wts.cpu().numpy()[:nnz]
    w_ref = oracle.block_importance(g_ref, lse_g, rp, L, b)
    for r in range(H * mb):
        lo, hi = rp[r], rp[r + 1]
        if hi > lo:
            np.testing.assert_allclose(w_gpu[lo:hi], w_ref[lo:hi], atol=2e-4, rtol=1e-3,
                                       err_msg=f"seed {seed} W row {r}")
            assert abs(float(w_gpu[lo:hi].astype(np.float64).sum()) - 1.0) < 1e-4
    sel = caq.topp_select(wts, idx.row_ptr, idx.col_idx, H, mb, nb, p)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sel.cpu().numpy(),
                                  oracle.topp_select(w_gpu, rp, ci, H, mb, nb, p))

    # the reorder's order, and the same outputs under it
    n_xcd, _, _ = caq.schedule_info(0, d)
    params = caq.ReorderParams(wave=max(1, mb // 3), n_slices=n_xcd, iters=5,
                               skip_mode=caq.WA_SKIP_NEVER)
    ro = caq.reorder_rows(idx, w.x0.to(dev), b, d, params)
    torch.cuda.synchronize()
    perm = ro.perm.cpu().numpy()
    for h in range(H):
        assert sorted(perm[h].tolist()) == list(range(mb))
    for sched in (caq.WA_SCHED_XCD_SLICED, caq.WA_SCHED_NATURAL):
        o1, lse1, g1 = caq.sparse_attn_fwd(q, k, v, L, b, idx.row_ptr, idx.col_idx,
                                           perm=ro.perm, perm_slices=ro.n_slices,
                                           schedule=sched, with_g=True)
        torch.cuda.synchronize()
        assert torch.equal(o1, o) and torch.equal(lse1, lse)
        assert torch.equal(g1[:nnz], g[:nnz])

    # the explicit path: gather, run in the new order, scatter back
    o_plain, lse_plain, _ = caq.sparse_attn_fwd(q, k, v, L, b, idx.row_ptr, idx.col_idx)
    qg = caq.gather_blocks(q, ro.perm, b)
    idx_g = caq.build_block_index(caq.gather_blocks(mask, ro.perm, 1))
    o_g, lse_g, _ = caq.sparse_attn_fwd(qg, k, v, L, b, idx_g.row_ptr, idx_g.col_idx)
    o_e = caq.scatter_blocks(o_g, ro.perm, b)
    lse_e = caq.scatter_blocks(lse_g, ro.perm, b)
    torch.cuda.synchronize()
    assert torch.equal(o_e, o_plain) and torch.equal(lse_e, lse_plain)

    # diagnostics: entropy LSE - E[z] and mean distance E|i - j| of every row
    ent = torch.empty(H, mb * b, dtype=torch.float32, device=dev)
    dist = torch.empty_like(ent)
    o_d, lse_d, _ = caq.sparse_attn_fwd(q, k, v, L, b, idx.row_ptr, idx.col_idx,
                                        entropy_out=ent, distance_out=dist)
    torch.cuda.synchronize()
    assert torch.equal(o_d, o_plain) and torch.equal(lse_d, lse_plain)
    m = w.mask.numpy()
    ref_e = oracle.attention_entropy(np64(w.q), np64(w.k), m, L, b, w.scale)[:, :L]
    ref_d = oracle.attention_distance(np64(w.q), np64(w.k), m, L, b, w.scale)[:, :L]
    ent_g, dist_g = ent.cpu().numpy()[:, :L], dist.cpu().numpy()[:, :L]
    assert np.all(np.isfinite(ent_g)) and np.all(np.isfinite(dist_g))
    np.testing.assert_allclose(ent_g, ref_e, rtol=0, atol=2e-2, err_msg=f"seed {seed} entropy")
    # bf16 probabilities: |error| < 2^-8 L per row (the bound of the diagnostics test)
    err = np.abs(dist_g - ref_d)
    assert err.max() < 2.0 ** -8 * max(L, 1), (seed, err.max())
