"""wa_sparse_attn_fwd with scores spread over hundreds of log2 units, against the
fp64 oracle: along a query block's list the row maximum rises far beyond any lazy
reference bound (the output and the running sum are rescaled), blocks lie far
below the row maximum (their block log-sum-exp takes their own maximum as offset)
and the probabilities kept against a stale reference reach the top of their
allowed range.  Inputs: synth.wide_range_case (Q x 8, K blocks x {0, 1, 8})."""

import numpy as np
import pytest
import torch

import cache_aware_query_amd as caq
import oracle
import synth
from helpers import assert_attention_close, banner, gpu, np64

pytestmark = pytest.mark.gpu

CASES = [(1000, 128, 128), (700, 64, 64), (1100, 128, 64)]


@pytest.mark.parametrize("seq_len,head_dim,block", CASES)
@pytest.mark.parametrize("with_g", [False, True])
def test_wide_score_range_matches_oracle(seq_len, head_dim, block, with_g):
    w = synth.wide_range_case(seq_len + head_dim + block, heads=2, seq_len=seq_len,
                              head_dim=head_dim, block=block)
    banner(f"wide range L={seq_len} d={head_dim} b={block} G={with_g}")
    dev = gpu()
    q, k, v, mask = (t.to(dev) for t in (w.q, w.k, w.v, w.mask))
    idx = caq.build_block_index(mask)
    o, lse, g = caq.sparse_attn_fwd(q, k, v, w.seq_len, w.block, idx.row_ptr, idx.col_idx,
                                    with_g=with_g)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.masked_attention(np64(w.q), np64(w.k), np64(w.v), w.mask.numpy(),
                                             w.seq_len, w.block, w.scale)
    L = w.seq_len
    assert_attention_close(np64(o)[:, :L], lse.cpu().numpy().astype(np.float64)[:, :L],
                           o_ref[:, :L], lse_ref[:, :L], f"wide range L={L} b={block}")
    if not with_g:
        return
    rp, ci, _, _, _ = oracle.block_index(w.mask.numpy())
    nnz = int(rp[-1])
    g_ref, _ = oracle.block_lse(np64(w.q), np64(w.k), rp, ci, w.seq_len, w.block, w.scale)
    g_gpu = g.cpu().numpy()[:nnz].astype(np.float64)
    mb = w.mask.shape[1]
    for r in range(w.mask.shape[0] * mb):
        u = r % mb
        nrows = min(block, L - u * block)
        lo, hi = rp[r], rp[r + 1]
        if hi > lo:
            gg, gr = g_gpu[lo:hi, :nrows], g_ref[lo:hi, :nrows]
            assert not np.isnan(gg).any()
            np.testing.assert_allclose(gg, gr, atol=5e-3, rtol=0)
