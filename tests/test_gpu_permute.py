"""Explicit reorder operators (WaveAlign §V) against the oracle, and the explicit
path (gather Q and mask rows, run, scatter O and LSE back) against the fused
indexing path: both give bitwise the same output."""

import numpy as np
import pytest
import torch

import cache_aware_query_amd as caq
import oracle
import synth
from helpers import banner, gpu

pytestmark = pytest.mark.gpu


def test_gather_scatter_match_oracle():
    dev = gpu()
    rng = np.random.default_rng(41)
    H, mb = 3, 37
    perm = np.stack([rng.permutation(mb) for _ in range(H)]).astype(np.int32)
    pt = torch.from_numpy(perm).to(dev)
    for rows, tail, dtype in ((8, (16,), torch.bfloat16), (1, (591,), torch.uint8),
                              (4, (), torch.float32), (2, (3,), torch.uint8)):
        x = torch.from_numpy(rng.integers(0, 200, size=(H, mb * rows) + tail).astype(np.float32))
        x = x.to(dtype)
        banner(f"permute rows={rows} tail={tail} {dtype}")
        g = caq.gather_blocks(x.to(dev), pt, rows)
        s = caq.scatter_blocks(g, pt, rows)
        torch.cuda.synchronize()
        xn = x.float().numpy()
        np.testing.assert_array_equal(g.float().cpu().numpy(), oracle.gather_blocks(xn, perm, rows))
        np.testing.assert_array_equal(s.float().cpu().numpy(), xn)


def test_explicit_path_equals_fused_path():
    dev = gpu()
    w = synth.make_workload("layer16k", device="cuda", heads=3)
    q, k, v, mask, x0 = w.q, w.k, w.v, w.mask, w.x0
    b = w.block
    banner("explicit vs fused reorder path")
    idx = caq.build_block_index(mask)
    ro = caq.reorder_rows(idx, x0, b, w.head_dim, caq.ReorderParams(skip_mode=caq.WA_SKIP_NEVER))
    o_f, lse_f, _ = caq.sparse_attn_fwd(q, k, v, w.seq_len, b, idx.row_ptr, idx.col_idx,
                                        perm=ro.perm, perm_slices=ro.n_slices)
    qg = caq.gather_blocks(q, ro.perm, b)
    mg = caq.gather_blocks(mask, ro.perm, 1)
    idx_g = caq.build_block_index(mg)
    o_g, lse_g, _ = caq.sparse_attn_fwd(qg, k, v, w.seq_len, b, idx_g.row_ptr, idx_g.col_idx,
                                        perm=None)
    o_e = caq.scatter_blocks(o_g, ro.perm, b)
    lse_e = caq.scatter_blocks(lse_g, ro.perm, b)
    torch.cuda.synchronize()
    assert dev.type == "cuda"
    assert torch.equal(o_e, o_f)
    assert torch.equal(lse_e, lse_f)
