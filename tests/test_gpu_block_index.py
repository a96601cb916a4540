"""wa_build_block_index against the oracle's block index: bit-exact CSR and CSC."""

import numpy as np
import pytest
import torch

import cache_aware_query_amd as caq
import oracle
import synth
from helpers import banner, gpu

pytestmark = pytest.mark.gpu


def _check(mask_cpu: torch.Tensor, what: str):
    dev = gpu()
    banner(f"block_index {what} shape={tuple(mask_cpu.shape)}")
    idx = caq.build_block_index(mask_cpu.to(dev))
    torch.cuda.synchronize()
    rp, ci, nnz, cp, csi = oracle.block_index(mask_cpu.numpy())
    total = int(rp[-1])
    assert np.array_equal(idx.row_ptr.cpu().numpy(), rp), what
    assert np.array_equal(idx.row_nnz.cpu().numpy(), nnz), what
    assert np.array_equal(idx.col_idx.cpu().numpy()[:total], ci), what
    assert np.array_equal(idx.csc_ptr.cpu().numpy(), cp), what
    assert np.array_equal(idx.csc_idx.cpu().numpy()[:total], csi), what


@pytest.mark.parametrize("name", ["tiny", "layer16k"])
def test_block_index_on_workload_masks(name):
    _check(synth.make_workload(name).mask, name)


def test_block_index_random_edges():
    rng = np.random.default_rng(0)
    for H, MB, NB, dens in ((1, 1, 1, 1.0), (2, 3, 200, 0.3), (3, 130, 67, 0.05), (1, 64, 64, 0.0),
                            (2, 65, 129, 0.9)):
        m = (rng.random((H, MB, NB)) < dens).astype(np.uint8)
        if MB > 2:
            m[:, 1] = 0
        if NB > 3:
            m[:, :, 2] = 0
        _check(torch.from_numpy(m), f"random H={H} MB={MB} NB={NB} density={dens}")


def test_block_index_full_size_wan():
    w = synth.make_workload("wan75k", device="cuda")
    _check(w.mask.cpu(), "wan75k full size")


def test_block_index_full_size_hunyuan():
    # 929 blocks: a ragged last 64-column and 64-row tile in the transposed pass.
    w = synth.make_workload("hunyuan119k", device="cuda")
    _check(w.mask.cpu(), "hunyuan119k full size")


def test_block_index_capacity_truncation():
    dev = gpu()
    m = torch.ones(1, 8, 8, dtype=torch.uint8)
    banner("block_index capacity truncation")
    idx = caq.build_block_index(m.to(dev), capacity=10)
    torch.cuda.synchronize()
    assert int(idx.row_ptr[-1]) == 64           # the true total is still reported
    assert idx.col_idx.cpu().tolist()[:10] == list(range(8)) + [0, 1]
