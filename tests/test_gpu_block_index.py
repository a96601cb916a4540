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


@pytest.mark.parametrize("offset", [1, 2, 3, 7, 8, 15])
def test_block_index_unaligned_mask_and_odd_rows(offset):
    """The kernels read the mask four and sixteen bytes per lane: a mask that starts
    off a 16-byte boundary, rows whose length is not a multiple of 16 (or that take
    a wavefront two passes), non-zero values other than 1 and non-zero bytes right
    outside the mask must all give the oracle's lists; 2,100 rows give the prefix
    sum runs of three counts per thread."""
    dev = gpu()
    rng = np.random.default_rng(offset)
    for H, MB, NB in ((1, 3, 5), (2, 7, 131), (3, 33, 2), (1, 2, 1), (1, 3, 16), (1, 4, 17),
                      (2, 5, 1100), (3, 700, 4)):
        m = (rng.random((H, MB, NB)) < 0.4).astype(np.uint8) * rng.integers(1, 255, (H, MB, NB),
                                                                             dtype=np.uint8)
        n = H * MB * NB
        buf = torch.full((offset + n + 5,), 255, dtype=torch.uint8, device=dev)
        buf[offset:offset + n] = torch.from_numpy(m.reshape(-1)).to(dev)
        mask = buf[offset:offset + n].view(H, MB, NB)
        assert mask.data_ptr() % 4 == offset % 4
        banner(f"block_index unaligned offset={offset} H={H} MB={MB} NB={NB}")
        idx = caq.build_block_index(mask)
        torch.cuda.synchronize()
        rp, ci, nnz, cp, csi = oracle.block_index((m != 0).astype(np.uint8))
        total = int(rp[-1])
        assert np.array_equal(idx.row_ptr.cpu().numpy(), rp)
        assert np.array_equal(idx.row_nnz.cpu().numpy(), nnz)
        assert np.array_equal(idx.col_idx.cpu().numpy()[:total], ci)
        assert np.array_equal(idx.csc_ptr.cpu().numpy(), cp)
        assert np.array_equal(idx.csc_idx.cpu().numpy()[:total], csi)
