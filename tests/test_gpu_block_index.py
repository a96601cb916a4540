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


@pytest.mark.parametrize("seed", range(48))
def test_block_index_random_sweep(seed):
    """Seeded random shapes (rectangular, 1 to 900 blocks a side), densities, byte
    values, mask offsets and capacities: the CSR and CSC bit-exact up to the capacity,
    the true totals always, and nothing written at or past the capacity (the output
    buffers are longer and pre-filled with a sentinel)."""
    dev = gpu()
    rng = np.random.default_rng(9900 + seed)
    H = int(rng.integers(1, 4))
    MB = int(rng.choice([int(rng.integers(1, 20)), int(rng.integers(20, 900))]))
    NB = int(rng.choice([int(rng.integers(1, 20)), int(rng.integers(20, 900))]))
    dens = float(rng.choice([0.0, 0.01, 0.1, 0.5, 1.0]))
    m = ((rng.random((H, MB, NB)) < dens) *
         rng.integers(1, 256, (H, MB, NB))).astype(np.uint8)
    rp, ci, nnz, cp, csi = oracle.block_index((m != 0).astype(np.uint8))
    total = int(rp[-1])
    cap = int(rng.choice([total, int(rng.integers(0, total + 1)), H * MB * NB]))
    offset = int(rng.integers(0, 16))
    n = H * MB * NB
    buf = torch.full((offset + n + 16,), 255, dtype=torch.uint8, device=dev)
    buf[offset:offset + n] = torch.from_numpy(m.reshape(-1)).to(dev)
    mask = buf[offset:offset + n].view(H, MB, NB)
    i32 = dict(dtype=torch.int32, device=dev)
    row_ptr = torch.empty(H * MB + 1, **i32)
    row_nnz = torch.empty(H * MB, **i32)
    csc_ptr = torch.empty(H * NB + 1, **i32)
    col_idx = torch.full((cap + 64,), -7, **i32)
    csc_idx = torch.full((cap + 64,), -7, **i32)
    banner(f"block_index sweep seed={seed} H={H} MB={MB} NB={NB} density={dens} "
           f"total={total} cap={cap} offset={offset}")
    lib = caq.load_library()
    caq._check(lib.wa_build_block_index(caq._ptr(mask), H, MB, NB, caq._ptr(row_ptr),
                                        caq._ptr(col_idx), cap, caq._ptr(row_nnz),
                                        caq._ptr(csc_ptr), caq._ptr(csc_idx), cap,
                                        caq._stream(dev)), "wa_build_block_index")
    torch.cuda.synchronize()
    kept = min(cap, total)
    np.testing.assert_array_equal(row_ptr.cpu().numpy(), rp)
    np.testing.assert_array_equal(row_nnz.cpu().numpy(), nnz)
    np.testing.assert_array_equal(csc_ptr.cpu().numpy(), cp)
    got_c, got_t = col_idx.cpu().numpy(), csc_idx.cpu().numpy()
    np.testing.assert_array_equal(got_c[:kept], ci[:kept])
    np.testing.assert_array_equal(got_t[:kept], csi[:kept])
    assert (got_c[kept:] == -7).all() and (got_t[kept:] == -7).all()
