"""wa_reorder_rows against the oracle's reordering (same mask, same start block).

Bit-exact: the statistics and skip flags, the identity order of skipped heads,
permutation validity, and the Stage-2 structure (each bucket holds the positions
of the GPU's own angle order and is sorted by descending NNZ, ties in angle
order).  fp64 on both sides: angles agree with the oracle's to 1e-9, and the
permutations are equal except where the oracle itself has a near-tie.
"""

import numpy as np
import pytest
import torch

import cache_aware_query_amd as caq
import oracle
import synth
from helpers import banner, gpu

pytestmark = pytest.mark.gpu


def _gpu_reorder(mask, x0, block, head_dim, params):
    dev = gpu()
    idx = caq.build_block_index(mask.to(dev))
    ro = caq.reorder_rows(idx, x0.to(dev), block, head_dim, params)
    torch.cuda.synchronize()
    return ro


def _oracle_params(p: caq.ReorderParams):
    return oracle.ReorderParams(wave=p.wave, n_slices=p.n_slices, iters=p.iters,
                                stage1=p.stage1, stage2=p.stage2, skip_mode=p.skip_mode,
                                ws_min_bytes=p.ws_min_bytes, flops_min=p.flops_min,
                                jaccard_max=p.jaccard_max)


def _check_structure(perm, angles, nnz, skipped, p):
    """Validity and Stage-2 structure of one head's GPU permutation."""
    mb = perm.size
    assert sorted(perm.tolist()) == list(range(mb))
    if skipped:
        assert perm.tolist() == list(range(mb))
        return
    if p.stage1 and np.all(np.isfinite(angles)):
        order = np.argsort(angles, kind="stable")
    else:
        order = np.arange(mb)
    buckets = oracle.wave_buckets(mb, p.n_slices, p.wave) if p.stage2 else [(0, mb)]
    pos_in_order = np.empty(mb, dtype=np.int64)
    pos_in_order[order] = np.arange(mb)
    for lo, hi in buckets:
        seg = perm[lo:hi]
        assert sorted(seg.tolist()) == sorted(order[lo:hi].tolist())
        if p.stage2:
            key = list(zip((-nnz[seg]).tolist(), pos_in_order[seg].tolist()))
            assert key == sorted(key)
        else:
            assert seg.tolist() == order[lo:hi].tolist()


CASES = [
    ("tiny", {}, caq.ReorderParams(wave=4, n_slices=2, skip_mode=caq.WA_SKIP_NEVER)),
    ("layer16k", {}, caq.ReorderParams(wave=64, n_slices=8, skip_mode=caq.WA_SKIP_NEVER)),
    ("layer16k", {}, caq.ReorderParams(wave=32, n_slices=1, skip_mode=caq.WA_SKIP_NEVER)),
    ("layer16k", {}, caq.ReorderParams(wave=64, n_slices=8, skip_mode=caq.WA_SKIP_ADAPTIVE,
                                       jaccard_max=0.35, flops_min=1e11)),
    ("layer16k", {}, caq.ReorderParams(wave=16, n_slices=4, stage1=False,
                                       skip_mode=caq.WA_SKIP_NEVER)),
    ("layer16k", {}, caq.ReorderParams(wave=16, n_slices=4, stage2=False,
                                       skip_mode=caq.WA_SKIP_NEVER)),
    ("wan75k", {"heads": 4}, caq.ReorderParams(wave=64, n_slices=8, skip_mode=caq.WA_SKIP_NEVER)),
    ("gsrs75k", {"heads": 2}, caq.ReorderParams(wave=64, n_slices=8, skip_mode=caq.WA_SKIP_NEVER)),
    # 929 blocks: the column-bitmask form near its limit, very sparse Top-p masks
    ("hunyuan119k", {"heads": 3}, caq.ReorderParams(wave=64, n_slices=8,
                                                    skip_mode=caq.WA_SKIP_NEVER)),
    ("hunyuan119k", {"heads": 3}, caq.ReorderParams(wave=64, n_slices=8,
                                                    skip_mode=caq.WA_SKIP_ADAPTIVE,
                                                    flops_min=1e10, jaccard_max=0.9)),
    # skips decided before the mask is read (Jaccard reported as NaN): every head, and
    # a work threshold above every head's selected FLOP
    ("layer16k", {}, caq.ReorderParams(wave=64, n_slices=8, skip_mode=caq.WA_SKIP_ALWAYS)),
    ("hunyuan119k", {"heads": 6}, caq.ReorderParams(wave=64, n_slices=8,
                                                    skip_mode=caq.WA_SKIP_ADAPTIVE,
                                                    flops_min=1e12, jaccard_max=0.9)),
    # a work threshold between the heads' selected FLOP: the work case is decided per
    # call, so the heavier heads carry the lighter ones
    ("hunyuan119k", {"heads": 6}, caq.ReorderParams(wave=64, n_slices=8,
                                                    skip_mode=caq.WA_SKIP_ADAPTIVE,
                                                    flops_min=1.45e10, jaccard_max=0.9)),
    ("wan75k", {"heads": 6}, caq.ReorderParams(wave=64, n_slices=8,
                                               skip_mode=caq.WA_SKIP_ADAPTIVE,
                                               flops_min=3.17e11)),
]


@pytest.mark.parametrize("name,over,params", CASES)
def test_reorder_matches_oracle(name, over, params):
    w = synth.make_workload(name, device="cuda" if name != "tiny" else "cpu", **over)
    banner(f"reorder {name} {over} {params}")
    _compare_with_oracle(w, params)


@pytest.mark.parametrize("mb,density", [
    (1000, 0.005),  # one lane per list, pair statistics from LDS row bitmasks
    (1000, 0.05),   # four lanes per list, row-bitmask statistics
    (1200, 0.005),  # row bitmasks no longer fit: pair statistics by merging the lists
    (1200, 0.3),    # pair statistics walked row by row per wave
    (2100, 0.05),   # 2,100 blocks, 4,096-key sorts
])
def test_reorder_from_transposed_lists_matches_oracle(mb, density):
    """A mask too large for the LDS column bitmasks takes the CSR + CSC gather form."""
    w = synth.random_tiny_case(5, heads=2, seq_len=mb * 64, head_dim=64, block=64,
                               density=density, empty_rows=(3,))
    assert caq.reorder_needs_csc(mb, mb)
    banner(f"reorder {mb} x {mb} (CSC form) rho={density}")
    _compare_with_oracle(w, caq.ReorderParams(wave=64, n_slices=8,
                                              skip_mode=caq.WA_SKIP_NEVER))


@pytest.mark.parametrize("mb,density", [(950, 0.05), (972, 0.3)])
def test_reorder_bitmask_form_near_its_limit(mb, density):
    """The largest masks that still take the column-bitmask form."""
    w = synth.random_tiny_case(9, heads=2, seq_len=mb * 64, head_dim=64, block=64,
                               density=density, empty_rows=(3,))
    assert not caq.reorder_needs_csc(mb, mb)
    banner(f"reorder {mb} x {mb} (bitmask form) rho={density}")
    _compare_with_oracle(w, caq.ReorderParams(wave=64, n_slices=8,
                                              skip_mode=caq.WA_SKIP_NEVER))


def _ritz_gap(mask_h, x0_h, iters):
    """Relative gap (l1 - l2) / l1 of the projected 2 x 2 matrix whose eigenvectors the
    Ritz step rotates the basis onto (1 when the rotation is well defined by far)."""
    mt = oracle.reorder.centered_mask(mask_h)
    if not np.any(mt):
        return 1.0
    x = oracle.reorder._qr2(np.asarray(x0_h, dtype=np.float64))
    for _ in range(iters):
        x = oracle.reorder._qr2(mt @ (mt.T @ x))
    proj = x.T @ (mt @ (mt.T @ x))
    lam = np.linalg.eigvalsh(0.5 * (proj + proj.T))
    return float((lam[1] - lam[0]) / lam[1]) if lam[1] > 0 else 1.0


def _compare_with_oracle(w, params, gap_min=None):
    mask = w.mask.cpu()
    x0 = w.x0.cpu()
    ro = _gpu_reorder(mask, x0, w.block, w.head_dim, params)
    perm_g = ro.perm.cpu().numpy()
    inv_g = ro.inv_perm.cpu().numpy()
    skip_g = ro.skipped.cpu().numpy().astype(bool)
    ang_g = ro.angles.cpu().numpy()
    st_g = ro.stats.cpu().numpy()
    m = mask.numpy()
    perm_o, _, skip_o, ang_o, st_o = oracle.reorder_rows(m, x0.numpy().astype(np.float64),
                                                         w.block, w.head_dim,
                                                         _oracle_params(params))
    # nnz, density, K/V bytes and FLOP bit-exact; the adjacent-row Jaccard too, except
    # where the skip was decided without it (WA_SKIP_ALWAYS, or the size/work rule of
    # the adaptive skip), where the library reports NaN
    np.testing.assert_array_equal(st_g[:, :4], st_o[:, :4])
    op = _oracle_params(params)
    call_flops = st_o[:, 3].max()
    early = np.array([op.skip_mode == oracle.reorder.SKIP_ALWAYS or
                      (op.skip_mode == oracle.reorder.SKIP_ADAPTIVE and
                       not (st_o[h, 2] > op.ws_min_bytes and call_flops >= op.flops_min))
                      for h in range(st_o.shape[0])])
    np.testing.assert_array_equal(np.isnan(st_g[:, 4]), early)
    np.testing.assert_array_equal(st_g[~early, 4], st_o[~early, 4])
    np.testing.assert_array_equal(skip_g, skip_o)
    H, mb = perm_g.shape
    for h in range(H):
        nnz = m[h].astype(np.int64).sum(1)
        _check_structure(perm_g[h], ang_g[h], nnz, skip_g[h], params)
        np.testing.assert_array_equal(inv_g[h][perm_g[h]], np.arange(mb))
        if (gap_min is not None and not skip_g[h] and params.stage1 and
                _ritz_gap(m[h], x0.numpy()[h], params.iters) < gap_min):
            # two nearly equal Ritz values: the final rotation, and so the angles, are
            # fixed only up to rounding amplified by 1 / gap; both sides are valid
            continue
        both = np.isfinite(ang_o[h])
        np.testing.assert_array_equal(np.isfinite(ang_g[h]), both)
        np.testing.assert_allclose(ang_g[h][both], ang_o[h][both], atol=1e-9, rtol=0)
        if not np.array_equal(perm_g[h], perm_o[h]):
            # Only a near-tie of the oracle's own angles may reorder rows.
            srt = np.sort(ang_o[h][both])
            assert srt.size and np.min(np.diff(srt)) < 1e-9, f"head {h}: permutations differ"


def _sweep_case(seed):
    rng = np.random.default_rng(9100 + seed)
    block = int(rng.choice([64, 128]))
    head_dim = int(rng.choice([64, 128]))
    mb = int(rng.choice([int(rng.integers(1, 40)), int(rng.integers(40, 400)),
                         int(rng.integers(973, 1300))], p=[0.45, 0.4, 0.15]))
    density = float(rng.choice([0.01, 0.05, 0.2, 0.5, 0.9]))
    heads = int(rng.integers(1, 4))
    params = caq.ReorderParams(wave=int(rng.choice([1, 7, 32, 64, 100])),
                               n_slices=int(rng.choice([1, 2, 3, 8, 16])),
                               iters=int(rng.choice([0, 1, 5, 10])),
                               stage1=bool(rng.random() < 0.85),
                               stage2=bool(rng.random() < 0.85),
                               skip_mode=caq.WA_SKIP_NEVER)
    if rng.random() < 0.3:
        params = caq.ReorderParams(wave=params.wave, n_slices=params.n_slices,
                                   iters=params.iters, skip_mode=caq.WA_SKIP_ADAPTIVE,
                                   flops_min=float(10 ** rng.uniform(6, 12)),
                                   jaccard_max=float(rng.uniform(0.05, 1.0)))
    w = synth.random_tiny_case(700 + seed, heads=heads, seq_len=mb * block, head_dim=head_dim,
                               block=block, density=density, diagonal=bool(rng.random() < 0.7),
                               empty_rows=tuple(int(x) for x in rng.choice(
                                   mb, size=min(mb, int(rng.integers(0, 3))), replace=False)))
    return w, params


@pytest.mark.parametrize("seed", range(96))
def test_reorder_random_sweep_matches_oracle(seed):
    """Seeded random sizes (1 to 1,299 blocks, both index forms), densities, wave sizes,
    slice counts, iteration counts (0 included), stage switches and adaptive thresholds."""
    w, params = _sweep_case(seed)
    H, mb, _ = w.mask.shape
    banner(f"reorder sweep seed={seed} H={H} MB={mb} b={w.block} d={w.head_dim} "
           f"nnz={int(w.mask.sum())} {params}")
    _compare_with_oracle(w, params, gap_min=1e-5)


def test_reorder_is_deterministic():
    w = synth.make_workload("layer16k", heads=4)
    p = caq.ReorderParams(skip_mode=caq.WA_SKIP_NEVER)
    banner("reorder determinism")
    a = _gpu_reorder(w.mask, w.x0, w.block, w.head_dim, p)
    b = _gpu_reorder(w.mask, w.x0, w.block, w.head_dim, p)
    assert torch.equal(a.perm, b.perm) and torch.equal(a.angles.nan_to_num(), b.angles.nan_to_num())


def test_dense_mask_keeps_identity_stage1():
    m = torch.ones(2, 16, 16, dtype=torch.uint8)
    x0 = torch.rand(2, 16, 2) * 2 - 1
    banner("reorder dense mask")
    ro = _gpu_reorder(m, x0, 128, 128, caq.ReorderParams(wave=4, n_slices=2,
                                                         skip_mode=caq.WA_SKIP_NEVER))
    assert ro.perm.cpu().tolist() == [list(range(16))] * 2
    assert torch.isnan(ro.angles).all()
    ro = _gpu_reorder(m, x0, 128, 128, caq.ReorderParams(jaccard_max=0.9))
    assert ro.skipped.cpu().tolist() == [1, 1]


@pytest.mark.parametrize("mb,density", [(300, 0.1), (1200, 0.05)])
def test_unaligned_index_lists_take_the_single_entry_gathers(mb, density):
    """Index arrays that are not 16-byte aligned are gathered one entry per load; the
    result equals the four-entry gathers of the aligned copy up to summation order
    (angles to 1e-12, the same statistics, skip flags and Stage-2 structure).  Both the
    column-bitmask form (300 blocks) and the list form (1,200 blocks) are covered."""
    dev = gpu()
    w = synth.random_tiny_case(17, heads=2, seq_len=mb * 64, head_dim=64, block=64,
                               density=density, empty_rows=(5,))
    banner(f"reorder unaligned index lists MB={mb}")
    idx = caq.build_block_index(w.mask.to(dev))

    def shifted(t):
        if t is None:
            return None
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        buf[1:].copy_(t)
        return buf[1:]   # data pointer 4 bytes past a 16-byte boundary
    idx_u = caq.BlockIndex(idx.row_ptr, shifted(idx.col_idx), idx.row_nnz, idx.csc_ptr,
                           shifted(idx.csc_idx), idx.heads, idx.mb, idx.nb)
    assert idx_u.col_idx.data_ptr() % 16 == 4
    p = caq.ReorderParams(wave=16, n_slices=4, skip_mode=caq.WA_SKIP_NEVER)
    x0 = w.x0.to(dev)
    a = caq.reorder_rows(idx, x0, w.block, w.head_dim, p)
    b = caq.reorder_rows(idx_u, x0, w.block, w.head_dim, p)
    torch.cuda.synchronize()
    assert torch.equal(a.stats, b.stats) and torch.equal(a.skipped, b.skipped)
    torch.testing.assert_close(a.angles, b.angles, atol=1e-12, rtol=0)
    m = w.mask.numpy()
    for h in range(2):
        _check_structure(b.perm[h].cpu().numpy(), b.angles[h].cpu().numpy(),
                         m[h].astype(np.int64).sum(1), bool(b.skipped[h]), p)


@pytest.mark.parametrize("kind,mb,nb", [("hub", 97, 97), ("hub", 300, 300), ("rect", 70, 200),
                                        ("rect", 200, 70), ("rect", 33, 17)])
def test_reorder_fixed_point_products_at_their_edges(kind, mb, nb):
    """The column products of the bitmask form run on the int8 matrix cores in fixed
    point (basis entries times 2^53, |x| <= 1).  A hub row selecting every block puts
    most of a basis vector on one row (entries near 1, the top of the digit range);
    rectangular masks leave partial 16-row slices and 32-column tiles on both sides.
    Angles to 1e-9 of the oracle, as everywhere."""
    from types import SimpleNamespace
    rng = np.random.default_rng(mb * 1000 + nb)
    m = np.zeros((2, mb, nb), dtype=np.uint8)
    for h in range(2):
        if kind == "hub":
            m[h, 0] = 1
            m[h, np.arange(mb), rng.integers(0, nb, mb)] = 1
            m[h, np.arange(mb), np.arange(mb) % nb] = 1
        else:
            m[h] = (rng.random((mb, nb)) < 0.15 + 0.1 * h).astype(np.uint8)
            m[h, np.arange(mb), np.arange(mb) % nb] = 1
    w = SimpleNamespace(mask=torch.from_numpy(m), x0=torch.from_numpy(rng.uniform(-1, 1, (2, mb, 2)).astype(np.float32)),
                        block=64, head_dim=64)
    banner(f"reorder fixed-point products {kind} MB={mb} NB={nb}")
    assert not caq.reorder_needs_csc(mb, nb)
    _compare_with_oracle(w, caq.ReorderParams(wave=16, n_slices=4, skip_mode=caq.WA_SKIP_NEVER))
