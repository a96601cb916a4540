"""wa_minhash_order against the oracle's MinHash order: bit-exact permutations
(integer work) on small ragged cases, empty rows, one and two hash functions, with
and without Stage 2, and at full workload sizes."""

import numpy as np
import pytest
import torch

import cache_aware_query_amd as caq
import oracle
import synth
from helpers import banner, gpu

pytestmark = pytest.mark.gpu


def _check(mask, n_hash, wave, n_slices, stage2, seed=0):
    dev = gpu()
    a, b = synth.minhash_params(n_hash, seed=synth.workloads.BASE_SEED + seed)
    idx = caq.build_block_index(mask.to(dev))
    perm, inv = caq.minhash_order(idx, a, b, wave, n_slices, stage2)
    torch.cuda.synchronize()
    perm_o, inv_o = oracle.minhash_order(mask.cpu().numpy(), a, b, wave, n_slices, stage2)
    np.testing.assert_array_equal(perm.cpu().numpy(), perm_o)
    np.testing.assert_array_equal(inv.cpu().numpy(), inv_o)


@pytest.mark.parametrize("n_hash", [1, 2])
@pytest.mark.parametrize("stage2", [False, True])
@pytest.mark.parametrize("mb,density", [(16, 0.4), (100, 0.2), (591, 0.05), (760, 0.3)])
def test_minhash_order_matches_oracle(mb, density, stage2, n_hash):
    w = synth.random_tiny_case(mb + n_hash, heads=2, seq_len=mb * 64, head_dim=64, block=64,
                               density=density, empty_rows=(1, mb - 1))
    banner(f"minhash order MB={mb} rho={density} stage2={stage2} n_hash={n_hash}")
    _check(w.mask, n_hash, wave=8, n_slices=4, stage2=stage2, seed=n_hash)


@pytest.mark.parametrize("name,over", [("wan75k", {}), ("hunyuan119k", {"heads": 6})])
def test_minhash_order_full_size(name, over):
    w = synth.make_workload(name, device="cuda", **over)
    n_xcd, _, wave = caq.schedule_info(0, w.head_dim)
    banner(f"minhash order {name} {over}")
    _check(w.mask, 2, wave=wave, n_slices=n_xcd, stage2=True)


def _check_lsh(mask, n_bands, wave, n_slices, stage2, seed=0):
    dev = gpu()
    a, b = synth.minhash_params(2 * n_bands, seed=synth.workloads.BASE_SEED + 100 + seed)
    idx = caq.build_block_index(mask.to(dev))
    perm, inv = caq.lsh_order(idx, a, b, wave, n_slices, stage2)
    torch.cuda.synchronize()
    perm_o, inv_o = oracle.lsh_order(mask.cpu().numpy(), a, b, n_bands, wave, n_slices, stage2)
    np.testing.assert_array_equal(perm.cpu().numpy(), perm_o)
    np.testing.assert_array_equal(inv.cpu().numpy(), inv_o)


@pytest.mark.parametrize("n_bands", [1, 4])
@pytest.mark.parametrize("stage2", [False, True])
@pytest.mark.parametrize("mb,density", [(16, 0.4), (100, 0.05), (591, 0.02), (760, 0.3)])
def test_lsh_order_matches_oracle(mb, density, stage2, n_bands):
    """Low densities make many rows share buckets (few blocks per row), so the groups
    are large and joined across bands."""
    w = synth.random_tiny_case(mb + 7 * n_bands, heads=2, seq_len=mb * 64, head_dim=64, block=64,
                               density=density, empty_rows=(1, mb - 1))
    banner(f"lsh order MB={mb} rho={density} stage2={stage2} n_bands={n_bands}")
    _check_lsh(w.mask, n_bands, wave=8, n_slices=4, stage2=stage2, seed=n_bands)


def test_lsh_order_structured_and_largest():
    """Wan-shaped masks (similar neighbouring rows), and the largest supported mask
    (4,096 blocks per side) whose LDS holds four bands of edges."""
    w = synth.make_workload("wan75k", device="cuda", heads=4)
    n_xcd, _, wave = caq.schedule_info(0, w.head_dim)
    banner("lsh order wan75k heads=4")
    _check_lsh(w.mask, 4, wave=wave, n_slices=n_xcd, stage2=True)
    big = synth.random_tiny_case(91, heads=1, seq_len=4096 * 64 - 5, head_dim=64, block=64,
                                 density=0.001, empty_rows=(3,))
    banner("lsh order MB=4096")
    _check_lsh(big.mask, 4, wave=64, n_slices=8, stage2=True, seed=9)


def _sweep_case(seed):
    rng = np.random.default_rng(9500 + seed)
    mb = int(rng.choice([int(rng.integers(1, 40)), int(rng.integers(40, 600)),
                         int(rng.integers(600, 1500))], p=[0.4, 0.4, 0.2]))
    w = synth.random_tiny_case(800 + seed, heads=int(rng.integers(1, 4)), seq_len=mb * 64,
                               head_dim=64, block=64,
                               density=float(rng.choice([0.005, 0.02, 0.1, 0.4, 0.9])),
                               diagonal=bool(rng.random() < 0.7),
                               empty_rows=tuple(int(x) for x in rng.choice(
                                   mb, size=min(mb, int(rng.integers(0, 3))), replace=False)))
    return (w, int(rng.choice([1, 2])), int(rng.integers(1, 5)),
            int(rng.choice([1, 7, 32, 64, 100])), int(rng.choice([1, 2, 3, 8, 16])),
            bool(rng.random() < 0.7))


@pytest.mark.parametrize("seed", range(48))
def test_comparator_random_sweep(seed):
    """Seeded random sizes (1 to 1,499 blocks), densities, hash and band counts, wave
    sizes, slice counts (more slices than blocks included) and Stage 2 on or off."""
    w, n_hash, n_bands, wave, n_slices, stage2 = _sweep_case(seed)
    banner(f"comparator sweep seed={seed} H={w.mask.shape[0]} MB={w.mask.shape[1]} "
           f"nnz={int(w.mask.sum())} n_hash={n_hash} n_bands={n_bands} wave={wave} "
           f"n_slices={n_slices} stage2={stage2}")
    _check(w.mask, n_hash, wave=wave, n_slices=n_slices, stage2=stage2, seed=seed)
    _check_lsh(w.mask, n_bands, wave=wave, n_slices=n_slices, stage2=stage2, seed=seed)
