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
