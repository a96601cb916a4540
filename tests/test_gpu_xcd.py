"""The dispatch the XCD-sliced schedule relies on: workgroup w of a launch runs on
XCD w mod n_xcd (round-robin over the L2 domains), read back from the XCC_ID
hardware register of every workgroup (WaveAlign §II-C: a wave is the set of row
tasks resident at once on the processors that share one L2)."""

import pytest
import torch

import cache_aware_query_amd as caq
from helpers import banner, gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("block", [128, 64])
def test_workgroups_are_dealt_round_robin_over_the_xcds(block):
    gpu()
    n_xcd, cus, wave = caq.schedule_info(0, 128)
    assert n_xcd >= 1 and cus >= 1
    # the XCD-sliced grid of the Wan-shaped workload: H * n_xcd * ceil(MB / n_xcd)
    n_wg = 40 * n_xcd * ((591 + n_xcd - 1) // n_xcd)
    banner(f"XCD placement n_wg={n_wg} block={block} n_xcd={n_xcd}")
    xcd = caq.xcd_placement(n_wg, block).cpu()
    assert int(xcd.min()) >= 0 and int(xcd.max()) < max(n_xcd, 16)
    # the first n_xcd workgroups land on distinct XCDs, and workgroup w shares the XCD
    # of workgroup w mod n_xcd
    first = xcd[:n_xcd]
    assert len(set(first.tolist())) == n_xcd
    w = torch.arange(n_wg)
    assert torch.equal(xcd, first[w % n_xcd])
    print(f"XCD of workgroups 0..{n_xcd - 1}: {first.tolist()}", flush=True)
