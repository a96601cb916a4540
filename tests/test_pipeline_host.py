"""HotPath's host-side bound of the adaptive skip: when even a full mask could not
pass the size and work rules, no reorder is launched and every head keeps its order;
otherwise the decision is left to the device."""

import torch

import cache_aware_query_amd as caq
from cache_aware_query_amd.pipeline import HotPath


def _path(heads, seq_len, d, b, capacity, head_capacity=None, **kw):
    params = caq.ReorderParams(wave=64, n_slices=8, skip_mode=caq.WA_SKIP_ADAPTIVE, **kw)
    return HotPath(heads, seq_len, d, b, "cpu", capacity=capacity, reorder=params,
                   schedule=caq.WA_SCHED_AUTO, gsrs_p=None, head_capacity=head_capacity)


def test_small_shapes_are_skipped_on_the_host():
    # 16 x 16 blocks of 64 tokens, d = 64: at most 256 pairs of 1 MFLOP per head
    hp = _path(1, 1024, 64, 64, 256, flops_min=2.2e11)
    assert hp.host_skip
    assert torch.equal(hp.perm[0], torch.arange(16, dtype=torch.int32))
    assert torch.equal(hp.inv_perm[0], torch.arange(16, dtype=torch.int32))
    assert int(hp.skipped.sum()) == 1
    # the capacity bounds the pairs too: 128 x 128 blocks but only 16,000 entries
    assert _path(12, 16384, 128, 128, 16000, flops_min=2.2e11).host_skip


def test_a_per_head_capacity_tightens_the_bound():
    # 929 x 929 blocks of 128 x 128 at d = 128 with 41,016 entries over 24 heads: the
    # total alone allows a head 3.4e11 FLOP (above 3.17e11), a per-head bound of 2,000
    # entries at most 1.7e10
    params = dict(heads=24, seq_len=118800, d=128, b=128, capacity=41016, flops_min=3.17e11)
    assert not _path(**params).host_skip
    assert _path(**params, head_capacity=2000).host_skip
    assert not _path(**params, head_capacity=40000).host_skip


def test_large_or_unbounded_shapes_are_decided_on_the_device():
    # 591 x 591 blocks: a full head would be 2.9 TFLOP
    assert not _path(40, 75600, 128, 128, 2_000_000, flops_min=2.2e11).host_skip
    # the K/V bytes rule: 16 blocks of 64 x 64 are 262 KB, a threshold above that skips
    assert _path(1, 1024, 64, 64, 256, ws_min_bytes=1e6, flops_min=0.0).host_skip
    assert not _path(1, 1024, 64, 64, 256, ws_min_bytes=1e3, flops_min=0.0).host_skip
    # only the adaptive mode is bounded on the host
    hp = HotPath(1, 1024, 64, 64, "cpu", capacity=256,
                 reorder=caq.ReorderParams(skip_mode=caq.WA_SKIP_NEVER, flops_min=1e30),
                 schedule=caq.WA_SCHED_XCD_SLICED, gsrs_p=None)
    assert not hp.host_skip
