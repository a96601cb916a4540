"""The hot path under HIP graph capture and on concurrent streams.

A captured step (index -> reorder -> attention with G -> W -> Top-p) is replayed
several times, with eager work and synchronisations between the replays, and every
replay must give bitwise the outputs of the eager step.  Two paths run at once on two
streams must give bitwise what each gives alone.
"""

import pytest
import torch

import cache_aware_query_amd as caq
import synth
from cache_aware_query_amd.pipeline import HotPath
from helpers import banner, gpu

pytestmark = pytest.mark.gpu


def _path(w, schedule, skip_mode):
    dev = gpu()
    H, mb = w.mask.shape[0], w.mask.shape[1]
    n_xcd, _, wave = caq.schedule_info(0, w.head_dim)
    params = caq.ReorderParams(wave=wave, n_slices=n_xcd, iters=5, skip_mode=skip_mode)
    return HotPath(H, w.seq_len, w.head_dim, w.block, dev, capacity=int(w.mask.sum()),
                   reorder=params, schedule=schedule, gsrs_p=0.9)


def _outputs(hp, nnz):
    return [hp.o.clone(), hp.lse.clone(), hp.g[:nnz].clone(), hp.w[:nnz].clone(),
            hp.next_mask.clone(), hp.perm.clone(), hp.skipped.clone()]


@pytest.mark.parametrize("schedule,skip_mode", [
    (caq.WA_SCHED_XCD_SLICED, caq.WA_SKIP_NEVER),
    (caq.WA_SCHED_AUTO, caq.WA_SKIP_NEVER),
    (caq.WA_SCHED_AUTO, caq.WA_SKIP_ALWAYS),
])
def test_captured_step_replays_match_eager(schedule, skip_mode):
    dev = gpu()
    w = synth.make_workload("layer16k", device="cuda", heads=3)
    nnz = int(w.mask.sum())
    hp = _path(w, schedule, skip_mode)
    banner(f"graph capture of the step schedule={schedule} skip={skip_mode}")
    hp.step(w.q, w.k, w.v, w.mask, w.x0)
    torch.cuda.synchronize()
    ref = _outputs(hp, nnz)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        hp.step(w.q, w.k, w.v, w.mask, w.x0)
    for r in range(4):
        # eager work between the replays: every output cleared
        for t in (hp.o, hp.lse, hp.g, hp.w, hp.next_mask, hp.perm, hp.skipped):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _outputs(hp, nnz)
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"replay {r}: output {i} differs from the eager step"
    assert dev.type == "cuda"


def test_two_streams_match_serial():
    dev = gpu()
    wa = synth.make_workload("layer16k", device="cuda", heads=3)
    wb = synth.random_tiny_case(61, heads=2, seq_len=3000, head_dim=64, block=64, density=0.3,
                                empty_rows=(2,), device="cuda")
    paths = [(_path(wa, caq.WA_SCHED_AUTO, caq.WA_SKIP_NEVER), wa),
             (_path(wb, caq.WA_SCHED_XCD_SLICED, caq.WA_SKIP_NEVER), wb)]
    banner("two streams against serial")
    serial = []
    for hp, w in paths:
        hp.step(w.q, w.k, w.v, w.mask, w.x0)
        torch.cuda.synchronize()
        serial.append(_outputs(hp, int(w.mask.sum())))
    for hp, w in paths:
        for t in (hp.o, hp.lse, hp.g, hp.w, hp.next_mask, hp.perm):
            t.zero_()
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=dev) for _ in paths]
    for _ in range(3):
        for (hp, w), s in zip(paths, streams):
            with torch.cuda.stream(s):
                hp.step(w.q, w.k, w.v, w.mask, w.x0)
    torch.cuda.synchronize()
    for (hp, w), ref in zip(paths, serial):
        got = _outputs(hp, int(w.mask.sum()))
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"output {i} differs from the serial run"
