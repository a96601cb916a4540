"""Calibration of the adaptive reorder skip on the GPU it runs on.

WaveAlign (§IV-E, §VI-F and Fig. 13) skips the reorder when it cannot pay for
itself: short sequences whose K/V working set already fits the cache, very sparse
masks with too little work, and masks whose adjacent rows are already similar.
The page decides from mask statistics and offline profiles of kernel latency and
reorder cost but gives no formula.  This module measures those profiles on the
local GPU, over a grid of sequence lengths and densities with the Wan-shaped
generator, and fits the three thresholds of the skip rule used by
wa_reorder_rows:

    reorder a head  iff  K/V bytes > ws_min_bytes
                    and  selected FLOP >= flops_min
                    and  adjacent-row Jaccard < jaccard_max

The fit picks the thresholds that make the most sweep points decide correctly
(reorder exactly where index + reorder + reordered kernel beat index + the
better unreordered kernel), each placed in the middle of the gap it falls in.  The result is
written as JSON next to this file and read by ReorderParams.calibrated().

Usage (on the GPU):  python -m cache_aware_query_amd.calibrate [--out PATH]
"""

from __future__ import annotations

import argparse
import itertools
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_PATH = os.path.join(HERE, "calib_mi355x.json")

FRAMES = (2, 4, 9, 18, 36)            # 7,200 .. 129,600 tokens on a 45 x 80 frame
DENSITIES = (0.02, 0.05, 0.10, 0.20, 0.40)


def _time(fn, budget_ms: float = 150.0) -> float:
    """Mean milliseconds per call, repeating until about ``budget_ms`` is spent."""
    import torch

    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    a.record()
    fn()
    b.record()
    torch.cuda.synchronize()
    reps = max(3, min(200, int(budget_ms / max(a.elapsed_time(b), 1e-3))))
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def measure(frames: int, density: float, heads: int, iters: int) -> dict:
    """One sweep point: per-head statistics and the reordered / unreordered times."""
    import torch

    from . import (WA_SCHED_NATURAL, WA_SCHED_XCD_SLICED, WA_SKIP_NEVER, ReorderParams,
                   schedule_info)
    from .pipeline import HotPath
    import synth

    dev = torch.device("cuda:0")
    w = synth.make_workload("wan75k", device=dev, grid=(frames, 45, 80), heads=heads,
                            density=density)
    H, mb = w.mask.shape[0], w.mask.shape[1]
    nnz = int(w.mask.sum())
    n_xcd, _, wave = schedule_info(0, w.head_dim)
    p = ReorderParams(wave=wave, n_slices=n_xcd, iters=iters, skip_mode=WA_SKIP_NEVER)
    hp = HotPath(H, w.seq_len, w.head_dim, w.block, dev, capacity=nnz, reorder=p,
                 schedule=WA_SCHED_XCD_SLICED, gsrs_p=None)
    hp.build_index(w.mask)
    hp.reorder_rows(w.x0)
    t_index = _time(lambda: hp.build_index(w.mask))
    t_reorder = _time(lambda: hp.reorder_rows(w.x0))
    t_reord = _time(lambda: hp.attention(w.q, w.k, w.v))
    stats = hp.stats.cpu().double()
    del hp
    hp = HotPath(H, w.seq_len, w.head_dim, w.block, dev, capacity=nnz, reorder=None,
                 schedule=WA_SCHED_XCD_SLICED, gsrs_p=None)
    hp.build_index(w.mask)
    t_index_id = _time(lambda: hp.build_index(w.mask))
    t_xcd = _time(lambda: hp.attention(w.q, w.k, w.v))
    hp.schedule = WA_SCHED_NATURAL
    t_nat = _time(lambda: hp.attention(w.q, w.k, w.v))
    del hp, w
    torch.cuda.empty_cache()
    e2e_reord = t_index + t_reorder + t_reord
    e2e_plain = t_index_id + min(t_xcd, t_nat)
    return {
        "frames": frames, "seq_len": frames * 45 * 80, "density_target": density, "heads": H,
        "mb": mb, "density": float(stats[:, 1].mean()),
        "ws_bytes": float(stats[:, 2].mean()), "flops_per_head": float(stats[:, 3].mean()),
        "jaccard": float(stats[:, 4].mean()),
        "t_reorder_ms": t_reorder, "t_attn_reordered_ms": t_reord,
        "t_attn_identity_xcd_ms": t_xcd, "t_attn_natural_ms": t_nat,
        "e2e_reordered_ms": e2e_reord, "e2e_unreordered_ms": e2e_plain,
        "gain_ms": e2e_plain - e2e_reord, "reorder_wins": bool(e2e_plain > e2e_reord),
    }


def _gaps(values, geometric: bool):
    """Thresholds in the middle of every gap between consecutive distinct values,
    plus one below the smallest and one above the largest."""
    v = sorted(set(values))
    mid = (lambda x, y: (x * y) ** 0.5) if geometric else (lambda x, y: 0.5 * (x + y))
    out = [v[0] * 0.5 if geometric else v[0] - 1.0]
    out += [mid(x, y) for x, y in zip(v, v[1:])]
    out.append(v[-1] * 2.0 if geometric else v[-1] + 1.0)
    return out


def fit(points: list) -> dict:
    """Thresholds (ws_min_bytes, flops_min, jaccard_max) deciding most points right.

    Candidates sit in the middle of the gaps between observed statistic values
    (geometric middles for the byte and FLOP counts), so a threshold is as far as
    possible from the points on either side.  Among the rules that decide the
    most points right, the one whose wrong reorders lose the least time wins, and
    remaining ties go to the least restrictive rule (larger jaccard_max, then
    smaller ws_min, then smaller flops_min): a statistic that the sweep does not
    need in order to separate wins from losses does not cause skips."""
    ws_c = _gaps([pt["ws_bytes"] for pt in points], True)
    fl_c = _gaps([pt["flops_per_head"] for pt in points], True)
    jc_c = [min(max(j, 0.0), 1.0 + 1e-9) for j in _gaps([pt["jaccard"] for pt in points], False)]
    jc_c += [0.0, 1.0 + 1e-9]
    best = None
    for ws, fl, jc in itertools.product(ws_c, fl_c, sorted(set(jc_c))):
        dec = [pt["ws_bytes"] > ws and pt["flops_per_head"] >= fl and pt["jaccard"] < jc
               for pt in points]
        correct = sum(d == pt["reorder_wins"] for d, pt in zip(dec, points))
        lost = sum(max(0.0, -pt["gain_ms"]) for d, pt in zip(dec, points) if d)
        key = (correct, -lost, jc, -ws, -fl)
        if best is None or key > best[0]:
            best = (key, ws, fl, jc)
    (correct, _, _, _, _), ws, fl, jc = best
    return {"ws_min_bytes": max(ws, 0.0), "flops_min": max(fl, 0.0), "jaccard_max": jc,
            "points_correct": correct, "points": len(points)}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--out", default=DEFAULT_PATH)
    ap.add_argument("--heads", type=int, default=40)
    ap.add_argument("--iters", type=int, default=5)
    args = ap.parse_args(argv)
    root = os.path.dirname(HERE)
    if root not in sys.path:
        sys.path.insert(0, root)
    import torch

    points = []
    t0 = time.time()
    for frames, dens in itertools.product(FRAMES, DENSITIES):
        pt = measure(frames, dens, args.heads, args.iters)
        points.append(pt)
        print(f"[calibrate] L={pt['seq_len']:>6} rho={pt['density']:.3f} "
              f"reorder={pt['t_reorder_ms']:.3f} ms kernel {pt['t_attn_reordered_ms']:.3f} vs "
              f"{min(pt['t_attn_identity_xcd_ms'], pt['t_attn_natural_ms']):.3f} ms "
              f"gain {pt['gain_ms']:+.3f} ms ({time.time() - t0:.0f} s)", flush=True)
    thr = fit(points)
    props = torch.cuda.get_device_properties(0)
    out = {"device": f"{props.name} ({getattr(props, 'gcnArchName', '?')}, {props.multi_processor_count} CUs)", "iters": args.iters, "heads": args.heads,
           "rule": "reorder iff ws_bytes > ws_min_bytes and flops >= flops_min and "
                   "jaccard < jaccard_max", **thr, "sweep": points}
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps({k: v for k, v in out.items() if k != "sweep"}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
