"""Calibration of the adaptive reorder skip on the GPU it runs on.

WaveAlign (§IV-E, §VI-F and Fig. 13) skips the reorder when it cannot pay for
itself: short sequences whose K/V working set already fits the cache, very sparse
masks with too little work, and masks whose adjacent rows are already similar.
The page decides from mask statistics and offline profiles of kernel latency and
reorder cost but gives no formula.  This module measures those profiles on the
local GPU and fits the three thresholds of the skip rule used by wa_reorder_rows:

    reorder a head  iff  K/V bytes > ws_min_bytes
                    and  selected FLOP of the call's heaviest head >= flops_min
                    and  adjacent-row Jaccard < jaccard_max

(the work case is decided per call: the heads of one call are reordered side by
side, so the call costs what its slowest head costs.  Every head of a sweep point
has the same density, so there the per-head and per-call work coincide.)

The sweep has a locality axis besides length and density, so that the similarity
case has something to separate:

* ``topk-raster``   per-head Top-k of pooled scores, tokens in row-major (t, y, x)
                    order (the Wan-shaped generator), 2..36 frames x 2..40% density;
* ``topk-hilbert``  the same masks' rule with tokens along a generalized Hilbert
                    curve over (t, y, x), so neighbouring query blocks are compact
                    neighbouring chunks and their rows already overlap more;
* ``neighbour``     banded masks (Chebyshev-2 neighbours on the (frame, row band)
                    grid plus a few far blocks): adjacent rows nearly equal;
* ``topp-hilbert``  per-row Top-p(0.9) masks over Hilbert-ordered tokens (very
                    sparse, a few blocks per row);
* ``random``        Bernoulli blocks plus the diagonal: no locality to recover.

Each point times, with the caches flushed before every call, the chain index +
reorder + reordered kernel against index + the better unreordered kernel
(XCD-sliced or heads-interleaved).  The fit takes, among thresholds placed in the
middle of the gaps between observed statistic values, the rule with the least
relative time lost by wrong decisions (each wrong point costs |gain| over its best
chain), then the most points decided right, then the least restrictive rule, so a
statistic that the sweep does not need in order to separate wins from losses
causes no skips.  ``inert`` in the result names the thresholds that decide no
point.  The result is written as JSON next to this file and read by
ReorderParams.calibrated().

Usage (on the GPU):  python -m cache_aware_query_amd.calibrate [--out PATH]
"""

from __future__ import annotations

import argparse
import itertools
import json
import os
import statistics
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_PATH = os.path.join(HERE, "calib_mi355x.json")

WAN_FRAMES = (2, 4, 9, 18, 36)         # 7,200 .. 129,600 tokens on a 45 x 80 frame
WAN_DENSITIES = (0.02, 0.05, 0.10, 0.20, 0.40)

# family -> (generator config, overrides, grids, densities); a density of None keeps
# the generator's own rule (neighbour bands, Top-p)
FAMILIES = {
    "topk-raster": ("wan75k", {}, [(t, 45, 80) for t in WAN_FRAMES], WAN_DENSITIES),
    "topk-hilbert": ("wan75k", {"hilbert": True}, [(t, 45, 80) for t in WAN_FRAMES],
                     WAN_DENSITIES),
    "neighbour": ("layer16k", {}, [(t, 32, 32) for t in (16, 32, 64, 128)], (None,)),
    "topp-hilbert": ("hunyuan119k", {}, [(t, 45, 80) for t in (9, 18, 33)], (None,)),
    "random": ("random20", {}, [(t, 45, 80) for t in (9, 18, 36)], (0.05, 0.20)),
}


def _timer(flush):
    """Median milliseconds of ``fn`` over ``reps`` calls, caches flushed before each
    (a 1 GiB buffer streamed: four times the Infinity Cache)."""
    import torch

    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def run(fn, reps: int = 7) -> float:
        fn()
        out = []
        for _ in range(reps):
            flush.add_(1)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b))
        return statistics.median(out)
    return run


def measure(family: str, grid: tuple, density, heads: int, iters: int, timer) -> dict:
    """One sweep point: per-head statistics and the reordered / unreordered chains."""
    import torch

    from . import (WA_SCHED_HEADS_INTERLEAVED, WA_SCHED_XCD_SLICED, WA_SKIP_NEVER,
                   ReorderParams, schedule_info)
    from .pipeline import HotPath
    import synth

    cfg, over, _, _ = FAMILIES[family]
    dev = torch.device("cuda:0")
    kw = dict(over, grid=grid, heads=heads)
    if density is not None:
        kw["density"] = density
    w = synth.make_workload(cfg, device=dev, **kw)
    H, mb = w.mask.shape[0], w.mask.shape[1]
    nnz = int(w.mask.sum())
    n_xcd, _, wave = schedule_info(0, w.head_dim)
    p = ReorderParams(wave=wave, n_slices=n_xcd, iters=iters, skip_mode=WA_SKIP_NEVER)
    hp = HotPath(H, w.seq_len, w.head_dim, w.block, dev, capacity=nnz, reorder=p,
                 schedule=WA_SCHED_XCD_SLICED, gsrs_p=None)
    hp.build_index(w.mask)
    hp.reorder_rows(w.x0)
    torch.cuda.synchronize()
    stats = hp.stats.cpu().double().numpy()

    def reordered():
        hp.build_index(w.mask)
        hp.reorder_rows(w.x0)
        hp.attention(w.q, w.k, w.v)
    t_reorder = timer(lambda: hp.reorder_rows(w.x0))
    e2e_reord = timer(reordered)
    t_attn_reord = timer(lambda: hp.attention(w.q, w.k, w.v))
    del hp
    hp = HotPath(H, w.seq_len, w.head_dim, w.block, dev, capacity=nnz, reorder=None,
                 schedule=WA_SCHED_XCD_SLICED, gsrs_p=None)

    def plain():
        hp.build_index(w.mask)
        hp.attention(w.q, w.k, w.v)
    e2e_xcd = timer(plain)
    hp.schedule = WA_SCHED_HEADS_INTERLEAVED
    e2e_hi = timer(plain)
    del hp, w
    torch.cuda.empty_cache()
    e2e_plain = min(e2e_xcd, e2e_hi)
    return {
        "family": family, "grid": list(grid), "seq_len": grid[0] * grid[1] * grid[2],
        "density_target": density, "heads": H, "mb": mb,
        "density": float(stats[:, 1].mean()),
        "ws_bytes": float(stats[:, 2].mean()), "flops_per_head": float(stats[:, 3].mean()),
        "flops_per_head_range": [float(stats[:, 3].min()), float(stats[:, 3].max())],
        "jaccard": float(stats[:, 4].mean()),
        "jaccard_range": [float(stats[:, 4].min()), float(stats[:, 4].max())],
        "t_reorder_ms": t_reorder, "t_attn_reordered_ms": t_attn_reord,
        "e2e_reordered_ms": e2e_reord, "e2e_unreordered_xcd_ms": e2e_xcd,
        "e2e_unreordered_heads_interleaved_ms": e2e_hi, "e2e_unreordered_ms": e2e_plain,
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


def _cost(pt) -> float:
    """Relative time lost when the point is decided wrongly: |gain| over the best chain."""
    best = min(pt.get("e2e_reordered_ms", 0.0) or 0.0, pt.get("e2e_unreordered_ms", 0.0) or 0.0)
    return abs(pt["gain_ms"]) / best if best > 0 else abs(pt["gain_ms"])


def fit(points: list) -> dict:
    """Thresholds (ws_min_bytes, flops_min, jaccard_max) with the least relative time
    lost by wrong decisions; ties to the most points right, then the least
    restrictive rule (larger jaccard_max, smaller ws_min, smaller flops_min)."""
    ws = np.array([pt["ws_bytes"] for pt in points])
    fl = np.array([pt["flops_per_head"] for pt in points])
    jc = np.array([pt["jaccard"] for pt in points])
    wins = np.array([pt["reorder_wins"] for pt in points])
    cost = np.array([_cost(pt) for pt in points])
    ws_c = _gaps(ws.tolist(), True)
    fl_c = _gaps(fl.tolist(), True)
    jc_c = sorted(set([min(max(j, 0.0), 1.0 + 1e-9) for j in _gaps(jc.tolist(), False)]
                      + [0.0, 1.0 + 1e-9]))
    best = None
    for w_, f_ in itertools.product(ws_c, fl_c):
        base = (ws > w_) & (fl >= f_)
        for j_ in jc_c:
            dec = base & (jc < j_)
            wrong = dec != wins
            key = (-float(cost[wrong].sum()), int((~wrong).sum()), j_, -w_, -f_)
            if best is None or key > best[0]:
                best = (key, w_, f_, j_)
    (neg_lost, correct, _, _, _), w_, f_, j_ = best
    w_, f_ = max(w_, 0.0), max(f_, 0.0)
    inert = [name for name, dec in (("ws_min_bytes", ws > w_), ("flops_min", fl >= f_),
                                    ("jaccard_max", jc < j_)) if dec.all()]
    return {"ws_min_bytes": w_, "flops_min": f_, "jaccard_max": j_,
            "points_correct": correct, "points": len(points),
            "relative_time_lost": -neg_lost, "inert": inert}


def decide(point: dict, thr: dict) -> str:
    """Which case of the rule decides a point: 'reorder', 'size', 'work' or 'similar'."""
    if not point["ws_bytes"] > thr["ws_min_bytes"]:
        return "size"
    if not point["flops_per_head"] >= thr["flops_min"]:
        return "work"
    if not point["jaccard"] < thr["jaccard_max"]:
        return "similar"
    return "reorder"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--out", default=DEFAULT_PATH)
    ap.add_argument("--heads", type=int, default=40)
    ap.add_argument("--iters", type=int, default=5)
    ap.add_argument("--families", default=",".join(FAMILIES))
    args = ap.parse_args(argv)
    root = os.path.dirname(HERE)
    if root not in sys.path:
        sys.path.insert(0, root)
    import torch

    flush = torch.zeros(1 << 30, dtype=torch.uint8, device="cuda:0")
    timer = _timer(flush)
    points = []
    t0 = time.time()
    for fam in args.families.split(","):
        _, _, grids, dens = FAMILIES[fam]
        for grid, rho in itertools.product(grids, dens):
            pt = measure(fam, grid, rho, args.heads, args.iters, timer)
            points.append(pt)
            print(f"[calibrate] {fam:>12} L={pt['seq_len']:>6} rho={pt['density']:.3f} "
                  f"J={pt['jaccard']:.3f} reorder={pt['t_reorder_ms']:.3f} ms chain "
                  f"{pt['e2e_reordered_ms']:.3f} vs {pt['e2e_unreordered_ms']:.3f} ms "
                  f"gain {pt['gain_ms']:+.3f} ms ({time.time() - t0:.0f} s)", flush=True)
    thr = fit(points)
    for pt in points:
        pt["decided_by"] = decide(pt, thr)
    props = torch.cuda.get_device_properties(0)
    out = {"device": f"{props.name} ({getattr(props, 'gcnArchName', '?')}, "
                     f"{props.multi_processor_count} CUs)",
           "iters": args.iters, "heads": args.heads,
           "timing": "median of 7 calls, caches flushed (1 GiB streamed) before each; a chain "
                     "is index + reorder + attention, or index + attention",
           "rule": "reorder iff ws_bytes > ws_min_bytes and flops (of the call's heaviest "
                   "head) >= flops_min and jaccard < jaccard_max", **thr, "sweep": points}
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps({k: v for k, v in out.items() if k != "sweep"}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
