"""Benchmark of the cache-aware block-sparse attention hot path on one MI355X.

One step = one pass of the whole path over the Wan-like workload (H=40, d=128,
L=75,600 tokens, block 128, per-head Top-k masks of pooled block scores):

  block index -> WaveAlign reorder (statistics, skip, subspace iteration,
  polar sort, wave buckets, NNZ sort) -> block-sparse attention in the
  reordered, XCD-sliced order with Phase-1 block LSE -> block importance ->
  Top-p selection of the next mask.

Inputs are synthetic (seeded), resident in HBM before timing.  The reported
value is selected-block attention TFLOP/s of the whole step (4*b*b*d FLOP per
selected block pair over the step time).  The roofline object reports the
attention launch alone (HIP events on the launch stream) against the roof its
operational intensity puts it under: the dense bf16 MFMA peak when its FLOP per
compulsory HBM byte exceed the ridge (312.5), else HBM bandwidth (8 TB/s) with
compulsory bytes per second; the CPU baseline is the fp64 oracle timed on a
bounded sample of the same workload.

With ``--workload gsrs75k`` one step is the GSRS search step instead: a full
pass with block LSE, block importance and Top-p(0.9) candidates, the reordered
sparse pass over the candidates with a second Top-p(0.8) restricted to them, and
the reordered sparse pass over that subset; the value counts the selected block
pairs of all three passes.

The reorder uses the adaptive skip with the thresholds of the stored calibration
(``--skip never`` reorders every head).

Usage: python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--workload wan75k]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
RIDGE_FLOP_PER_BYTE = PEAK_BF16_TFLOPS * 1e3 / PEAK_HBM_GBS  # 312.5


def _attn_compulsory_bytes(H: int, lp: int, d: int, b: int, nnz: int, with_g: bool) -> float:
    """Algorithmic HBM bytes of one attention launch: Q, K and V read and O written once
    (4 * H * L_pad * d bf16), the row LSE (fp32), the block LSE G (nnz * b fp32) when it is
    emitted, and the CSR (row_ptr and col_idx, int32)."""
    return (4.0 * H * lp * d * 2 + 4.0 * H * lp + (4.0 * nnz * b if with_g else 0.0)
            + 4.0 * (H * (lp // b) + 1) + 4.0 * nnz)


def _importance_bytes(H: int, lp: int, b: int, nnz: int, mb: int) -> float:
    """Compulsory HBM bytes of one block-importance launch: G read (b floats per CSR
    entry), the row LSE read, W written (one float per entry) and the CSR row pointers."""
    return 4.0 * (nnz * b + H * lp + nnz + H * mb + 1)


def _roofline(flops: float, alg_bytes: float, attn_ms: float, traffic) -> dict:
    """The roofline of the attention launch: its operational intensity (FLOP over
    compulsory bytes) decides the roof.  Above the ridge (312.5 FLOP/B) the bound is the
    bf16 MFMA peak and ``achieved`` counts selected-block FLOP per second; below it, HBM
    bandwidth, and ``achieved`` counts compulsory bytes per second.  ``other`` gives the
    fraction of the other roof for reference."""
    s = attn_ms * 1e-3
    tflops = flops / s / 1e12
    gbs = alg_bytes / s / 1e9
    intensity = flops / alg_bytes
    mfma = {"achieved": round(tflops, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4)}
    hbm = {"achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
           "frac": round(gbs / PEAK_HBM_GBS, 4)}
    main, other, bound = (mfma, hbm, "mfma") if intensity >= RIDGE_FLOP_PER_BYTE else (hbm, mfma, "hbm")
    return {"bound": bound, **main, "traffic": traffic,
            "intensity_flop_per_byte": round(intensity, 1),
            "compulsory_bytes": round(alg_bytes), "other": {"bound": "hbm" if bound == "mfma"
                                                             else "mfma", **other}}
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "cache_aware_query_amd", "csrc", "attention.hip")


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _counter_profile(workload: str):
    """Figures of the committed counter summary of this workload (HBM bytes, L2 hits)
    if it was taken on the current attention kernel source; otherwise an empty dict."""
    path = os.path.join(PROFILES, f"attn_{workload}_traffic.txt")
    if not os.path.exists(path):
        return {}
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                a, b = line.split("=", 1)
                kv[a.strip()] = b.strip()
    if kv.get("kernel_sha256_16") != _kernel_hash():
        return {}
    out = {}
    for key in ("hbm_bytes_per_launch", "hbm_read_bytes_per_launch", "l2_hit_pct"):
        try:
            out[key] = float(kv[key])
        except (KeyError, ValueError):
            pass
    return out


def _time_interleaved(fns: dict, rounds: int, reps: int, label: str = "") -> dict:
    """Median over rounds of the average ms of each fn, the fns taking turns.  The
    order rotates from round to round and every timed window follows one untimed call
    of the same fn, so that no fn always inherits the clock and cache state that one
    particular other fn leaves behind."""
    import statistics

    keys = list(fns)
    times = {k: [] for k in keys}
    for r in range(rounds):
        for k in keys[r % len(keys):] + keys[:r % len(keys)]:
            fns[k]()
            times[k].append(_time_calls(fns[k], reps))
        if label:
            _log(f"{label}: round {r + 1} of {rounds} done")
    return {k: statistics.median(v) for k, v in times.items()}


def _time_calls(fn, reps):
    """Average ms of fn() over reps calls, timed with events on the current stream."""
    import torch

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        fn()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / reps


def cpu_baseline(w, budget_s: float = 12.0):
    """The fp64 oracle on the workload, head by head in runs of 16 query blocks, until
    the budget is spent (a long head is sampled by its leading query blocks)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle

    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    b, d, L = w.block, w.head_dim, w.seq_len
    H, mb = w.mask.shape[0], w.mask.shape[1]
    flops, heads, blocks, t0 = 0.0, 0, 0, time.perf_counter()
    while heads < H and time.perf_counter() - t0 < budget_s:
        h = heads
        qh, kh, vh = (t[h].float().cpu().numpy().astype(np.float64) for t in (w.q, w.k, w.v))
        mh = w.mask[h].cpu().numpy()
        u = 0
        while u < mb and time.perf_counter() - t0 < budget_s:
            u1 = min(mb, u + 16)
            rows = np.arange(u * b, min(L, u1 * b))
            oracle.masked_attention_rows(qh, kh, vh, mh, rows, L, b, w.scale)
            flops += 4.0 * b * b * d * float(mh[u:u1].sum())
            blocks += u1 - u
            u = u1
        heads += 1
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 oracle attention on {blocks} query blocks of {heads} of {H} heads "
                      f"({mb} blocks per head) of the same workload ({dt:.1f} s, BLAS "
                      f"threads={threads}, host cpus={os.cpu_count()})"}


def gsrs_main(args, w, params):
    """The GSRS search step (full pass, candidates, restricted selection, sparse passes)."""
    import torch

    if args.schedule_steps > 0:
        return gsrs_schedule_main(args, w, params)

    from cache_aware_query_amd.pipeline import GsrsSearch

    H, mb = w.mask.shape[0], w.mask.shape[1]
    b, d, L = w.block, w.head_dim, w.seq_len
    dev = w.q.device
    gs = GsrsSearch(H, L, d, b, dev, reorder=params, p1=0.9, p2=0.8)
    _log(f"GSRS search step: H={H} L={L} MB={mb} capacity per pass={gs.dense.cap}")

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        gs.dense.build_index(gs.ones)
        gs.dense.attention(w.q, w.k, w.v)
        if ev is not None:
            ev[1].record()
        gs.dense.select()
        gs.s1.step(w.q, w.k, w.v, gs.mask1, w.x0)
        gs.s2.step(w.q, w.k, w.v, gs.mask2, w.x0)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    pairs = gs.selected_pairs()
    flops = [4.0 * b * b * d * n for n in pairs]
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    dense_ms = sum(a.elapsed_time(b_) for a, b_ in evs) / args.steps
    value = sum(flops) / (ms_per_step * 1e-3) / 1e12
    subset_violations = int((gs.mask2.to(torch.int16) > gs.mask1.to(torch.int16)).sum().item())
    reps = max(3, args.steps // 2)
    detail = {"pairs_full_pass": pairs[0], "pairs_s1_p0.9": pairs[1], "pairs_s2_p0.8": pairs[2],
              "density_s1": round(pairs[1] / (H * mb * mb), 5),
              "density_s2": round(pairs[2] / (H * mb * mb), 5),
              "s2_outside_s1": subset_violations,
              "full_pass_attn_ms": round(dense_ms, 4),
              "skipped_heads_s1": int(gs.s1.skipped.sum().item()),
              "skipped_heads_s2": int(gs.s2.skipped.sum().item())}
    if not args.no_variants:
        detail.update({
            "full_select_ms": round(_time_calls(gs.dense.select, reps), 4),
            "s1_reorder_ms": round(_time_calls(lambda: gs.s1.reorder_rows(w.x0), reps), 4),
            "s1_attn_ms": round(_time_calls(lambda: gs.s1.attention(w.q, w.k, w.v), reps), 4),
            "s1_select_ms": round(_time_calls(gs.s1.select, reps), 4),
            "s2_attn_ms": round(_time_calls(lambda: gs.s2.attention(w.q, w.k, w.v), reps), 4)})
    line = {
        "metric": "selected-block attention TFLOP/s + HBM read GB + L2 hit %, "
                  f"L={L:,} H={H} d={d}",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "heads": H, "seq_len": L, "head_dim": d,
                   "block": b, "p1": 0.9, "p2": 0.8},
        "roofline": _roofline(flops[0], _attn_compulsory_bytes(H, mb * b, d, b, pairs[0], True),
                              dense_ms, None),
        "detail": detail,
    }
    print(json.dumps(line), flush=True)


def gsrs_schedule_main(args, w, params):
    """The GSRS denoising schedule: warmup, four searches, mask reuse in between."""
    import torch

    import synth
    from cache_aware_query_amd.pipeline import GsrsSchedule

    H, mb = w.mask.shape[0], w.mask.shape[1]
    b, d, L = w.block, w.head_dim, w.seq_len
    search = (10, 20, 30, 40)
    gs = GsrsSchedule(H, L, d, b, w.q.device, reorder=params, steps=args.schedule_steps,
                      search_steps=search, thresholds=(0.95, 0.9, 0.85, 0.8))
    # Inputs drift across steps: state k holds from search k on, state 0 before.
    states = synth.drift_states(w, len(search) + 1)

    def inputs(t):
        k = sum(1 for s_ in search if t >= s_)
        q, kk, v = states[k]
        return q, kk, v, w.x0

    def run_once(record):
        evs, sizes = [], {}

        def on_step(t, kind):
            if record:
                e = torch.cuda.Event(enable_timing=True)
                e.record()
                evs.append((t, kind, e))
                if kind == "search":
                    sizes[t] = (gs.search.row_ptr[-1:].clone(), gs.sparse.row_ptr[-1:].clone())
        e0 = torch.cuda.Event(enable_timing=True)
        e0.record()
        gs.run(inputs, on_step)
        return e0, evs, sizes

    _log(f"GSRS schedule: {args.schedule_steps} steps, searches at {search}")
    for _ in range(args.warmup):
        run_once(False)
    torch.cuda.synchronize()
    per_kind = {"warmup": 0.0, "search": 0.0, "reuse": 0.0}
    total_ms, pairs = 0.0, 0
    full_pairs = H * mb * mb
    t0 = time.perf_counter()
    runs = [run_once(True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    densities = {}
    for e0, evs, sizes in runs:
        prev, cur_pairs = e0, full_pairs
        for t, kind, e in evs:
            dt = prev.elapsed_time(e)
            per_kind[kind] += dt
            total_ms += dt
            if kind == "search":
                s1_pairs = int(sizes[t][0].item())
                step_pairs = full_pairs if t == search[0] else s1_pairs
                cur_pairs = int(sizes[t][1].item())
                densities[t] = round(cur_pairs / full_pairs, 4)
            else:
                step_pairs = full_pairs if kind == "warmup" else cur_pairs
            pairs += step_pairs
            prev = e
    # Diagnostics outside the timed runs (GSRS §3 attention recall, Fig. 2): with the
    # last step's inputs, the share of the full attention that the candidate set S1
    # and the final mask keep.
    import cache_aware_query_amd as caq

    q, kk, v, _ = inputs(args.schedule_steps - 1)
    gs.full.attention(q, kk, v)
    gs.full.importance()
    recall = {name: round(float(caq.mask_recall(gs.full.w, gs.full.row_ptr, gs.full.col_idx,
                                                m).mean().item()), 4)
              for name, m in (("candidate_set_s1", gs.s1), ("final_mask", gs.mask))}
    # Row entropy and mean attention distance along the schedule (GSRS §4, Fig. 1), from
    # one more run in which every attention pass also writes both (untimed).
    diag = None
    if args.diagnostics:
        gd = GsrsSchedule(H, L, d, b, w.q.device, reorder=params, steps=args.schedule_steps,
                          search_steps=search, thresholds=(0.95, 0.9, 0.85, 0.8),
                          diagnostics=True)
        gd.run(inputs)
        diag = {str(t): {"kind": kind, "mean_entropy": round(float(e.item()), 4),
                         "mean_distance_tokens": round(float(dist.item()), 1)}
                for t, kind, e, dist in gd.trace
                if kind == "search" or t in (0, search[0] - 1, args.schedule_steps - 1)}
        del gd
    n = args.steps
    ms_per_run = total_ms / n
    flops = 4.0 * b * b * d * pairs / n
    value = flops / (ms_per_run * 1e-3) / 1e12
    line = {
        "metric": "selected-block attention TFLOP/s + HBM read GB + L2 hit %, "
                  f"L={L:,} H={H} d={d}",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": n,
        "warmup": args.warmup, "ms_per_step": round(ms_per_run, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "gsrs75k-schedule", "heads": H, "seq_len": L, "head_dim": d,
                   "block": b, "denoising_steps": args.schedule_steps,
                   "search_steps": list(search), "p": [0.95, 0.9, 0.85, 0.8]},
        "detail": {"ms_by_kind_per_run": {k: round(v / n, 3) for k, v in per_kind.items()},
                   "steps_by_kind": {k: gs.kinds.count(k) for k in per_kind},
                   "mask_density_after_search": densities,
                   "recall_at_last_step": recall,
                   "diagnostics_by_step": diag,
                   "selected_tflop_per_run": round(flops / 1e12, 3),
                   "wall_ms_per_run": round(wall_ms, 3)},
    }
    print(json.dumps(line), flush=True)


def _skip_report(hp, w, params) -> dict:
    """Per-head skip decision and the statistic that took it (outside the timed region).

    The rule is run once more on the device with every head's statistics reported,
    whatever the host-side bound decided: s = size (K/V bytes), w = work (selected
    FLOP of the heaviest head: the work case is decided per call), j = similarity
    (adjacent-row Jaccard), r = reordered."""
    import numpy as np

    import cache_aware_query_amd as caq

    ro = caq.reorder_rows(hp.index(), w.x0, w.block, w.head_dim, params)
    st = ro.stats.cpu().double().numpy()
    skipped = ro.skipped.cpu().numpy().astype(bool)
    by = []
    call_flops = float(st[:, 3].max())
    for h in range(st.shape[0]):
        if not st[h, 2] > params.ws_min_bytes:
            by.append("s")
        elif not call_flops >= params.flops_min:
            by.append("w")
        elif not st[h, 4] < params.jaccard_max:
            by.append("j")
        else:
            by.append("r")
        assert (by[-1] != "r") == skipped[h]
    return {"thresholds": {"ws_min_bytes": params.ws_min_bytes, "flops_min": params.flops_min,
                           "jaccard_max": params.jaccard_max},
            "decided_by": "".join(by),
            "legend": "s size, w work, j similarity, r reordered",
            "per_head_gflop": [round(float(x) / 1e9, 2) for x in st[:, 3]],
            "per_head_jaccard": [None if np.isnan(x) else round(float(x), 4) for x in st[:, 4]],
            "host_bound_skipped_all": bool(hp.host_skip)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan75k")
    ap.add_argument("--iters", type=int, default=5,
                    help="subspace iterations T of the reorder (the pages use 5..15)")
    ap.add_argument("--skip", choices=("adaptive", "never", "always"), default="adaptive",
                    help="reorder skip rule: the stored calibration, reorder every head, or "
                         "keep every head in its original order")
    ap.add_argument("--schedule-steps", type=int, default=0,
                    help="with --workload gsrs75k: run the whole GSRS denoising schedule of this "
                         "many steps (searches at 10, 20, 30, 40) per bench step")
    ap.add_argument("--diagnostics", action="store_true",
                    help="with --schedule-steps: also report the mean row entropy and mean "
                         "attention distance of the search steps (one extra, untimed run)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="before the steps, run three plain device copies of this many MiB "
                         "(a known-size reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads would shard across GPUs with no exchange); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import cache_aware_query_amd as caq
    import synth
    from cache_aware_query_amd.pipeline import HotPath

    dev = torch.device("cuda:0")
    _log(f"generating workload {args.workload}")
    w = synth.make_workload(args.workload, device=dev)
    H, mb = w.mask.shape[0], w.mask.shape[1]
    b, d, L = w.block, w.head_dim, w.seq_len
    nnz = int(w.mask.sum())
    flops = 4.0 * b * b * d * nnz
    n_xcd, cus, wave = caq.schedule_info(0, d)
    if args.skip == "adaptive":
        params = caq.ReorderParams.calibrated(wave=wave, n_slices=n_xcd, iters=args.iters)
    else:
        params = caq.ReorderParams(wave=wave, n_slices=n_xcd, iters=args.iters,
                                   skip_mode=(caq.WA_SKIP_NEVER if args.skip == "never"
                                              else caq.WA_SKIP_ALWAYS))
    if args.workload == "gsrs75k":
        return gsrs_main(args, w, params)
    # With the adaptive skip the attention follows the skip flags on the device: the
    # default path (WA_SCHED_DEFAULT: all heads at once for small heads, else
    # XCD-sliced in the original order) when every head kept its order, XCD-sliced in
    # the reordered order otherwise.  A forced skip rule keeps the XCD-sliced schedule, so that "always"
    # measures the identity order under the same schedule as the reordered one.
    main_sched = caq.WA_SCHED_AUTO if args.skip == "adaptive" else caq.WA_SCHED_XCD_SLICED
    # The buffers are sized for this workload's masks: the CSR capacity is its total
    # selected entries and the per-head capacity its largest head's, allocation bounds a
    # caller knows from how its masks are made (they bound the skip rules on the host).
    head_cap = int(w.mask.sum(dim=(1, 2)).max())
    hp = HotPath(H, L, d, b, dev, capacity=nnz, reorder=params, schedule=main_sched, gsrs_p=0.9,
                 head_capacity=head_cap)
    _log(f"H={H} L={L} d={d} b={b} MB={mb} nnz={nnz} density={nnz / (H * mb * mb):.4f} "
         f"xcd={n_xcd} cus/xcd={cus} wave={wave} T={args.iters} csc={hp.with_csc}")

    if args.copy_calib_mb > 0:
        n = args.copy_calib_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        _log(f"copy calibration: 3 copies of {n} bytes")
        del src, dst

    def step(ev=None):
        hp.build_index(w.mask)
        hp.reorder_rows(w.x0)
        if ev is not None:
            ev[0].record()
        hp.attention(w.q, w.k, w.v)
        if ev is not None:
            ev[1].record()
        hp.select()

    # Caches are flushed before every timed step: a 1 GiB buffer (four times the
    # Infinity Cache) is read and written, so no step finds the last one's data in L2
    # or the Infinity Cache.  Back-to-back ("warm") steps are timed after, for context.
    flush_buf = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)

    def timed_steps(cold):
        ev_step = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
        ev_attn = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            if cold:
                flush_buf.add_(1)
            ev_step[i][0].record()
            step(ev_attn[i])
            ev_step[i][1].record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / args.steps
        step_ms = [a.elapsed_time(b_) for a, b_ in ev_step]
        attn_ms_ = [a.elapsed_time(b_) for a, b_ in ev_attn]
        return statistics.median(step_ms), statistics.median(attn_ms_), wall

    for _ in range(args.warmup):
        step()
    _log(f"{args.warmup} warmup steps done")
    ms_per_step, attn_ms, wall_ms = timed_steps(cold=True)
    _log(f"{args.steps} timed steps done: {ms_per_step:.3f} ms per step")
    warm_step_ms, warm_attn_ms, _ = timed_steps(cold=False)
    del flush_buf
    value = flops / (ms_per_step * 1e-3) / 1e12
    prof = _counter_profile(args.workload)

    detail = {"attn_ms": round(attn_ms, 4), "nnz_pairs": nnz,
              "timing": "median of the timed steps, caches flushed (1 GiB streamed) before "
                        "each; warm = back to back",
              "wall_ms_per_step_incl_flush": round(wall_ms, 4),
              "warm_ms_per_step": round(warm_step_ms, 4), "warm_attn_ms": round(warm_attn_ms, 4),
              "selected_tflop": round(flops / 1e12, 4),
              "skipped_heads": int(hp.skipped.sum().item()),
              "skip_per_head": "".join(str(int(x)) for x in hp.skipped.cpu().tolist()),
              "skip_rule": args.skip,
              "head_capacity": head_cap,
              "reorder_iters": args.iters,
              "hbm_read_gb_per_launch": (round(prof["hbm_read_bytes_per_launch"] / 1e9, 3)
                                         if "hbm_read_bytes_per_launch" in prof else None),
              "l2_hit_pct": prof.get("l2_hit_pct")}
    if params.skip_mode == caq.WA_SKIP_ADAPTIVE:
        detail["skip_decisions"] = _skip_report(hp, w, params)
    if not args.no_variants:
        _log("stage times and variants")
        reps = max(3, args.steps // 2)
        # Stage times of the reordered step.
        t_index = _time_calls(lambda: hp.build_index(w.mask), reps)
        t_reorder = _time_calls(lambda: hp.reorder_rows(w.x0), reps)
        t_select = _time_calls(hp.select, reps)
        t_importance = _time_calls(hp.importance, reps)
        # The same kernel without reordering (identity order; its index has no
        # transposed lists), and the stage ablation (WaveAlign Fig. 12, every head
        # reordered), each with buffers of its own.
        hp_id = HotPath(H, L, d, b, dev, capacity=nnz, reorder=None,
                        schedule=caq.WA_SCHED_XCD_SLICED, gsrs_p=0.9)

        def share_g(path):
            # The comparison paths are only timed: they write their block LSE (G, one
            # float per entry and query row) into one buffer, so that a long workload
            # does not hold a copy per path.
            path.g = hp_id.g
            return path
        hp_id.build_index(w.mask)
        t_index_id = _time_calls(lambda: hp_id.build_index(w.mask), reps)
        ablation = {}
        for name, s1, s2 in (("stage1_only", True, False), ("stage2_only", False, True),
                             ("both_no_skip", True, True)):
            pa = caq.ReorderParams(wave=wave, n_slices=n_xcd, iters=args.iters, stage1=s1,
                                   stage2=s2, skip_mode=caq.WA_SKIP_NEVER)
            hpa = share_g(HotPath(H, L, d, b, dev, capacity=nnz, reorder=pa,
                                  schedule=caq.WA_SCHED_XCD_SLICED, gsrs_p=0.9))
            hpa.build_index(w.mask)
            hpa.reorder_rows(w.x0)
            ablation[name] = hpa
        # The MinHash comparator of WaveAlign Table II (min-wise hashing of each row's
        # K/V block set, rows by signature, then the same Stage 2), every head.
        hp_mh = share_g(HotPath(H, L, d, b, dev, capacity=nnz,
                                reorder=caq.ReorderParams(wave=wave, n_slices=n_xcd,
                                                          skip_mode=caq.WA_SKIP_NEVER),
                                schedule=caq.WA_SCHED_XCD_SLICED, gsrs_p=0.9))
        hp_mh.build_index(w.mask)
        mh_a, mh_b = synth.minhash_params(2)

        def minhash():
            caq.minhash_order(hp_mh.index(), mh_a, mh_b, wave, n_xcd, True,
                              out=(hp_mh.perm, hp_mh.inv_perm))
        minhash()
        t_minhash = _time_calls(minhash, reps)
        # The banded LSH comparator of the same table (four bands of two MinHash
        # values; each row joins the lowest row it shares a bucket with), every head.
        hp_lsh = share_g(HotPath(H, L, d, b, dev, capacity=nnz,
                                 reorder=caq.ReorderParams(wave=wave, n_slices=n_xcd,
                                                           skip_mode=caq.WA_SKIP_NEVER),
                                 schedule=caq.WA_SCHED_XCD_SLICED, gsrs_p=0.9))
        hp_lsh.build_index(w.mask)
        lsh_a, lsh_b = synth.minhash_params(8, seed=synth.workloads.BASE_SEED + 100)

        def lsh():
            caq.lsh_order(hp_lsh.index(), lsh_a, lsh_b, wave, n_xcd, True,
                          out=(hp_lsh.perm, hp_lsh.inv_perm))
        lsh()
        t_lsh = _time_calls(lsh, reps)
        # The explicit form of applying the permutation ([WA] §V: gather the Q blocks
        # into execution order before the kernel, scatter O back after it), which the
        # fused kernel avoids; both copies are HBM-bound.
        lib = caq.load_library()
        q_x, o_x = torch.empty_like(w.q), torch.empty_like(hp.o)
        blk_bytes = b * d * w.q.element_size()

        def explicit_permute():
            caq._check(lib.wa_gather_blocks(caq._ptr(w.q), caq._ptr(q_x), caq._ptr(hp.perm), H,
                                            mb, blk_bytes, caq._stream(dev)), "wa_gather_blocks")
            caq._check(lib.wa_scatter_blocks(caq._ptr(hp.o), caq._ptr(o_x), caq._ptr(hp.perm), H,
                                             mb, blk_bytes, caq._stream(dev)),
                       "wa_scatter_blocks")
        explicit_permute()
        t_perm = _time_calls(explicit_permute, reps)
        perm_bytes = 2 * 2 * H * mb * blk_bytes  # Q and O, each read and written once
        del q_x, o_x
        ablation["minhash_order"] = hp_mh
        ablation["lsh_order"] = hp_lsh
        _log("comparator orders built and timed")

        def with_schedule(path, sched, permuted=True):
            def run():
                path.schedule = sched
                path.attention(w.q, w.k, w.v, permuted=permuted)
            return run

        # Attention variants timed in interleaved rounds (medians), so that clock
        # drift during the run does not favour whichever variant runs first.  The
        # head-interleaved order is the concurrent-head execution of WaveAlign
        # §VI-B ("Original" on the A40).  The unreordered variants run on the main
        # path's own buffers (original order, no permutation read), so that buffer
        # placement does not separate them from the reordered one.
        caq.attn_schedule_select(hp.skipped, hp.workspace)  # AUTO follows hp's skip flags
        variants = {
            "reordered_auto": with_schedule(hp, caq.WA_SCHED_AUTO),
            "reordered_xcd": with_schedule(hp, caq.WA_SCHED_XCD_SLICED),
            "identity_xcd": with_schedule(hp, caq.WA_SCHED_XCD_SLICED, False),
            "natural_order": with_schedule(hp, caq.WA_SCHED_NATURAL, False),
            "heads_interleaved": with_schedule(hp, caq.WA_SCHED_HEADS_INTERLEAVED, False),
        }
        for name, hpa in ablation.items():
            variants[name] = with_schedule(hpa, caq.WA_SCHED_XCD_SLICED)
        t = _time_interleaved(variants, rounds=5, reps=max(2, reps // 2), label="attention variants")
        hp.schedule = main_sched

        # End to end, reorder cost included: each chain (index, order, attention) timed
        # as one unit, the chains taking turns, medians over the rounds.
        def chain(path, order, sched, permuted=True):
            def run():
                path.build_index(w.mask, transposed=permuted)
                order()
                path.schedule = sched
                path.attention(w.q, w.k, w.v, permuted=permuted)
            return run
        chains = {
            "reordered": chain(hp, lambda: hp.reorder_rows(w.x0), main_sched),
            "minhash": chain(hp_mh, minhash, caq.WA_SCHED_XCD_SLICED),
            "lsh": chain(hp_lsh, lsh, caq.WA_SCHED_XCD_SLICED),
            "unreordered_identity_xcd": chain(hp, lambda: None, caq.WA_SCHED_XCD_SLICED, False),
            "unreordered_natural": chain(hp, lambda: None, caq.WA_SCHED_NATURAL, False),
            "unreordered_heads_interleaved": chain(hp, lambda: None,
                                                   caq.WA_SCHED_HEADS_INTERLEAVED, False),
        }
        # Each chain is captured once as a graph and replayed, so the comparison times
        # the GPU work of the chains, not the host's launch overhead (which dominates
        # the smallest workloads); a chain that cannot be captured runs eagerly.
        graphs, chain_mode = {}, "graph replay"
        for name, fn in chains.items():
            fn()
            torch.cuda.synchronize()
            try:
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr, capture_error_mode="relaxed"):
                    fn()
                gr.replay()
                torch.cuda.synchronize()
                graphs[name] = gr.replay
            except RuntimeError as exc:
                _log(f"chain {name} not captured ({exc}); timed eagerly")
                graphs[name] = fn
                chain_mode = "graph replay where captured, else eager"
        # Each timing window spans at least about 10 ms of replays, so that the
        # shortest chains (tens of microseconds) are not timed at event resolution.
        est = max(_time_calls(fn, 2) for fn in graphs.values())
        chain_reps = int(min(400, max(2, reps // 2, -(-10.0 // max(est, 1e-3)))))
        te = _time_interleaved(graphs, rounds=9, reps=chain_reps, label="end-to-end chains")
        detail["e2e_timing_reps"] = chain_reps
        del graphs
        hp.schedule = main_sched
        hp.build_index(w.mask)
        hp.reorder_rows(w.x0)
        # Locality proxies of the orders on the host (WaveAlign §IV-B Problem (1) per
        # wave, distinct K/V blocks per XCD wave, an LRU model of each XCD's L2).
        from cache_aware_query_amd import locality
        mask_h = w.mask.cpu().numpy()
        ident = np.tile(np.arange(mb, dtype=np.int64), (H, 1))
        lru_heads = range(min(H, 8))
        orders = {"wavealign": hp.perm.cpu().numpy(), "identity": ident,
                  "minhash": hp_mh.perm.cpu().numpy(), "lsh": hp_lsh.perm.cpu().numpy()}
        detail["locality_proxies"] = {}
        for name, pm in orders.items():
            detail["locality_proxies"][name] = {
                "wave_objective": locality.wave_objective(mask_h, pm, n_xcd, wave),
                "distinct_kv_per_wave": round(locality.distinct_kv_per_wave(
                    mask_h, pm, n_xcd, wave), 1),
                "lru_l2_hit_model": round(locality.lru_l2_model(
                    mask_h, pm, n_xcd, wave, 64, heads=lru_heads), 4)}
            _log(f"locality proxies of the {name} order done")
        detail["locality_proxies"]["lru_model_heads"] = len(lru_heads)
        del mask_h
        # Speedup gap (WaveAlign §III-A, Fig. 2): the ideal speedup 1/rho of the sparse
        # kernel over the same kernel on an all-ones mask, against the measured one
        # (both without G, the sparse one in its reordered order).
        dense_pairs = H * mb * mb
        if 4.0 * b * b * d * dense_pairs <= 150e12:
            hp_dense = HotPath(H, L, d, b, dev, capacity=dense_pairs, reorder=None,
                               schedule=caq.WA_SCHED_XCD_SLICED, gsrs_p=None)
            hp_dense.build_index(torch.ones(H, mb, mb, dtype=torch.uint8, device=dev))
            t_dense = _time_calls(lambda: hp_dense.attention(w.q, w.k, w.v), 2)
            t_sparse = _time_calls(lambda: hp.attention_plain(w.q, w.k, w.v), reps)
            rho = nnz / dense_pairs
            s_act = t_dense / t_sparse
            detail["speedup_gap"] = {"dense_attn_ms": round(t_dense, 3),
                                     "sparse_attn_ms_no_g": round(t_sparse, 4),
                                     "density": round(rho, 5),
                                     "ideal_speedup": round(1.0 / rho, 3),
                                     "actual_speedup": round(s_act, 3),
                                     "gap": round((1.0 / rho) / s_act, 3)}
            del hp_dense
        del hp_id, ablation
        e2e_reord = te["reordered"]
        best_plain = min((k for k in te if k.startswith("unreordered_")), key=lambda k: te[k])
        e2e_plain = te[best_plain]
        detail.update({"index_ms": round(t_index, 4),
                       "reorder_ms": round(t_reorder, 4),
                       "gsrs_select_ms": round(t_select, 4),
                       "index_ms_without_reorder": round(t_index_id, 4)})
        imp_gbs = _importance_bytes(H, mb * b, b, nnz, mb) / (t_importance * 1e-3) / 1e9
        detail["block_importance"] = {"ms": round(t_importance, 4), "bound": "hbm",
                                      "achieved_gb_per_s": round(imp_gbs, 1),
                                      "peak_gb_per_s": PEAK_HBM_GBS,
                                      "frac": round(imp_gbs / PEAK_HBM_GBS, 4)}
        detail.update({f"attn_ms_{k}": round(v, 4) for k, v in t.items()})
        detail["minhash_order_ms"] = round(t_minhash, 4)
        detail["lsh_order_ms"] = round(t_lsh, 4)
        detail["e2e_ms_lsh"] = round(te["lsh"], 4)
        detail["explicit_permute_ms"] = round(t_perm, 4)
        detail["explicit_permute_gb_per_s"] = round(perm_bytes / (t_perm * 1e-3) / 1e9, 1)
        detail["e2e_ms_minhash"] = round(te["minhash"], 4)
        detail.update({"e2e_ms_reordered": round(e2e_reord, 4),
                       "e2e_ms_unreordered_best": round(e2e_plain, 4),
                       "e2e_unreordered_best_is": best_plain,
                       "e2e_ms_by_chain": {k: round(v, 4) for k, v in te.items()},
                       "e2e_timing": chain_mode,
                       "reorder_speedup_incl_overhead": round(e2e_plain / e2e_reord, 4),
                       "host_skipped_reorder": bool(hp.host_skip)})

    line = {
        "metric": "selected-block attention TFLOP/s + HBM read GB + L2 hit %, "
                  f"L={L:,} H={H} d={d}",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "heads": H, "seq_len": L, "head_dim": d,
                   "block": b, "density": round(nnz / (H * mb * mb), 5)},
        "roofline": _roofline(flops, _attn_compulsory_bytes(H, hp.lp, d, b, nnz, True), attn_ms,
                              prof.get("hbm_bytes_per_launch")),
        "detail": detail,
    }
    if not args.no_cpu_baseline:
        _log("timing the oracle on a bounded sample")
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
