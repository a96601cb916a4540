"""Host logic of the skip calibration: the threshold fit and the stored profile."""

import json
import os

import cache_aware_query_amd as caq
from cache_aware_query_amd import calibrate


def _pt(ws, fl, jac, gain):
    return {"ws_bytes": ws, "flops_per_head": fl, "jaccard": jac, "gain_ms": gain,
            "reorder_wins": gain > 0}


def test_fit_separates_by_work():
    # Reordering pays exactly for the heads with the most work.
    pts = [_pt(1e7 * s, 1e11 * f, 0.3, (0.2 if f >= 8 else -0.1))
           for s in (1, 2, 4) for f in (1, 2, 4, 8, 16)]
    thr = calibrate.fit(pts)
    assert thr["points_correct"] == thr["points"] == len(pts)
    for p in pts:
        dec = (p["ws_bytes"] > thr["ws_min_bytes"] and p["flops_per_head"] >= thr["flops_min"]
               and p["jaccard"] < thr["jaccard_max"])
        assert dec == p["reorder_wins"]
    assert 4e11 < thr["flops_min"] <= 8e11


def test_fit_separates_by_similarity_and_size():
    pts = [_pt(ws, 1e12, jac, 0.1 if (ws > 3e7 and jac < 0.5) else -0.05)
           for ws in (1e7, 2e7, 4e7, 8e7) for jac in (0.2, 0.4, 0.6, 0.8)]
    thr = calibrate.fit(pts)
    assert thr["points_correct"] == len(pts)
    assert 2e7 <= thr["ws_min_bytes"] < 4e7
    assert 0.4 < thr["jaccard_max"] <= 0.6


def test_fit_never_reorders_when_it_never_pays():
    pts = [_pt(1e7 * s, 1e11 * s, 0.3, -0.01 * s) for s in range(1, 6)]
    thr = calibrate.fit(pts)
    assert thr["points_correct"] == len(pts)
    assert not any(p["ws_bytes"] > thr["ws_min_bytes"] and p["flops_per_head"] >= thr["flops_min"]
                   and p["jaccard"] < thr["jaccard_max"] for p in pts)


def test_stored_profile_loads():
    path = os.path.join(os.path.dirname(caq.__file__), "calib_mi355x.json")
    with open(path) as f:
        c = json.load(f)
    assert c["points"] == len(c["sweep"]) and c["points_correct"] <= c["points"]
    p = caq.ReorderParams.calibrated()
    assert p.skip_mode == caq.WA_SKIP_ADAPTIVE
    assert p.ws_min_bytes == c["ws_min_bytes"] and p.flops_min == c["flops_min"]
    assert 0.0 <= p.jaccard_max <= 1.0 + 1e-6
    assert caq.ReorderParams.calibrated(iters=3).iters == 3


def test_fit_weighs_wrong_points_by_relative_time_lost():
    # Two points cannot both be decided right by a work threshold: a small loss at more
    # work than a large win.  The fit keeps the large win and names the inert cases.
    pts = [_pt(1e7, 1e11, 0.3, -0.5), _pt(1e7, 2e11, 0.3, 5.0), _pt(1e7, 4e11, 0.3, -0.01)]
    for p, t in zip(pts, (10.0, 50.0, 100.0)):
        p["e2e_reordered_ms"] = t - p["gain_ms"] / 2
        p["e2e_unreordered_ms"] = t + p["gain_ms"] / 2
    thr = calibrate.fit(pts)
    assert 1e11 < thr["flops_min"] <= 2e11
    assert thr["points_correct"] == 2
    assert set(thr["inert"]) == {"ws_min_bytes", "jaccard_max"}
    assert calibrate.decide(pts[0], thr) == "work" and calibrate.decide(pts[1], thr) == "reorder"


def test_stored_profile_names_its_deciding_cases():
    path = os.path.join(os.path.dirname(caq.__file__), "calib_mi355x.json")
    with open(path) as f:
        c = json.load(f)
    fams = {p["family"] for p in c["sweep"]}
    assert {"topk-raster", "topk-hilbert", "neighbour", "random"} <= fams
    for p in c["sweep"]:
        assert p["decided_by"] == calibrate.decide(p, c)
