"""Host logic of bench.py: the roofline object, the compulsory bytes of a launch, the
counter summaries matched to the kernel source, and the one-GPU guard."""

import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_compulsory_bytes_by_hand():
    # H = 2, L_pad = 256, d = 64, b = 128: Q, K, V, O 4 * 2 * 256 * 64 * 2 B; LSE 2 * 256 * 4 B;
    # G 5 pairs * 128 rows * 4 B; row_ptr (2 * 2 + 1) * 4 B; col_idx 5 * 4 B
    got = bench._attn_compulsory_bytes(2, 256, 64, 128, 5, True)
    assert got == 262144 + 2048 + 2560 + 20 + 20
    assert bench._attn_compulsory_bytes(2, 256, 64, 128, 5, False) == 262144 + 2048 + 20 + 20


def test_roofline_picks_the_roof_by_intensity():
    # above the ridge (312.5 FLOP/B): the MFMA roof, achieved in FLOP/s
    r = bench._roofline(flops=2.5e13, alg_bytes=1e10, attn_ms=20.0, traffic=None)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert r["achieved"] == pytest.approx(1250.0) and r["frac"] == pytest.approx(0.5)
    assert r["other"]["bound"] == "hbm" and r["other"]["achieved"] == pytest.approx(500.0)
    assert r["intensity_flop_per_byte"] == pytest.approx(2500.0)
    # below it: the HBM roof, achieved in compulsory bytes per second
    r = bench._roofline(flops=1e12, alg_bytes=1e10, attn_ms=2.0, traffic=123.0)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(5000.0) and r["frac"] == pytest.approx(0.625)
    assert r["traffic"] == 123.0 and r["other"]["bound"] == "mfma"


def test_counter_profile_follows_the_kernel_source(tmp_path, monkeypatch):
    src = tmp_path / "attention.hip"
    src.write_text("// a kernel\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()[:16]
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "attn_demo_traffic.txt").write_text(
        "# comment = ignored\n"
        f"kernel_sha256_16 = {sha}\n"
        "hbm_bytes_per_launch = 1000\nhbm_read_bytes_per_launch = 900\nl2_hit_pct = 55.5\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    assert bench._counter_profile("demo") == {"hbm_bytes_per_launch": 1000.0,
                                              "hbm_read_bytes_per_launch": 900.0,
                                              "l2_hit_pct": 55.5}
    assert bench._counter_profile("absent") == {}
    src.write_text("// the kernel changed\n")   # stale counters are not reported
    assert bench._counter_profile("demo") == {}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_importance_bytes_by_hand():
    # H = 2, L_pad = 256, b = 128, nnz = 5, MB = 2: G 5 * 128 * 4 B, LSE 2 * 256 * 4 B,
    # W 5 * 4 B, row_ptr (2 * 2 + 1) * 4 B
    assert bench._importance_bytes(2, 256, 128, 5, 2) == 2560 + 2048 + 20 + 20
