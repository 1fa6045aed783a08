"""Host logic of bench.py (no GPU): per-kernel rates, the roofline entry and
its counter-derived fields, and the one-GPU guard."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_kernel_entry_rates_and_fractions():
    f = bench._kernel_entry(1000.0, 2.5e12, "flop")          # 2.5e12 FLOP in 1 ms
    assert f["tflops"] == pytest.approx(2500.0)
    assert f["frac_peak"] == pytest.approx(2500.0 / bench.PEAK_FP8_TFLOPS)
    b = bench._kernel_entry(50.0, 2.0e8, "bytes")            # 200 MB in 50 us
    assert b["gbs"] == pytest.approx(4000.0)
    assert b["frac_peak"] == pytest.approx(4000.0 / bench.PEAK_HBM_GBS)


def _with_profile(tmp_path, monkeypatch, source_hash):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "hbm_traffic.json").write_text(json.dumps({
        "source_hash": source_hash,
        "kernels": {"gemm Wgrad": 2.4e9, "quant X": 2.4e8},
        "clock_ghz": {"gemm Wgrad": 2.0},
    }))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda: "abc")


def test_roofline_takes_counters_only_for_the_current_kernels(tmp_path, monkeypatch):
    _with_profile(tmp_path, monkeypatch, "abc")
    k = bench._kernel_entry(1200.0, 2.1e12, "flop")
    r = bench._roofline("gemm Wgrad", k)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == bench.PEAK_FP8_TFLOPS
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-4)
    assert r["traffic"] == 2.4e9
    # the published peak scaled from 2.4 GHz to the measured clock
    assert r["frac_at_clock"] == pytest.approx(k["tflops"] / (bench.PEAK_FP8_TFLOPS * 2.0 / 2.4), abs=1e-4)
    q = bench._roofline("quant X", bench._kernel_entry(50.0, 2.4e8, "bytes"))
    assert q["bound"] == "hbm" and q["unit"] == "GB/s" and q["traffic"] == 2.4e8 and "frac_at_clock" not in q


def test_roofline_drops_counters_of_other_kernel_sources(tmp_path, monkeypatch):
    _with_profile(tmp_path, monkeypatch, "stale")
    r = bench._roofline("gemm Wgrad", bench._kernel_entry(1200.0, 2.1e12, "flop"))
    assert r["traffic"] is None and "clock_ghz" not in r


def test_source_hash_covers_every_kernel_source():
    # a kernel edit must invalidate the stored counters: every device source is hashed
    csrc = os.path.join(ROOT, "precision_fp8_quant_amd", "csrc")
    device = {f for f in os.listdir(csrc) if f.endswith((".hip", ".h")) and f != "fp8q_launch.h"}
    import inspect
    src = inspect.getsource(bench.source_hash)
    assert all(f in src for f in device), device


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
