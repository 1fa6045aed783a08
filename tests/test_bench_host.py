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


def test_cpu_baseline_records_the_parity_of_every_slice():
    """The CPU leg compares the timed GPU run's outputs with the oracle on each slice it times: quantizers bit for
    bit, GEMMs by relative Frobenius error against the stated bound.  Small synthetic slices (the leg takes its
    shapes from them); the "GPU" outputs are the oracle's own, with one planted byte and one planted GEMM error."""
    import numpy as np
    from oracle import gemm as og, quant as oq
    from workloads import bf16_bits_as_f32, to_bf16_bits
    rng = np.random.default_rng(7)
    b16 = lambda shape, sigma: to_bf16_bits((rng.standard_normal(shape) * sigma).astype(np.float32))
    host = {"x": b16((256, 1024), 1.0), "wt": b16((512, 1024), 0.02), "wt_in": b16((512, 256), 0.02),
            "dy": b16((256, 512), 1e-3), "dy_t": b16((256, 256), 1e-3), "x_t": b16((256, 256), 1.0),
            "mx": b16((512, 1024), 1.0), "mw": b16((4, 512, 1024), 0.02),
            "counts": np.array([100, 128, 50, 128]), "padded": np.array([128, 128, 128, 128])}
    f = bf16_bits_as_f32
    x = f(host["x"])
    gpu = {}
    gpu["qx"], gpu["sx"] = oq.quant_1x128(x)
    gpu["pow2_q"], gpu["pow2_s"] = oq.quant_1x128(x, oq.MODE_POW2)
    gpu["qxt"], gpu["sxt"] = oq.quant_128x1(x)
    gpu["qw"], gpu["sw"] = oq.quant_128x128(f(host["wt"]))
    qa, sa = gpu["qx"], gpu["sx"]
    gpu["y"] = og.round_output(og.gemm_ref(qa, sa, gpu["qw"], gpu["sw"], og.FPROP), "bf16")
    qa, sa = oq.quant_1x128(f(host["dy"]))
    qb, sb = oq.quant_128x128(np.ascontiguousarray(f(host["wt_in"]).T))
    gpu["dx"] = og.round_output(og.gemm_ref(qa, sa, qb, sb, og.DGRAD), "bf16")
    qa, sa = oq.quant_128x1(f(host["dy_t"]))
    qb, sb = oq.quant_128x1(f(host["x_t"]))
    gpu["dw"] = og.round_output(og.gemm_ref(qa, sa, qb, sb, og.WGRAD), "f32")
    qa, sa = oq.quant_1x128(f(host["mx"]))
    qbs = [oq.quant_128x128(f(w)) for w in host["mw"]]
    gpu["my"] = og.round_output(og.grouped_ref(qa, sa, np.stack([q for q, _ in qbs]), np.stack([s for _, s in qbs]),
                                               np.arange(4, dtype=np.int32)), "bf16")
    from workloads import tiny_fprop
    t = tiny_fprop()
    gpu["tiny_qa"], gpu["tiny_sa"] = oq.quant_1x128(t["a"])
    gpu["tiny_qb"], gpu["tiny_sb"] = oq.quant_128x128(t["bt"])
    gpu["tiny_c"] = og.round_output(og.gemm_ref(gpu["tiny_qa"], gpu["tiny_sa"], gpu["tiny_qb"], gpu["tiny_sb"],
                                                og.FPROP), "f32")
    gpu["qxt"] = gpu["qxt"].copy()
    gpu["qxt"][5, 7] ^= 1                                  # one planted code byte
    gpu["dx"] = gpu["dx"] * 1.01                           # a planted 1% GEMM error
    lines = {l["kernel"]: l for l in bench.cpu_baseline(host, gpu)["per_config"]}
    assert lines["quant_1x128 X (max-abs)"]["parity"] == "bit-exact"
    assert lines["quant_1x128 X (pow2)"]["parity"] == "bit-exact"
    assert lines["quant_128x128 W (max-abs)"]["parity"] == "bit-exact"
    assert lines["quant_128x1 X (max-abs)"]["parity"] == "MISMATCH: 1 bytes differ"
    for k in ("gemm Fprop", "gemm Wgrad", "gemm grouped MoE"):
        assert lines[k]["parity"]["ok"] and lines[k]["parity"]["rel_frobenius"] == 0.0, k
    # against the unrounded product: the output dtype's own rounding (BF16 about 1.7e-3, FP32 about 3e-8)
    assert 1e-3 < lines["gemm Fprop"]["parity"]["rel_frobenius_raw"] < 3e-3
    assert 0 < lines["gemm Wgrad"]["parity"]["rel_frobenius_raw"] < 1e-7
    assert not lines["gemm Dgrad"]["parity"]["ok"]
    assert lines["gemm Dgrad"]["parity"]["rel_frobenius"] > lines["gemm Dgrad"]["parity"]["bound"]
    tiny = lines["quant 1x128 + 128x128 + Fprop (int64)"]["parity"]
    assert tiny["codes_and_scales"] == "bit-exact" and tiny["ok"] and tiny["rel_frobenius"] == 0.0


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    """The profiles are keyed to the kernels' code: a comment or blank-space edit keeps the hash, a code edit
    changes it."""
    import shutil
    src = os.path.join(ROOT, "precision_fp8_quant_amd", "csrc")
    dst = tmp_path / "precision_fp8_quant_amd" / "csrc"
    dst.mkdir(parents=True)
    for f in ("quant.hip", "gemm.hip", "gemm_kernel.h", "gemm_pow2.hip", "fp8q_device.h"):
        shutil.copy(os.path.join(src, f), dst / f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.source_hash()
    k = dst / "gemm_kernel.h"
    text = k.read_text()
    k.write_text(text.replace("namespace fp8q {", "namespace fp8q {  // a new comment\n/* and a block\n comment */\n\n", 1))
    assert bench.source_hash() == h0
    k.write_text(text.replace("constexpr int64_t kCUs = 256;", "constexpr int64_t kCUs = 255;", 1))
    assert bench.source_hash() != h0
