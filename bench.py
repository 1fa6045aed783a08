"""Benchmark of the fine-grained FP8 training hot path on one MI355X.

One step = every stage of the path over one batch of synthetic input:
  * FP8 Linear layer, 8192 tokens, 7168 -> 18432 channels, forward + backward:
      1x128 and 128x1 quantization of X (bf16) in one pass (1x128 for
        Fprop, 128x1 kept for Wgrad), the same for dY (1x128 for Dgrad,
        128x1 for Wgrad),
      128x128 quantization of the weight (bf16, stored [out][in]) with its
        transposed copy for Dgrad,
      Fprop  Y  = X W       (M=8192,  N=18432, K=7168,  BF16 out),
      Dgrad  dX = dY W^T    (M=8192,  N=7168,  K=18432, BF16 out),
      Wgrad  dW = dY^T X    (M=18432, N=7168,  K=8192,  FP32 out);
  * MoE expert layer forward: 64 experts, 65536 routed tokens (Zipf 1.1,
    rows padded to 128), K=7168, N=2048: 1x128 quantization of the tokens,
    128x128 quantization of the stacked expert weights, grouped Fprop (BF16 out).

value = useful GEMM FLOP of the step (padding rows excluded) / step time, in
TFLOP/s; every kernel of the step is inside the timed region.  Per-kernel
durations come from HIP events recorded on the stream the kernels run on.

After the timed steps, kernels outside the step are timed one by one, each
after a clean eviction of the memory-side cache (their entries carry
"outside_step"; a quantizer's entry also has "warm", the same call timed back
to back without the eviction): the quantizer-only workload as stated (max-abs 1x128 and
128x1 of the activation, max-abs 128x128 of the weight without the
transposed copy), the single-tiling 1x128 and 128x1 quantizers of dY (what
the one-pass quantizer replaces), the power-of-two scale mode of the
activation and weight quantizers, the FP8 -> FP8 1x128 -> 128x1
re-quantization of the activation, and the Fprop and Wgrad GEMMs on
power-of-two operands through the hardware-scaled MFMA path.

vendor_gemm_context: the ROCm library's FP8 GEMM (hipBLASLt) on the Fprop
shape and codes, with per-tensor and with MX scales (it offers no 1x128 /
128x128 block scaling on ROCm), for context; not part of the step.

cpu_baseline: the CPU oracle timed on this host on a bounded slice of every
workload (per_config), with the host's core count and CPU model; each line
also records the parity of the timed GPU run on its slice (quantizer codes and
scales bit for bit, GEMM outputs within the relative Frobenius bound).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--copy-calibration]
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 block-scaled GEMM TFLOP/s & % FP8 MFMA peak; quantizer GB/s (1 GPU)"
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
PEAK_CLOCK_GHZ = 2.4          # the engine clock the published MFMA peak assumes

T, D_IN, D_OUT = 8192, 7168, 18432
G_MOE, N_MOE = 64, 2048


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="accepted for older command lines; the 1 GiB device copy always runs")
    return p.parse_args()


def source_hash():
    """Hash of the device sources with comments and blank space removed: an edit of the kernels' code changes it,
    an edit of their comments does not (the profiles keyed to it stay valid).  No string literal in these files
    holds a comment marker."""
    h = hashlib.sha256()
    for f in ("quant.hip", "gemm.hip", "gemm_kernel.h", "gemm_pow2.hip", "fp8q_device.h"):
        with open(os.path.join(ROOT, "precision_fp8_quant_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


class Step:
    """Device buffers and the kernel sequence of one step."""

    def __init__(self, fp8q):
        from tests.helpers import dev_bf16   # plain host->device copy helper
        from workloads import linear_layer, moe_layer, output_grad
        self.fp8q = fp8q
        t0 = time.time()
        lin = linear_layer()
        dy = output_grad()["dy"]
        moe = moe_layer()
        log(f"[bench] synthetic inputs generated in {time.time() - t0:.1f}s")
        self.x, self.wt, self.dy = dev_bf16(lin["x"]), dev_bf16(lin["wt"]), dev_bf16(dy)
        self.mx, self.mw = dev_bf16(moe["x"]), dev_bf16(moe["wt"])
        self.gmap = torch.from_numpy(moe["group_of_mtile"]).cuda()
        self.moe_tokens = int(moe["counts"].sum())
        self.m_pad = moe["x"].shape[0]
        # per-expert roofline of the grouped GEMM: each expert's time is bounded by
        # its FLOP at the MFMA peak or its bytes (codes, scales, its weights, BF16
        # output of its padded rows) at the HBM peak, whichever is larger
        roof_s = 0.0
        for cnt, pad in zip(moe["counts"], moe["padded"]):
            if pad == 0:
                continue
            flop = 2.0 * int(cnt) * N_MOE * D_IN
            nbytes = pad * D_IN + pad * (D_IN // 128) * 4 + N_MOE * D_IN + (N_MOE // 128) * (D_IN // 128) * 4 \
                + pad * N_MOE * 2
            roof_s += max(flop / (PEAK_FP8_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9))
        self.grouped_roof_us = roof_s * 1e6
        self.host = host_slices(lin, dy, moe)
        del lin, dy, moe
        dev = self.x.device
        u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
        # quantized operands
        self.qx, self.sx = e((T, D_IN), u8), e((D_IN // 128, T), f32)
        self.qw, self.sw = e((D_OUT, D_IN), u8), e((D_OUT // 128, D_IN // 128), f32)
        self.qwt, self.swt = e((D_IN, D_OUT), u8), e((D_IN // 128, D_OUT // 128), f32)
        self.qdy, self.sdy = e((T, D_OUT), u8), e((D_OUT // 128, T), f32)
        self.qdyt, self.sdyt = e((D_OUT, T), u8), e((T // 128, D_OUT), f32)
        self.qxt, self.sxt = e((D_IN, T), u8), e((T // 128, D_IN), f32)
        self.qmx, self.smx = e((self.m_pad, D_IN), u8), e((D_IN // 128, self.m_pad), f32)
        self.qmw, self.smw = e((G_MOE * N_MOE, D_IN), u8), e((G_MOE * N_MOE // 128, D_IN // 128), f32)
        # outputs
        self.y, self.dx = e((T, D_OUT), bf), e((T, D_IN), bf)
        self.dw = e((D_OUT, D_IN), f32)
        self.my = e((self.m_pad, N_MOE), bf)
        self.pow2_q, self.pow2_s = e((T, D_IN), u8), e((D_IN // 128, T), f32)
        self.rq_qt, self.rq_st = e((D_IN, T), u8), e((T // 128, D_IN), f32)
        self.qw_p2, self.sw_p2 = e((D_OUT, D_IN), u8), e((D_OUT // 128, D_IN // 128), f32)
        self.qdyt_p2, self.sdyt_p2 = e((D_OUT, T), u8), e((T // 128, D_OUT), f32)

        bf16_quant_bytes = lambda r, c: r * c * 2 + r * c + (r * c // 128) * 4      # in + codes + scales
        dual_bytes = lambda r, c: r * c * 2 + 2 * r * c + 2 * (r * c // 128) * 4    # in + both tilings
        block_bytes = lambda r, c, t: r * c * 2 + r * c * (2 if t else 1) + (r // 128) * (c // 128) * 4 * (2 if t else 1)
        gf = lambda m, n, k: 2.0 * m * n * k
        # (name, launch fn, algorithmic work, kind of work)
        q = fp8q
        self.kernels = [
            ("quant 1x128+128x1 X", lambda: q.fp8_quant_tile_dual(self.x, q.MAXABS, self.qx, self.sx, self.qxt,
                                                                  self.sxt),
             dual_bytes(T, D_IN), "bytes"),
            ("quant_128x128 W (+transposed)", lambda: q.fp8_quant_block(self.wt, q.MAXABS, True, self.qw, self.sw,
                                                                       self.qwt, self.swt),
             block_bytes(D_OUT, D_IN, True), "bytes"),
            ("gemm Fprop", lambda: q.fp8_gemm_blockscaled(q.FPROP, self.qx, self.sx, self.qw, self.sw, c=self.y),
             gf(T, D_OUT, D_IN), "flop"),
            ("quant 1x128+128x1 dY", lambda: q.fp8_quant_tile_dual(self.dy, q.MAXABS, self.qdy, self.sdy,
                                                                   self.qdyt, self.sdyt),
             dual_bytes(T, D_OUT), "bytes"),
            ("gemm Dgrad", lambda: q.fp8_gemm_blockscaled(q.DGRAD, self.qdy, self.sdy, self.qwt, self.swt, c=self.dx),
             gf(T, D_IN, D_OUT), "flop"),
            ("gemm Wgrad", lambda: q.fp8_gemm_blockscaled(q.WGRAD, self.qdyt, self.sdyt, self.qxt, self.sxt, c=self.dw),
             gf(D_OUT, D_IN, T), "flop"),
            ("quant_1x128 MoE tokens", lambda: q.fp8_quant_tile(self.mx, q.TILE_1x128, q.MAXABS, self.qmx, self.smx),
             bf16_quant_bytes(self.m_pad, D_IN), "bytes"),
            ("quant_128x128 MoE weights", lambda: q.fp8_quant_block(self.mw, q.MAXABS, False, self.qmw, self.smw),
             block_bytes(G_MOE * N_MOE, D_IN, False), "bytes"),
            ("gemm grouped MoE", lambda: q.fp8_gemm_blockscaled_grouped(
                self.gmap, self.qmx, self.smx, self.qmw.view(G_MOE, N_MOE, D_IN),
                self.smw.view(G_MOE, N_MOE // 128, D_IN // 128), c=self.my),
             gf(self.moe_tokens, N_MOE, D_IN), "flop"),
        ]
        self.extra = [
            # the activation and weight quantizers of the quantizer-only workload, each on its own
            ("quant_1x128 X (max-abs)", lambda: q.fp8_quant_tile(self.x, q.TILE_1x128, q.MAXABS, self.qx, self.sx),
             bf16_quant_bytes(T, D_IN), "bytes"),
            ("quant_128x1 X (max-abs)", lambda: q.fp8_quant_tile(self.x, q.TILE_128x1, q.MAXABS, self.qxt,
                                                                 self.sxt),
             bf16_quant_bytes(T, D_IN), "bytes"),
            ("quant_128x128 W (max-abs, no transposed copy)", lambda: q.fp8_quant_block(self.wt, q.MAXABS, False,
                                                                                       self.qw, self.sw),
             block_bytes(D_OUT, D_IN, False), "bytes"),
            # the two single-tiling calls that the one-pass quantizer of dY replaces (same outputs)
            ("quant_1x128 dY (single tiling)", lambda: q.fp8_quant_tile(self.dy, q.TILE_1x128, q.MAXABS, self.qdy,
                                                                         self.sdy),
             bf16_quant_bytes(T, D_OUT), "bytes"),
            ("quant_128x1 dY (single tiling)", lambda: q.fp8_quant_tile(self.dy, q.TILE_128x1, q.MAXABS,
                                                                         self.qdyt, self.sdyt),
             bf16_quant_bytes(T, D_OUT), "bytes"),
            ("quant_1x128 X (pow2 scales)", lambda: q.fp8_quant_tile(self.x, q.TILE_1x128, q.POW2,
                                                                     self.pow2_q, self.pow2_s),
             bf16_quant_bytes(T, D_IN), "bytes"),
            # consumes the pow2 codes written by the line above
            ("requant 1x128->128x1 X (pow2 scales)", lambda: q.fp8_requant_1x128_to_128x1(
                self.pow2_q, self.pow2_s, q.POW2, self.rq_qt, self.rq_st),
             2 * T * D_IN + 2 * (T * D_IN // 128) * 4, "bytes"),
            # power-of-two operands for the hardware-scaled MFMA GEMMs (outputs reuse y / dW)
            ("quant_128x128 W (pow2 scales)", lambda: q.fp8_quant_block(self.wt, q.POW2, False, self.qw_p2,
                                                                       self.sw_p2),
             block_bytes(D_OUT, D_IN, False), "bytes"),
            ("gemm Fprop pow2 (hardware-scaled MFMA)", lambda: q.fp8_gemm_blockscaled_pow2(
                q.FPROP, self.pow2_q, self.pow2_s, self.qw_p2, self.sw_p2, c=self.y),
             gf(T, D_OUT, D_IN), "flop"),
            ("quant_128x1 dY (pow2 scales)", lambda: q.fp8_quant_tile(self.dy, q.TILE_128x1, q.POW2, self.qdyt_p2,
                                                                      self.sdyt_p2),
             bf16_quant_bytes(T, D_OUT), "bytes"),
            ("gemm Wgrad pow2 (hardware-scaled MFMA)", lambda: q.fp8_gemm_blockscaled_pow2(
                q.WGRAD, self.qdyt_p2, self.sdyt_p2, self.rq_qt, self.rq_st, c=self.dw),
             gf(D_OUT, D_IN, T), "flop"),
            # max-abs dY^T (from the step) against the power-of-two X^T: only B's scales in the MFMA
            ("gemm Wgrad, pow2 X only (B scales in the MFMA)", lambda: q.fp8_gemm_blockscaled_pow2(
                q.WGRAD, self.qdyt, self.sdyt, self.rq_qt, self.rq_st, c=self.dw, pow2_operands=q.POW2_B),
             gf(D_OUT, D_IN, T), "flop"),
        ]
        self.step_flop = sum(w for _, _, w, kind in self.kernels if kind == "flop")

    def output_slices(self):
        """Host copies of the step's outputs on the slices the CPU leg computes with the oracle (taken right after
        the timed steps, before the outside-step kernels reuse the buffers)."""
        h = lambda t: t.cpu().numpy()
        starts = np.cumsum([0] + list(self.host["padded"][:3]))
        rows = np.concatenate([np.arange(s0, s0 + 128) for s0 in starts])
        return {"qx": h(self.qx[:2048]), "sx": h(self.sx[:, :2048]),
                "qxt": h(self.qxt[:, :2048]), "sxt": h(self.sxt[:16]),
                "qw": h(self.qw[:2048]), "sw": h(self.sw[:16]),
                "y": h(self.y[:2048, :4096].float()), "dx": h(self.dx[:1024, D_IN - 1024:].float()),
                "dw": h(self.dw[:1024, :1024]), "my": h(self.my[torch.from_numpy(rows).cuda()][:, :512].float())}

    def tiny_outputs(self):
        """The tiny Fprop (128x256x128, FP32 in and out) through the library, for the CPU leg's parity record."""
        from workloads import tiny_fprop
        q = self.fp8q
        d = tiny_fprop()
        a = torch.from_numpy(d["a"]).cuda()
        bt = torch.from_numpy(d["bt"]).cuda()
        qa, sa = q.fp8_quant_tile(a, q.TILE_1x128, q.MAXABS)
        qb, sb = q.fp8_quant_block(bt, q.MAXABS)
        c = q.fp8_gemm_blockscaled(q.FPROP, qa, sa, qb, sb, out_dtype=torch.float32)
        return {"tiny_qa": qa.cpu().numpy(), "tiny_sa": sa.cpu().numpy(), "tiny_qb": qb.cpu().numpy(),
                "tiny_sb": sb.cpu().numpy(), "tiny_c": c.cpu().numpy()}

    def run(self, events=None):
        for i, (_, fn, _, _) in enumerate(self.kernels):
            if events is not None:
                events[i][0].record()
            fn()
            if events is not None:
                events[i][1].record()


def _host_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_slices(lin, dy, moe):
    """Host copies of the slices of the same synthetic inputs that cpu_baseline times the oracle on."""
    starts = np.concatenate([[0], np.cumsum(moe["padded"])])[:4]
    rows = np.concatenate([np.arange(s0, s0 + 128) for s0 in starts])
    return {"x": lin["x"][:2048].copy(), "wt": lin["wt"][:4096].copy(),
            "wt_in": np.ascontiguousarray(lin["wt"][:, D_IN - 1024:]), "dy": dy[:1024].copy(),
            "dy_t": np.ascontiguousarray(dy[:, :1024]), "x_t": np.ascontiguousarray(lin["x"][:, :1024]),
            "mx": moe["x"][rows], "mw": np.stack([moe["wt"][e * N_MOE:e * N_MOE + 512] for e in range(4)]),
            "counts": np.asarray(moe["counts"][:4]), "padded": np.asarray(moe["padded"][:4])}


def cpu_baseline(host, gpu=None):
    """The oracle, as it stands, timed on this host's cores on a bounded slice of every workload (the median of 3
    runs for the tiny problem and the quantizer slices, one run for each GEMM slice).

    Operand preparation (widening, and the oracle's own quantization of the GEMM operand slices) is outside
    the timed parts; each GEMM line times the exact per-K-group product of its slice.  The headline value is the
    Fprop slice's rate; every line is in per_config.  With `gpu` (the step's outputs on the same slices), every
    line also records the parity of the timed GPU run on its slice: bit-exact codes and scales for the quantizers,
    the relative Frobenius error against the oracle's product rounded to the output dtype for the GEMMs (bound
    1e-3 for BF16, 2e-4 for FP32 outputs)."""
    from threadpoolctl import threadpool_info
    from oracle import gemm as og, quant as oq
    from workloads import bf16_bits_as_f32, tiny_fprop
    lines = []

    out = {}

    def timed(fn, key=None, runs=1):
        # the median of `runs` timings (3 for the tiny and quantizer slices, 1 for the GEMM slices)
        ts = []
        for _ in range(runs):
            t0 = time.perf_counter()
            r = fn()
            ts.append(time.perf_counter() - t0)
        if key is not None:
            out[key] = r
        return float(np.median(ts))

    def add(config, kernel, secs, work, kind, sample, parity=None):
        rate = work / secs / (1e12 if kind == "flop" else 1e9)
        line = {"config": config, "kernel": kernel, "oracle_s": round(secs, 3),
                "rate": round(rate, 5), "unit": "TFLOP/s" if kind == "flop" else "GB/s", "sample": sample}
        if gpu is not None and parity is not None:
            line["parity"] = parity()
        lines.append(line)

    def exact(*pairs):          # codes and scales, bit for bit
        bad = 0
        for g, o in pairs:
            g8, o8 = np.ascontiguousarray(g).view(np.uint8), np.ascontiguousarray(o).view(np.uint8)
            bad += int(np.count_nonzero(g8 != o8)) if g8.shape == o8.shape else max(g8.size, o8.size)
        return "bit-exact" if bad == 0 else f"MISMATCH: {bad} bytes differ"

    def close(got, ref, out_dtype):
        # rel_frobenius: against the exact product rounded once to the output dtype (the bar);
        # rel_frobenius_raw: against the unrounded FP64 product (BF16's own rounding floor is ~1.7e-3)
        bound = 1e-3 if out_dtype == "bf16" else 2e-4
        got = np.asarray(got, dtype=np.float64)
        err = float(og.rel_frobenius(got, og.round_output(ref, out_dtype)))
        raw = float(og.rel_frobenius(got, ref))
        return {"rel_frobenius": float(f"{err:.3g}"), "rel_frobenius_raw": float(f"{raw:.3g}"), "bound": bound,
                "ok": err <= bound}

    # tiny Fprop: quantize both operands and multiply, whole problem
    d = tiny_fprop()
    def tiny():
        qa, sa = oq.quant_1x128(d["a"])
        qb, sb = oq.quant_128x128(d["bt"])
        return qa, sa, qb, sb, og.gemm_ref(qa, sa, qb, sb, og.FPROP, exact_int=True)

    def tiny_parity():
        qa, sa, qb, sb, c = out["tiny"]
        codes = exact((gpu["tiny_qa"], qa), (gpu["tiny_sa"], sa), (gpu["tiny_qb"], qb), (gpu["tiny_sb"], sb))
        return {"codes_and_scales": codes, **close(gpu["tiny_c"], c, "f32")}
    add("tiny Fprop 128x256x128", "quant 1x128 + 128x128 + Fprop (int64)", timed(tiny, "tiny", runs=3),
        2.0 * 128 * 128 * 256, "flop", "whole problem", tiny_parity)
    # quantizer-only workload: 2048 of the 8192 activation rows, 2048 of the 18432 weight rows
    x = bf16_bits_as_f32(host["x"][:2048])
    qbytes = x.size * 2 + x.size + x.size // 128 * 4
    add("quantizer-only", "quant_1x128 X (max-abs)", timed(lambda: oq.quant_1x128(x), "q1", runs=3), qbytes, "bytes",
        "X rows 0..2047 of 8192", lambda: exact((gpu["qx"], out["q1"][0]), (gpu["sx"], out["q1"][1])))
    add("quantizer-only", "quant_1x128 X (pow2)", timed(lambda: oq.quant_1x128(x, oq.MODE_POW2), "p1", runs=3), qbytes,
        "bytes", "X rows 0..2047 of 8192",
        lambda: exact((gpu["pow2_q"], out["p1"][0]), (gpu["pow2_s"], out["p1"][1])))
    add("quantizer-only", "quant_128x1 X (max-abs)", timed(lambda: oq.quant_128x1(x), "t1", runs=3), qbytes, "bytes",
        "X rows 0..2047 of 8192", lambda: exact((gpu["qxt"], out["t1"][0]), (gpu["sxt"], out["t1"][1])))
    w = bf16_bits_as_f32(host["wt"][:2048])
    add("quantizer-only", "quant_128x128 W (max-abs)", timed(lambda: oq.quant_128x128(w), "b1", runs=3),
        w.size * 3 + (w.size // 16384) * 4, "bytes", "W rows 0..2047 of 18432",
        lambda: exact((gpu["qw"], out["b1"][0]), (gpu["sw"], out["b1"][1])))
    # Fprop: 2048 tokens x 4096 output channels, full K = 7168
    qa, sa = oq.quant_1x128(bf16_bits_as_f32(host["x"]))
    qb, sb = oq.quant_128x128(bf16_bits_as_f32(host["wt"]))
    f_s = timed(lambda: og.gemm_ref(qa, sa, qb, sb, og.FPROP), "fprop")
    f_flop = 2.0 * qa.shape[0] * qb.shape[0] * D_IN
    add("Fprop", "gemm Fprop", f_s, f_flop, "flop", f"M={qa.shape[0]} of 8192, N={qb.shape[0]} of 18432, K={D_IN}",
        lambda: close(gpu["y"], out["fprop"], "bf16"))
    # Dgrad: 1024 tokens x the last 1024 input channels (the columns whose tiles run in the last wave, with K
    # split in two), full K = 18432
    qa, sa = oq.quant_1x128(bf16_bits_as_f32(host["dy"]))
    qb, sb = oq.quant_128x128(np.ascontiguousarray(bf16_bits_as_f32(host["wt_in"]).T))
    add("Dgrad + Wgrad", "gemm Dgrad", timed(lambda: og.gemm_ref(qa, sa, qb, sb, og.DGRAD), "dgrad"),
        2.0 * qa.shape[0] * qb.shape[0] * D_OUT, "flop", f"M=1024 of 8192, N=1024 of 7168 (input channels 6144..7167), K={D_OUT}",
        lambda: close(gpu["dx"], out["dgrad"], "bf16"))
    # Wgrad: 1024 output x 1024 input channels, full K = 8192 tokens
    qa, sa = oq.quant_128x1(bf16_bits_as_f32(host["dy_t"]))
    qb, sb = oq.quant_128x1(bf16_bits_as_f32(host["x_t"]))
    add("Dgrad + Wgrad", "gemm Wgrad", timed(lambda: og.gemm_ref(qa, sa, qb, sb, og.WGRAD), "wgrad"),
        2.0 * qa.shape[0] * qb.shape[0] * T, "flop", f"M=1024 of 18432, N=1024 of 7168, K={T}",
        lambda: close(gpu["dw"], out["wgrad"], "f32"))
    # grouped: the first 128-row tile of experts 0..3, N = 512 of 2048 (real rows only in the FLOP count)
    qa, sa = oq.quant_1x128(bf16_bits_as_f32(host["mx"]))
    qbs = [oq.quant_128x128(bf16_bits_as_f32(wv)) for wv in host["mw"]]
    qb = np.stack([q_ for q_, _ in qbs])
    sb = np.stack([s_ for _, s_ in qbs])
    gmap = np.arange(4, dtype=np.int32)
    real = sum(min(128, int(c)) for c in host["counts"])
    add("grouped MoE", "gemm grouped MoE", timed(lambda: og.grouped_ref(qa, sa, qb, sb, gmap), "grouped"),
        2.0 * real * 512 * D_IN, "flop", "first 128-row tile of experts 0..3, N=512 of 2048, K=7168",
        lambda: close(gpu["my"], out["grouped"], "bf16"))

    blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    head = next(l for l in lines if l["kernel"] == "gemm Fprop")
    return {"value": head["rate"], "unit": "TFLOP/s", "cores": max(blas + [1]), "kind": "oracle",
            "sample": f"Fprop slice {head['sample']}: the oracle's exact per-K-group GEMM, {head['oracle_s']} s "
                      f"(every workload's slice in per_config)",
            "nproc": os.cpu_count(), "host_cpu": _host_model(),
            "threads_note": "numpy elementwise work (the quantizers) runs on one thread; the per-group FP64 "
                            "matmuls use the BLAS threads given in cores",
            "oracle_s_total": round(sum(l["oracle_s"] for l in lines), 2), "per_config": lines}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported in this build "
              "(the path's multi-GPU sharding is a design note, not code)", file=sys.stderr)
        sys.exit(2)
    import precision_fp8_quant_amd as fp8q
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.set_device(0)
    step = Step(fp8q)

    # untimed warm-up
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    nk = len(step.kernels)
    events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nk)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step.run(events[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"[bench] timed {args.steps} steps in {elapsed:.3f}s")

    per_kernel = {}
    for i, (name, _, work, kind) in enumerate(step.kernels):
        us = float(np.mean([events[s][i][0].elapsed_time(events[s][i][1]) for s in range(args.steps)])) * 1e3
        per_kernel[name] = _kernel_entry(us, work, kind)
    gpu_out = None if args.no_cpu_baseline else step.output_slices()

    # extra kernels outside the step, in order (power-of-two scale mode, FP8 re-tiling, hardware-scaled GEMMs).
    # Timed one call at a time, each preceded (outside its events) by a read of 512 MiB that evicts the
    # 256 MB MALL with clean lines, so that inputs below its size are not served from it on repeated calls
    # (a fill would leave dirty lines whose write-back the timed kernel would pay); inside the step every
    # kernel already follows one that streams gigabytes.
    scrub = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    for name, fn, work, kind in step.extra:
        for _ in range(2):      # warm-up in the timed pattern: the first call after the first eviction read ran 3x slower
            scrub.amax()
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in ev:
            scrub.amax()
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
        per_kernel[name] = dict(_kernel_entry(us, work, kind), outside_step=True)
        if kind == "bytes":
            # warm: the same call back to back, its input (and output) partly left in the MALL by the call before
            wev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
            for a, b in wev:
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            wus = float(np.mean([a.elapsed_time(b) for a, b in wev])) * 1e3
            per_kernel[name]["warm"] = _kernel_entry(wus, work, kind)

    del scrub

    # a plain 1 GiB device copy: the secondary HBM reference (and the calibration
    # point of the rocprofv3 FETCH_SIZE / WRITE_SIZE counters)
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    cps = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        cps.append(a.elapsed_time(b) * 1e3)
    per_kernel["calibration copy 1 GiB"] = dict(_kernel_entry(float(np.median(cps)), 2 << 30, "bytes"),
                                                outside_step=True)
    del src, dst

    vendor = vendor_gemm_context(step, args.steps, per_kernel)

    g = per_kernel["gemm grouped MoE"]
    g["per_expert_roof_us"] = round(step.grouped_roof_us, 1)
    g["per_expert_roof_frac"] = round(step.grouped_roof_us / g["us"], 4)

    ms_per_step = elapsed / args.steps * 1e3
    value = step.step_flop / (elapsed / args.steps) / 1e12

    in_step = {k: v for k, v in per_kernel.items() if not v.get("outside_step")}
    dom_name = max(in_step, key=lambda k: in_step[k]["us"])
    dom = in_step[dom_name]
    roof = _roofline(dom_name, dom)

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f8e4m3 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": "FP8 Linear fwd+bwd (8192 tokens, 7168->18432) + MoE grouped Fprop "
                               "(64 experts, 65536 tokens Zipf(1.1), 7168->2048)",
                   "tokens": T, "d_in": D_IN, "d_out": D_OUT, "moe_experts": G_MOE, "moe_tokens": step.moe_tokens,
                   "moe_rows_padded": step.m_pad, "scale_mode": "maxabs", "parallelism": "single GPU"},
        "gemm_flop_per_step": step.step_flop,
        "kernels": per_kernel,
        "roofline": roof,
        "cpu_baseline": None,
        "vendor_gemm_context": vendor,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        gpu_out["pow2_q"], gpu_out["pow2_s"] = step.pow2_q[:2048].cpu().numpy(), step.pow2_s[:, :2048].cpu().numpy()
        gpu_out.update(step.tiny_outputs())
        result["cpu_baseline"] = cpu_baseline(step.host, gpu_out)
    print(json.dumps(result), flush=True)


def vendor_gemm_context(step, steps, per_kernel):
    """The ROCm library's own FP8 GEMM (hipBLASLt, through torch's scaled matrix multiply) on the Fprop shape and
    the same E4M3 codes, for context: it has no 1x128 / 128x128 block scaling on ROCm, so it runs with one scale
    per tensor (no per-group work at all) and with MX scales (one E8M0 exponent per 32 K values in the matrix core,
    the library's counterpart of the hardware-scaled path).  Not part of the step or of the path."""
    import torch.nn.functional as F
    qa = step.qx.view(torch.float8_e4m3fn)
    qb = step.qw.view(torch.float8_e4m3fn).t()
    one = torch.ones((), dtype=torch.float32, device="cuda")
    e8 = lambda rows: torch.full((rows, D_IN // 32), 1.0, device="cuda").to(torch.float8_e8m0fnu)
    ea, eb = e8(T), e8(D_OUT)
    cases = {
        "per-tensor scales": (lambda: torch._scaled_mm(qa, qb, scale_a=one, scale_b=one, out_dtype=torch.bfloat16),
                              "gemm Fprop"),
        "MX scales (E8M0 per 32 K, in the matrix core)": (
            lambda: F.scaled_mm(qa, qb, ea, F.ScalingType.BlockWise1x32, eb, F.ScalingType.BlockWise1x32,
                                F.SwizzleType.NO_SWIZZLE, F.SwizzleType.NO_SWIZZLE),
            "gemm Fprop pow2 (hardware-scaled MFMA)"),
    }
    out = {"library": "hipBLASLt (torch scaled_mm)", "shape": f"M={T} N={D_OUT} K={D_IN}, BF16 out",
           "operands": "the step's Fprop E4M3 codes", "cases": {}}
    for name, (fn, ours) in cases.items():
        try:
            for _ in range(2):
                fn()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
            for a, b in ev:
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
            e = _kernel_entry(us, 2.0 * T * D_OUT * D_IN, "flop")
            e["ours"] = ours
            e["library_us_over_ours"] = round(e["us"] / per_kernel[ours]["us"], 3) if ours in per_kernel else None
            out["cases"][name] = e
        except Exception as ex:        # the library may lack the mode on a given ROCm
            out["cases"][name] = {"unavailable": f"{type(ex).__name__}: {str(ex).splitlines()[0][:120]}"}
    return out


def _kernel_entry(us, work, kind):
    if kind == "flop":
        tf = work / (us * 1e-6) / 1e12
        return {"us": round(us, 2), "tflops": round(tf, 1), "frac_peak": round(tf / PEAK_FP8_TFLOPS, 4),
                "flop": work}
    gbs = work / (us * 1e-6) / 1e9
    return {"us": round(us, 2), "gbs": round(gbs, 1), "frac_peak": round(gbs / PEAK_HBM_GBS, 4), "bytes": work}


def _roofline(name, k):
    """Roofline entry of the dominant kernel.  traffic (calibrated HBM bytes per launch) and, for an MFMA-bound
    kernel, its average shader clock come from profiles/hbm_traffic.json, and its matrix-core busy fraction from
    profiles/gemm_counters.json, each only while that file's kernel source hash matches; frac_at_clock sets the
    achieved rate against the published peak scaled from its 2.4 GHz to that clock."""
    traffic, clock, util = None, None, None
    tpath = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if os.path.exists(tpath):
        with open(tpath) as fh:
            t = json.load(fh)
        if t.get("source_hash") == source_hash():
            traffic = t.get("kernels", {}).get(name)
            clock = t.get("clock_ghz", {}).get(name)
    cpath = os.path.join(ROOT, "profiles", "gemm_counters.json")
    if os.path.exists(cpath):
        with open(cpath) as fh:
            c = json.load(fh)
        if c.get("source_hash") == source_hash():
            util = c.get("gemms", {}).get(name)
    if "tflops" in k:
        r = {"kernel": name, "bound": "mfma", "achieved": k["tflops"], "peak": PEAK_FP8_TFLOPS,
             "unit": "TFLOP/s", "frac": round(k["tflops"] / PEAK_FP8_TFLOPS, 4), "traffic": traffic,
             "avg_us": k["us"]}
        if clock:
            r["clock_ghz"] = clock
            r["frac_at_clock"] = round(k["tflops"] / (PEAK_FP8_TFLOPS * clock / PEAK_CLOCK_GHZ), 4)
        if util:
            # matrix-core busy fraction of all SIMD cycles, and the VALU work beside it (rocprofv3 counters)
            r["mfma_busy"] = util["mfma_busy"]
            r["valu_insts_per_mfma"] = util["valu_insts_per_mfma"]
            r["valu_busy_est"] = util["valu_busy_est"]
        return r
    return {"kernel": name, "bound": "hbm", "achieved": k["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(k["gbs"] / PEAK_HBM_GBS, 4), "traffic": traffic, "avg_us": k["us"]}


if __name__ == "__main__":
    main()
