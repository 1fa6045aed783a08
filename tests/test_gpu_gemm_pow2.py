"""GPU parity of the hardware-scaled GEMM (fp8_gemm_blockscaled_pow2) against
the CPU oracle, through the C ABI, and the accumulation-precision probe.

The pow2 path hands every (power-of-two) scale to the MFMA as an E8M0 code and
accumulates all K-groups inside the MFMA, so it computes the same sum as the
oracle's block-scaled GEMM in a different rounding order.  Criterion: relative
Frobenius error <= 1e-3 against the oracle's exact product rounded once to the
output dtype; a small-integer case is exact and must match bit for bit (it
pins the E8M0 scale operands: per A row, per B row or block).
"""

import numpy as np
import pytest
import torch

from oracle import gemm as og, quant as oq
from tests.helpers import dev, dev_bf16, host, host_bf16_as_f64, require_gpu
from workloads import linear_layer, output_grad, random_fp8_operands

pytestmark = pytest.mark.gpu

TOL = 1e-3
TOL_F32 = 2e-4      # same FP32-output bound as the promoted GEMM (8-product MFMA blocks)
KINDS = {"fprop": 0, "dgrad": 1, "wgrad": 2}
MASKS = {"A": 1, "B": 2, "AB": 3}


def _mixed_operands(seed, m, n, k, kind, mask):
    """Random codes; the scales of the operands named in mask are powers of two,
    the others arbitrary positive floats."""
    p2 = random_fp8_operands(seed, m, n, k, kind=kind, pow2=True)
    anyv = random_fp8_operands(seed, m, n, k, kind=kind, pow2=False)
    return {"qa": p2["qa"], "qb": p2["qb"],
            "sa": p2["sa"] if "A" in mask else anyv["sa"],
            "sb": p2["sb"] if "B" in mask else anyv["sb"]}


def _out_host(c):
    return host_bf16_as_f64(c) if c.dtype == torch.bfloat16 else host(c).astype(np.float64)


@pytest.mark.parametrize("kind", ["fprop", "dgrad", "wgrad"])
@pytest.mark.parametrize("mnk", [(256, 384, 640), (256, 256, 128), (512, 512, 640), (256, 768, 1152)])
def test_pow2_exact_small_integer_problem(kind, mnk):
    """128x256 tiles (256, 384, 640) and 256x256 tiles: one K-group, and odd
    K-group counts over several tiles."""
    fp8q = require_gpu()
    rng = np.random.default_rng(131 + sum(mnk))
    m, n, k = mnk
    ints = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50], np.uint8)   # 0,1..8
    def codes(shape):
        c = ints[rng.integers(0, ints.size, size=shape)]
        return (c | (rng.integers(0, 2, size=shape) << 7).astype(np.uint8)).astype(np.uint8)
    qa, qb = codes((m, k)), codes((n, k))
    sa = np.exp2(rng.integers(-3, 3, size=(k // 128, m))).astype(np.float32)
    if kind == "wgrad":
        sb = np.exp2(rng.integers(-2, 3, size=(k // 128, n))).astype(np.float32)
    else:
        sb = np.exp2(rng.integers(-2, 3, size=(n // 128, k // 128))).astype(np.float32)
    c = fp8q.fp8_gemm_blockscaled_pow2(KINDS[kind], dev(qa), dev(sa), dev(qb), dev(sb), out_dtype=torch.float32)
    ref = og.gemm_ref(qa, sa, qb, sb, kind, exact_int=True)
    got = _out_host(c)
    assert np.array_equal(got, ref), f"max abs diff {np.max(np.abs(got - ref))}"


@pytest.mark.parametrize("kind", ["fprop", "dgrad", "wgrad"])
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("mnk", [(256, 384, 640), (128, 128, 128), (384, 256, 1024), (256, 256, 4096)])
def test_pow2_random_operands(kind, out, mnk):
    fp8q = require_gpu()
    m, n, k = mnk
    ops = random_fp8_operands(141 + m + n + k, m, n, k, kind=kind, pow2=True)
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    c = fp8q.fp8_gemm_blockscaled_pow2(KINDS[kind], dev(ops["qa"]), dev(ops["sa"]), dev(ops["qb"]),
                                       dev(ops["sb"]), out_dtype=dt)
    ref = og.gemm_ref(ops["qa"], ops["sa"], ops["qb"], ops["sb"], kind)
    err = og.rel_frobenius(_out_host(c), og.round_output(ref, out))
    assert err <= (TOL if out == "bf16" else TOL_F32), err


def test_pow2_extreme_scale_exponents():
    # E8M0 codes from 2^-126 to 2^100 on A rows against moderate B scales
    fp8q = require_gpu()
    rng = np.random.default_rng(151)
    m, n, k = 256, 256, 512
    ops = random_fp8_operands(152, m, n, k, kind="fprop", pow2=True)
    sa = np.exp2(rng.integers(-126, 101, size=(k // 128, m)).astype(np.float64)).astype(np.float32)
    sb = np.exp2(rng.integers(-20, 1, size=(n // 128, k // 128)).astype(np.float64)).astype(np.float32)
    c = fp8q.fp8_gemm_blockscaled_pow2(0, dev(ops["qa"]), dev(sa), dev(ops["qb"]), dev(sb), out_dtype=torch.float32)
    ref = og.gemm_ref(ops["qa"], sa, ops["qb"], sb, "fprop")
    got = _out_host(c)
    # rows are dominated by their largest group scale; compare row by row
    for r in range(0, m, 17):
        assert og.rel_frobenius(got[r], og.round_output(ref[r], "f32")) <= TOL_F32, r


@pytest.mark.parametrize("mask", ["A", "B"])
@pytest.mark.parametrize("kind", ["fprop", "dgrad", "wgrad"])
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("mnk", [(256, 384, 640), (384, 256, 1024), (512, 512, 2048)])
def test_one_pow2_operand_random(mask, kind, out, mnk):
    """One operand's scales applied in the MFMA, the other's by the promotion."""
    fp8q = require_gpu()
    m, n, k = mnk
    ops = _mixed_operands(211 + m + n + k, m, n, k, kind, mask)
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    c = fp8q.fp8_gemm_blockscaled_pow2(KINDS[kind], dev(ops["qa"]), dev(ops["sa"]), dev(ops["qb"]), dev(ops["sb"]),
                                       out_dtype=dt, pow2_operands=MASKS[mask])
    ref = og.gemm_ref(ops["qa"], ops["sa"], ops["qb"], ops["sb"], kind)
    err = og.rel_frobenius(_out_host(c), og.round_output(ref, out))
    assert err <= (TOL if out == "bf16" else TOL_F32), err


@pytest.mark.parametrize("mask", ["A", "B"])
@pytest.mark.parametrize("kind", ["fprop", "wgrad"])
def test_one_pow2_operand_exact_small_integers(mask, kind):
    fp8q = require_gpu()
    rng = np.random.default_rng(221)
    m, n, k = 256, 256, 384
    ints = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50], np.uint8)
    def codes(shape):
        c = ints[rng.integers(0, ints.size, size=shape)]
        return (c | (rng.integers(0, 2, size=shape) << 7).astype(np.uint8)).astype(np.uint8)
    qa, qb = codes((m, k)), codes((n, k))
    sa = np.exp2(rng.integers(-3, 3, size=(k // 128, m))).astype(np.float32)
    shape_b = (k // 128, n) if kind == "wgrad" else (n // 128, k // 128)
    sb = np.exp2(rng.integers(-2, 3, size=shape_b)).astype(np.float32)
    c = fp8q.fp8_gemm_blockscaled_pow2(KINDS[kind], dev(qa), dev(sa), dev(qb), dev(sb), out_dtype=torch.float32,
                                       pow2_operands=MASKS[mask])
    ref = og.gemm_ref(qa, sa, qb, sb, kind, exact_int=True)
    got = _out_host(c)
    assert np.array_equal(got, ref), f"max abs diff {np.max(np.abs(got - ref))}"


@pytest.mark.parametrize("mask", ["A", "B"])
@pytest.mark.parametrize("kind", ["fprop", "wgrad"])
def test_one_pow2_operand_accumulate(mask, kind):
    """FP32 accumulate into an existing C with one operand's scales in the MFMA."""
    fp8q = require_gpu()
    m, n, k = 256, 512, 640
    ops = _mixed_operands(231 + len(kind), m, n, k, kind, mask)
    c0 = np.random.default_rng(232).standard_normal((m, n)).astype(np.float32)
    c = dev(c0.copy())
    fp8q.fp8_gemm_blockscaled_pow2(KINDS[kind], dev(ops["qa"]), dev(ops["sa"]), dev(ops["qb"]), dev(ops["sb"]), c=c,
                                   accumulate=True, pow2_operands=MASKS[mask])
    ref = og.gemm_ref(ops["qa"], ops["sa"], ops["qb"], ops["sb"], kind) + c0.astype(np.float64)
    assert og.rel_frobenius(host(c).astype(np.float64), ref) <= TOL_F32


def test_pow2_wgrad_accumulate_and_k_zero():
    fp8q = require_gpu()
    m, n, k = 256, 512, 384
    ops = random_fp8_operands(161, m, n, k, kind="wgrad", pow2=True)
    c0 = np.random.default_rng(162).standard_normal((m, n)).astype(np.float32)
    c = dev(c0.copy())
    fp8q.fp8_gemm_blockscaled_pow2(2, dev(ops["qa"]), dev(ops["sa"]), dev(ops["qb"]), dev(ops["sb"]), c=c,
                                   accumulate=True)
    ref = og.gemm_ref(ops["qa"], ops["sa"], ops["qb"], ops["sb"], "wgrad") + c0.astype(np.float64)
    assert og.rel_frobenius(host(c).astype(np.float64), ref) <= TOL_F32
    z = torch.full((256, 256), 7.0, device="cuda")
    e = torch.empty((256, 0), dtype=torch.uint8, device="cuda")
    es = torch.empty((0, 256), dtype=torch.float32, device="cuda")
    fp8q.fp8_gemm_blockscaled_pow2(2, e, es, e, es, c=z)
    assert np.all(host(z) == 0.0)


def test_pow2_deterministic():
    fp8q = require_gpu()
    ops = random_fp8_operands(171, 512, 512, 1024, pow2=True)
    args = [dev(ops[x]) for x in ("qa", "sa", "qb", "sb")]
    c1 = host(fp8q.fp8_gemm_blockscaled_pow2(0, *args, out_dtype=torch.float32))
    c2 = host(fp8q.fp8_gemm_blockscaled_pow2(0, *args, out_dtype=torch.float32))
    assert np.array_equal(c1.view(np.uint32), c2.view(np.uint32))


# ----------------------------------------------------------------------------
# Many 256x256 tiles, each checked on its own; FP32 plain and accumulating;
# the tail of a grid split off as 128x256 tiles.
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("kind,out,k", [("fprop", "bf16", 256), ("dgrad", "f32", 640), ("wgrad", "f32", 1152),
                                         ("wgrad", "f32acc", 384), ("fprop", "f32acc", 128)])
def test_pow2_many_tiles_every_tile(kind, out, k):
    fp8q = require_gpu()
    m = n = 2048                                   # 64 tiles of 256x256
    ops = random_fp8_operands(401 + k, m, n, k, kind=kind, pow2=True)
    ref = og.gemm_ref(ops["qa"], ops["sa"], ops["qb"], ops["sb"], kind)
    args = [dev(ops[x]) for x in ("qa", "sa", "qb", "sb")]
    c0 = np.random.default_rng(402).standard_normal((m, n)).astype(np.float32)
    outs = []
    for _ in range(2):
        if out == "f32acc":
            c = dev(c0.copy())
            fp8q.fp8_gemm_blockscaled_pow2(KINDS[kind], *args, c=c, accumulate=True)
            got, want, tol = host(c).astype(np.float64), ref + c0.astype(np.float64), TOL_F32
        else:
            dt = torch.bfloat16 if out == "bf16" else torch.float32
            c = fp8q.fp8_gemm_blockscaled_pow2(KINDS[kind], *args, out_dtype=dt)
            got, want, tol = _out_host(c), og.round_output(ref, out), (TOL if out == "bf16" else TOL_F32)
        outs.append(got)
        for r0 in range(0, m, 256):
            for c0_ in range(0, n, 256):
                t = (slice(r0, r0 + 256), slice(c0_, c0_ + 256))
                assert og.rel_frobenius(got[t], want[t]) <= tol, (r0, c0_)
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("kind", ["fprop", "dgrad"])
def test_pow2_tail_balanced_two_grid_launch(kind):
    """M=512, N=129*256: 258 tiles of 256x256, so the last 256-column band runs
    as a second grid of 128x256 tiles."""
    fp8q = require_gpu()
    m, n, k = 512, 129 * 256, 384
    ops = random_fp8_operands(411, m, n, k, kind=kind, pow2=True)
    ref = og.gemm_ref(ops["qa"], ops["sa"], ops["qb"], ops["sb"], kind)
    c = fp8q.fp8_gemm_blockscaled_pow2(KINDS[kind], *[dev(ops[x]) for x in ("qa", "sa", "qb", "sb")],
                                       out_dtype=torch.bfloat16)
    got, want = host_bf16_as_f64(c), og.round_bf16(ref)
    for cols in (slice(0, 128 * 256), slice(128 * 256, n)):          # first grid, second grid
        assert og.rel_frobenius(got[:, cols], want[:, cols]) <= TOL, cols


@pytest.fixture(scope="module")
def layer():
    return linear_layer()


def test_pow2_fprop_full_size_sampled(layer):
    """Y = X W at M=8192, N=18432, K=7168 with power-of-two scales on both
    operands (quantizers in POW2 mode), BF16 out, sampled entries."""
    fp8q = require_gpu()
    d = layer
    qx, sx = fp8q.fp8_quant_tile(dev_bf16(d["x"]), fp8q.TILE_1x128, fp8q.POW2)
    qw, sw = fp8q.fp8_quant_block(dev_bf16(d["wt"]), fp8q.POW2)
    y = fp8q.fp8_gemm_blockscaled_pow2(0, qx, sx, qw, sw, out_dtype=torch.bfloat16)
    rng = np.random.default_rng(181)
    rows = np.sort(rng.choice(8192, 24, replace=False))
    bands = [0, 71, 143]
    cols = np.concatenate([b * 128 + np.sort(rng.choice(128, 16, replace=False)) for b in bands])
    qx_r, sx_r = oq.quant_1x128(oq.bf16_bits_to_f32(d["x"][rows]), "pow2")
    qw_r = np.zeros((18432, 7168), np.uint8)
    sw_r = np.zeros((144, 56), np.float32)
    for b in bands:
        rs = slice(b * 128, (b + 1) * 128)
        qw_r[rs], sw_r[b:b + 1] = oq.quant_128x128(oq.bf16_bits_to_f32(d["wt"][rs]), "pow2")
    rr, cc = np.meshgrid(np.arange(rows.size), cols, indexing="ij")
    ref = og.gemm_ref_entries(qx_r, sx_r, qw_r, sw_r, rr.ravel(), cc.ravel(), "fprop")
    got = host_bf16_as_f64(y)[rows][:, cols].ravel()
    assert og.rel_frobenius(got, og.round_bf16(ref)) <= TOL


def test_wgrad_full_size_pow2_x_operand_only(layer):
    """dW = dY^T X at full size with dY^T max-abs 128x1 and X^T power-of-two
    128x1 (pow2_operands = B), FP32 out, sampled entries."""
    fp8q = require_gpu()
    d = layer
    dy = output_grad()["dy"]
    qdyt, sdy = fp8q.fp8_quant_tile(dev_bf16(dy), fp8q.TILE_128x1, fp8q.MAXABS)
    qxt, sx = fp8q.fp8_quant_tile(dev_bf16(d["x"]), fp8q.TILE_128x1, fp8q.POW2)
    dw = fp8q.fp8_gemm_blockscaled_pow2(2, qdyt, sdy, qxt, sx, out_dtype=torch.float32, pow2_operands=fp8q.POW2_B)
    rng = np.random.default_rng(185)
    ms = np.sort(rng.choice(18432, 24, replace=False))
    ns = np.sort(rng.choice(7168, 40, replace=False))
    qa_r, sa_r = oq.quant_128x1(oq.bf16_bits_to_f32(dy[:, ms]), "maxabs")
    qb_r, sb_r = oq.quant_128x1(oq.bf16_bits_to_f32(d["x"][:, ns]), "pow2")
    rr, cc = np.meshgrid(np.arange(ms.size), np.arange(ns.size), indexing="ij")
    ref = og.gemm_ref_entries(qa_r, sa_r, qb_r, sb_r, rr.ravel(), cc.ravel(), "wgrad")
    got = host(dw)[ms][:, ns].ravel().astype(np.float64)
    assert og.rel_frobenius(got, og.round_output(ref, "f32")) <= TOL_F32


def test_pow2_wgrad_full_size_sampled(layer):
    """dW = dY^T X at M=18432, N=7168, K=8192 with both operands 128x1 POW2, FP32 out."""
    fp8q = require_gpu()
    d = layer
    dy = output_grad()["dy"]
    qdyt, sdy = fp8q.fp8_quant_tile(dev_bf16(dy), fp8q.TILE_128x1, fp8q.POW2)
    qxt, sx = fp8q.fp8_quant_tile(dev_bf16(d["x"]), fp8q.TILE_128x1, fp8q.POW2)
    dw = fp8q.fp8_gemm_blockscaled_pow2(2, qdyt, sdy, qxt, sx, out_dtype=torch.float32)
    rng = np.random.default_rng(183)
    ms = np.sort(rng.choice(18432, 24, replace=False))
    ns = np.sort(rng.choice(7168, 40, replace=False))
    qa_r, sa_r = oq.quant_128x1(oq.bf16_bits_to_f32(dy[:, ms]), "pow2")
    qb_r, sb_r = oq.quant_128x1(oq.bf16_bits_to_f32(d["x"][:, ns]), "pow2")
    rr, cc = np.meshgrid(np.arange(ms.size), np.arange(ns.size), indexing="ij")
    ref = og.gemm_ref_entries(qa_r, sa_r, qb_r, sb_r, rr.ravel(), cc.ravel(), "wgrad")
    got = host(dw)[ms][:, ns].ravel().astype(np.float64)
    assert og.rel_frobenius(got, og.round_output(ref, "f32")) <= TOL_F32


# ----------------------------------------------------------------------------
# Accumulation-precision probe (the pages' one GEMM-accuracy experiment is a
# K=4096 product with limited accumulation precision: dssusan.co.kr FP8
# excerpt, paragraph 4; the ~14-bit accumulation of their hardware:
# paragraph 2).  Unit scales, so the only difference between the two paths is
# where the sum is kept: promoted to VALU FP32 once per 128-deep group
# (fp8_gemm_blockscaled) or accumulated inside the MFMA across all 32 groups
# (fp8_gemm_blockscaled_pow2).
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("data", ["uniform_codes", "quantized_normal"])
def test_accumulation_precision_probe_k4096(data):
    fp8q = require_gpu()
    m = n = 256
    k = 4096
    rng = np.random.default_rng(191)
    if data == "uniform_codes":
        ops = random_fp8_operands(192, m, n, k, pow2=True)
        qa, qb = ops["qa"], ops["qb"]
    else:
        qa, _ = oq.quant_1x128(rng.standard_normal((m, k)).astype(np.float32), "pow2")
        qb, _ = oq.quant_1x128(rng.standard_normal((n, k)).astype(np.float32), "pow2")
    sa = np.ones((k // 128, m), np.float32)
    sb = np.ones((n // 128, k // 128), np.float32)
    exact = og.gemm_ref(qa, sa, qb, sb, "fprop", exact_int=True)
    args = [dev(qa), dev(sa), dev(qb), dev(sb)]
    prom = host(fp8q.fp8_gemm_blockscaled(0, *args, out_dtype=torch.float32)).astype(np.float64)
    chain = host(fp8q.fp8_gemm_blockscaled_pow2(0, *args, out_dtype=torch.float32)).astype(np.float64)
    scale = np.sqrt(np.mean(exact ** 2))
    res = {}
    for name, got in (("promoted_per_128", prom), ("mfma_chained", chain)):
        res[name] = (og.rel_frobenius(got, exact), float(np.max(np.abs(got - exact)) / scale))
    print(f"\n[probe K=4096 {data}] rel_frobenius / max|err|/rms: " +
          ", ".join(f"{k_}: {v[0]:.3e} / {v[1]:.3e}" for k_, v in res.items()))
    for name, (fro, _) in res.items():
        assert fro <= TOL, (name, fro)
