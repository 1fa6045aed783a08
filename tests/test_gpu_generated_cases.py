"""Generated GPU parity cases: shapes, leading dimensions, offsets and paths drawn
from one seeded generator, every case through the C ABI against the oracle.

The hand-picked cases elsewhere pin each kernel's rules one at a time; these
cross them.  Every operand and output is a row-strided view at a column offset
inside a larger buffer with one more row, and the bytes around each view are
filled on purpose:
  * inputs: NaN codes around FP8 operands, NaN around BF16/FP32 inputs and
    around every scale array -- a read outside the operand turns an output into
    NaN (or a scale into one);
  * outputs: a sentinel around codes, scales and GEMM outputs -- a write
    outside the output changes it.
Cases:
  * GEMMs: Fprop, Dgrad, Wgrad on the promoted path and the three hardware-
    scaled paths (A, B or both operands' power-of-two scales in the MFMA), BF16,
    FP32 and accumulating FP32 output, M and N in 128..2048 and K in 128..1280
    (every plain tile configuration).  Bar: relative Frobenius error <= 1e-3
    over the whole output against the oracle's product rounded once to the
    output dtype; on every 128x128 block, <= 2e-4 for the FP32 result, and a
    BF16 output must be exactly the rounding of the same call's FP32 result.
  * grouped GEMMs: N in 128..2048 (all three grouped tile configurations), group
    ids in runs, lone tiles and out-of-range ids (whose rows keep the sentinel).
  * quantizers: 1x128 (ragged rows), 128x1 (ragged columns), the one-pass dual,
    128x128 with and without the transposed copy, and the FP8 re-quantizer, in
    BF16 and FP32, max-abs and power-of-two scales, on data whose magnitude
    varies from 2^-40 to 2^40 between cases.  Bar: bit-exact codes and scales.
"""

import os

import numpy as np
import pytest
import torch

from oracle import gemm as og, quant as oq
from tests.helpers import assert_bytes_equal, dev, host
from tests.helpers import require_gpu
from workloads import add_outliers, normal_f32, random_fp8_operands, to_bf16_bits

pytestmark = pytest.mark.gpu

TOL = 1e-3
TOL_F32 = 2e-4
KINDS = {"fprop": 0, "dgrad": 1, "wgrad": 2}
PATHS = {"promoted": 0, "pow2_a": 1, "pow2_b": 2, "pow2_ab": 3}
NAN_CODE = 0x7F
CODE_SENTINEL = 0xA5
OUT_SENTINEL = -7.5              # exact in BF16 and FP32
# FP8Q_GENERATED_ROUNDS=R draws R rounds of cases (round r from seeds shifted by r): a wider sweep on demand
ROUNDS = int(os.environ.get("FP8Q_GENERATED_ROUNDS", "1"))


def _draw_gemm_cases(n, rnd=0):
    rng = np.random.default_rng(20261203 + 7919 * rnd)
    cases = []
    for i in range(n):
        kind = ["fprop", "dgrad", "wgrad"][i % 3]
        path = list(PATHS)[(i // 3) % 4]
        out = ["bf16", "f32", "f32acc"][int(rng.integers(0, 3))]
        m, nn = (128 * int(v) for v in rng.integers(1, 17, size=2))
        k = 128 * int(rng.integers(1, 11))
        pads = tuple(16 * int(v) for v in rng.integers(0, 3, size=4))      # A offset, A pad, B offset, B pad
        cpad = tuple(int(v) for v in rng.integers(0, 3, size=2))           # C offset, pad in 16-byte units
        cases.append((1000 * rnd + i, kind, path, out, m, nn, k, pads, cpad))
    return cases


GEMM_CASES = [c for r in range(ROUNDS) for c in _draw_gemm_cases(48, r)]


def _case_id(c):
    i, kind, path, out, m, n, k, _, _ = c
    return f"{i}-{kind}-{path}-{out}-{m}x{n}x{k}"


def _guarded(shape, dtype, off, pad, fill):
    """A rows x cols view at column `off` of a buffer with `pad` more columns and
    one more row, everything filled with `fill`."""
    rows, cols = shape
    buf = torch.full((rows + 1, off + cols + pad), fill, dtype=dtype, device="cuda")
    return buf, buf[:rows, off:off + cols]


def _guarded_dense(shape, off, fill):
    """A dense float32 array of `shape` at element `off` (a multiple of 4) of a
    longer 1-D buffer filled with `fill`."""
    n = int(np.prod(shape))
    buf = torch.full((off + n + 4,), fill, dtype=torch.float32, device="cuda")
    return buf, buf[off:off + n].view(shape)


def _outside(buf_host, rows, off, cols):
    """The cells of a guarded buffer (host copy) outside its view."""
    mask = np.ones(buf_host.shape, dtype=bool)
    mask[:rows, off:off + cols] = False
    return buf_host[mask]


def _dense_outside(buf_host, off, n):
    return np.concatenate([buf_host[:off], buf_host[off + n:]])


def _sentinel_bits(dtype):
    t = torch.tensor([OUT_SENTINEL], dtype=dtype)
    return host(t)[0] if dtype == torch.bfloat16 else np.float32(OUT_SENTINEL)


def _put(view, arr):
    view.copy_(torch.from_numpy(np.ascontiguousarray(arr)).to(view.device))


def _gemm_operands(seed, kind, path, m, n, k):
    """Random codes; the scales of the operands the path hands to the MFMA are
    powers of two, the others arbitrary positive floats."""
    p2 = random_fp8_operands(seed, m, n, k, kind=kind, pow2=True)
    anyv = random_fp8_operands(seed, m, n, k, kind=kind, pow2=False)
    a_p2 = path in ("pow2_a", "pow2_ab")
    b_p2 = path in ("pow2_b", "pow2_ab")
    return {"qa": p2["qa"], "qb": p2["qb"], "sa": p2["sa"] if a_p2 else anyv["sa"],
            "sb": p2["sb"] if b_p2 else anyv["sb"]}


def _bf16_through_f32(got, want, f32):
    """BF16 output: the bar over the whole output, then per block through the
    FP32 result of the same call.  A 128x128 block's norm is often carried by a
    few large entries (full-range codes), and one of them lying close to a BF16
    rounding midpoint goes either way with the FP32 summation order: one BF16
    step (2^-8 to 2^-7 relative) on that entry, about 1e-3 on the block.  So the
    same GEMM with FP32 output (`f32`) is held to the FP32 bar on every block by
    the caller, and the BF16 output must be exactly its round-to-nearest-even
    (the epilogue rounds the same FP32 accumulators)."""
    assert og.rel_frobenius(got, want) <= TOL
    assert np.array_equal(got, og.round_bf16(f32)), "BF16 output is not the rounding of the FP32 result"


@pytest.mark.parametrize("case", GEMM_CASES, ids=_case_id)
def test_generated_gemm(case):
    fp8q = require_gpu()
    i, kind, path, out, m, n, k, (a_off, a_pad, b_off, b_pad), (c_off16, c_pad16) = case
    print(f"generated GEMM case {_case_id(case)}", flush=True)
    ops = _gemm_operands(9000 + i, kind, path, m, n, k)
    ref = og.gemm_ref(ops["qa"], ops["sa"], ops["qb"], ops["sb"], kind)

    abuf, a = _guarded((m, k), torch.uint8, a_off, a_pad, NAN_CODE)
    bbuf, b = _guarded((n, k), torch.uint8, b_off, b_pad, NAN_CODE)
    _put(a, ops["qa"])
    _put(b, ops["qb"])
    sabuf, sa = _guarded_dense(ops["sa"].shape, 4 * (i % 3), float("nan"))
    sbbuf, sb = _guarded_dense(ops["sb"].shape, 4 * ((i + 1) % 3), float("nan"))
    _put(sa, ops["sa"])
    _put(sb, ops["sb"])

    dt = torch.bfloat16 if out == "bf16" else torch.float32
    per16 = 16 // (2 if dt == torch.bfloat16 else 4)
    c_off, c_pad = per16 * c_off16, per16 * c_pad16
    cbuf, c = _guarded((m, n), dt, c_off, c_pad, OUT_SENTINEL)
    want = og.round_output(ref, "bf16" if out == "bf16" else "f32")
    if out == "f32acc":
        c0 = np.random.default_rng(9500 + i).standard_normal((m, n)).astype(np.float32)
        _put(c, c0)
        want = ref + c0.astype(np.float64)

    def call(cc, acc):
        args = (KINDS[kind], a, sa, b, sb)
        if path == "promoted":
            fp8q.fp8_gemm_blockscaled(*args, c=cc, accumulate=acc)
        else:
            fp8q.fp8_gemm_blockscaled_pow2(*args, c=cc, accumulate=acc, pow2_operands=PATHS[path])

    call(c, out == "f32acc")
    h = host(cbuf)
    outside = _outside(h, m, c_off, n)
    if dt == torch.bfloat16:
        assert np.all(outside == _sentinel_bits(dt)), "a write landed outside C"
        got = (h[:m, c_off:c_off + n].astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    else:
        assert np.all(outside == np.float32(OUT_SENTINEL)), "a write landed outside C"
        got = h[:m, c_off:c_off + n].astype(np.float64)
    assert np.all(np.isfinite(got)), "NaN in C: a read went outside an operand or its scales"
    if dt == torch.bfloat16:
        c32 = torch.full((m, n), OUT_SENTINEL, dtype=torch.float32, device="cuda")
        call(c32, False)
        f = host(c32).astype(np.float64)
        _bf16_through_f32(got, want, f)
        got, want = f, og.round_output(ref, "f32")
    for r in range(0, m, 128):
        for cc in range(0, n, 128):
            blk = (slice(r, r + 128), slice(cc, cc + 128))
            err = og.rel_frobenius(got[blk], want[blk])
            assert err <= TOL_F32, (r, cc, err)


def _draw_wide_cases(rnd=0):
    """M=512 and N = 256 * nt with nt in 129..192: 2*nt tiles of 256x256, more than the 256 CUs, with a last wave of
    2..128 tiles in whole 256-column bands, so the launch balances it: as K halves into scratch in C's head columns
    for BF16 output when the head has room (N_head >= 4 N_tail), else as a grid of 128x256 tiles."""
    rng = np.random.default_rng(20261206 + 7919 * rnd)
    cases = []
    for i in range(6):
        kind = ["fprop", "dgrad"][i % 2]
        path = list(PATHS)[(i // 2) % 4]
        out = ["bf16", "f32"][int(rng.integers(0, 2)) if i >= 2 else 0]
        nt = int(rng.integers(129, 193))
        k = 128 * int(rng.integers(2, 11))
        cases.append((1000 * rnd + i, kind, path, out, 512, 256 * nt, k, (0, 16, 16, 0), (1, 1)))
    return cases


WIDE_CASES = [c for r in range(ROUNDS) for c in _draw_wide_cases(r)]


@pytest.mark.parametrize("case", WIDE_CASES, ids=_case_id)
def test_generated_last_wave(case):
    """Like test_generated_gemm on shapes whose last wave is balanced: the whole output checked against the bar,
    every 256x256 tile to a bound a missing or misplaced tile cannot meet, FP32 results per tile to the FP32 bar,
    and nothing outside C written."""
    fp8q = require_gpu()
    i, kind, path, out, m, n, k, (a_off, a_pad, b_off, b_pad), (c_off16, c_pad16) = case
    print(f"generated last-wave case {_case_id(case)}", flush=True)
    ops = _gemm_operands(9600 + i, kind, path, m, n, k)
    ref = og.gemm_ref(ops["qa"], ops["sa"], ops["qb"], ops["sb"], kind)
    abuf, a = _guarded((m, k), torch.uint8, a_off, a_pad, NAN_CODE)
    bbuf, b = _guarded((n, k), torch.uint8, b_off, b_pad, NAN_CODE)
    _put(a, ops["qa"])
    _put(b, ops["qb"])
    sabuf, sa = _guarded_dense(ops["sa"].shape, 4, float("nan"))
    sbbuf, sb = _guarded_dense(ops["sb"].shape, 8, float("nan"))
    _put(sa, ops["sa"])
    _put(sb, ops["sb"])
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    per16 = 16 // (2 if dt == torch.bfloat16 else 4)
    c_off, c_pad = per16 * c_off16, per16 * c_pad16
    cbuf, c = _guarded((m, n), dt, c_off, c_pad, OUT_SENTINEL)
    args = (KINDS[kind], a, sa, b, sb)
    if path == "promoted":
        fp8q.fp8_gemm_blockscaled(*args, c=c)
    else:
        fp8q.fp8_gemm_blockscaled_pow2(*args, c=c, pow2_operands=PATHS[path])
    h = host(cbuf)
    sent = _sentinel_bits(dt) if dt == torch.bfloat16 else np.float32(OUT_SENTINEL)
    assert np.all(_outside(h, m, c_off, n) == sent), "a write landed outside C"
    view = h[:m, c_off:c_off + n]
    if dt == torch.bfloat16:
        got = (view.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
        want, tol_tile = og.round_bf16(ref), 4e-3
        assert og.rel_frobenius(got, want) <= TOL
    else:
        got, want, tol_tile = view.astype(np.float64), og.round_output(ref, "f32"), TOL_F32
    assert np.all(np.isfinite(got))
    for r in range(0, m, 256):
        for cc in range(0, n, 256):
            t = (slice(r, r + 256), slice(cc, cc + 256))
            assert og.rel_frobenius(got[t], want[t]) <= tol_tile, (r, cc)


def _draw_grouped_cases(rnd=0):
    rng = np.random.default_rng(20261204 + 7919 * rnd)
    cases = []
    for i, n in enumerate([128, 384, 256, 768, 512, 2048, 640, 1536, 1024, 896]):
        g = int(rng.integers(1, 6))
        k = 128 * int(rng.integers(1, 8))
        tiles_m = int(rng.integers(3, 40))
        runs = np.repeat(rng.integers(0, g, size=tiles_m), rng.integers(1, 5, size=tiles_m))[:tiles_m]
        gmap = runs.astype(np.int32)
        lone = rng.integers(0, tiles_m, size=3)
        gmap[lone] = rng.integers(0, g, size=3)
        skip = rng.integers(0, tiles_m, size=2)
        gmap[skip[0]] = -1
        gmap[skip[1]] = g                                    # both out of range
        out = ["bf16", "f32"][i % 2]
        cases.append((1000 * rnd + i, n, g, k, gmap, out, 16 * int(rng.integers(0, 3)),
                      16 * int(rng.integers(0, 3))))
    return cases


GROUPED_CASES = [c for r in range(ROUNDS) for c in _draw_grouped_cases(r)]


@pytest.mark.parametrize("case", GROUPED_CASES, ids=lambda c: f"{c[0]}-n{c[1]}-g{c[2]}-k{c[3]}-{c[5]}")
def test_generated_grouped(case):
    fp8q = require_gpu()
    i, n, g, k, gmap, out, a_off, a_pad = case
    print(f"generated grouped case {i}: n={n} g={g} k={k} tiles={gmap.size} {out}", flush=True)
    rng = np.random.default_rng(9700 + i)
    m = 128 * gmap.size
    ops = random_fp8_operands(9800 + i, m, n * g, k)
    qa, sa = ops["qa"], ops["sa"]
    qb = np.ascontiguousarray(ops["qb"].reshape(g, n, k))
    sb = np.exp2(rng.uniform(-10, -2, size=(g, n // 128, k // 128))).astype(np.float32)
    live = (gmap >= 0) & (gmap < g)
    ref = og.grouped_ref(qa, sa, qb, sb, np.where(live, gmap, 0))

    abuf, a = _guarded((m, k), torch.uint8, a_off, a_pad, NAN_CODE)
    _put(a, qa)
    sabuf, sa_d = _guarded_dense(sa.shape, 4, float("nan"))
    _put(sa_d, sa)
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    per16 = 16 // (2 if dt == torch.bfloat16 else 4)
    c_off = per16 * (i % 3)
    cbuf, c = _guarded((m, n), dt, c_off, per16, OUT_SENTINEL)
    fp8q.fp8_gemm_blockscaled_grouped(dev(gmap), a, sa_d, dev(qb), dev(sb), c=c)

    h = host(cbuf)
    sent = _sentinel_bits(dt)
    assert np.all(_outside(h, m, c_off, n) == sent), "a write landed outside C"
    view = h[:m, c_off:c_off + n]
    if dt == torch.bfloat16:
        got = (view.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
        c32 = torch.full((m, n), OUT_SENTINEL, dtype=torch.float32, device="cuda")
        fp8q.fp8_gemm_blockscaled_grouped(dev(gmap), a, sa_d, dev(qb), dev(sb), c=c32)
        f = host(c32).astype(np.float64)
        on = np.repeat(live, 128)
        _bf16_through_f32(got[on], og.round_bf16(ref)[on], f[on])
        got = f
    else:
        got = view.astype(np.float64)
    want = og.round_output(ref, "f32")
    for t in range(gmap.size):
        rows = slice(128 * t, 128 * (t + 1))
        if not live[t]:
            assert np.all(view[rows] == sent), f"tile {t} (group id {gmap[t]}) should be skipped"
            continue
        assert np.all(np.isfinite(got[rows])), t
        for cc in range(0, n, 128):
            err = og.rel_frobenius(got[rows, cc:cc + 128], want[rows, cc:cc + 128])
            assert err <= TOL_F32, (t, cc, err)


# ----------------------------------------------------------------------------
# Quantizers
# ----------------------------------------------------------------------------

def _draw_quant_cases(rnd=0):
    rng = np.random.default_rng(20261205 + 7919 * rnd)
    cases = []
    ops = ["1x128", "128x1", "dual", "block", "block_t", "requant"]
    for i in range(48):
        op = ops[i % len(ops)]
        dtype = ["bf16", "f32"][(i // len(ops)) % 2]
        mode = ["maxabs", "pow2"][int(rng.integers(0, 2))]
        if op == "1x128":
            rows, cols = int(rng.integers(1, 700)), 128 * int(rng.integers(1, 13))
        elif op == "128x1":
            rows, cols = 128 * int(rng.integers(1, 7)), 8 * int(rng.integers(1, 200))
        else:
            rows, cols = 128 * int(rng.integers(1, 7)), 128 * int(rng.integers(1, 9))
        if op == "block" and dtype == "bf16" and i < 20:
            cols = 256 * int(rng.integers(1, 5))            # the two-block kernel for BF16 weights
        expo = int(rng.integers(-40, 41))
        offs = tuple(int(v) for v in rng.integers(0, 3, size=4))  # x offset, x pad, out offset, out pad (16 B)
        cases.append((1000 * rnd + i, op, dtype, mode, rows, cols, expo, offs))
    return cases


QUANT_CASES = [c for r in range(ROUNDS) for c in _draw_quant_cases(r)]
MODE_CODE = {"maxabs": 0, "pow2": 1}


def _qdata(seed, shape, expo):
    rng = np.random.default_rng(seed)
    x = add_outliers(rng, normal_f32(rng, shape, 1.0), 0.01, 100.0) * np.float32(2.0 ** expo)
    x[rng.random(shape) < 0.002] = 0.0
    return x.astype(np.float32)


def _input_view(x_f32, dtype, off16, pad16):
    """The input as a strided view (NaN around it) and the float32 values the oracle sees."""
    rows, cols = x_f32.shape
    if dtype == "bf16":
        bits = to_bf16_bits(x_f32)
        buf, v = _guarded((rows, cols), torch.bfloat16, 8 * off16, 8 * pad16, float("nan"))
        v.copy_(torch.from_numpy(bits.view(np.int16)).to(v.device).view(torch.bfloat16))
        return v, oq.bf16_bits_to_f32(bits)
    buf, v = _guarded((rows, cols), torch.float32, 4 * off16, 4 * pad16, float("nan"))
    _put(v, x_f32)
    return v, x_f32


class _Out:
    """A guarded code output (strided view) or scale output (dense view)."""

    def __init__(self, shape, codes, off16, pad16, slot):
        self.shape, self.codes = shape, codes
        if codes:
            self.off = 16 * off16
            self.buf, self.view = _guarded(shape, torch.uint8, self.off, 16 * pad16, CODE_SENTINEL)
        else:
            self.off = 4 * slot
            self.buf, self.view = _guarded_dense(shape, self.off, OUT_SENTINEL)

    def check(self, want, what):
        h = host(self.buf)
        if self.codes:
            rows, cols = self.shape
            assert np.all(_outside(h, rows, self.off, cols) == CODE_SENTINEL), f"{what}: write outside the view"
            assert_bytes_equal(h[:rows, self.off:self.off + cols], want, what)
        else:
            n = int(np.prod(self.shape))
            assert np.all(_dense_outside(h, self.off, n) == np.float32(OUT_SENTINEL)), f"{what}: write outside"
            assert_bytes_equal(h[self.off:self.off + n].reshape(self.shape), want, what)


def _cdiv(a, b):
    return -(-a // b)


@pytest.mark.parametrize("case", QUANT_CASES, ids=lambda c: f"{c[0]}-{c[1]}-{c[2]}-{c[3]}-{c[4]}x{c[5]}")
def test_generated_quantizer(case):
    fp8q = require_gpu()
    i, op, dtype, mode, rows, cols, expo, (xo, xp, oo, op16) = case
    print(f"generated quantizer case {i}: {op} {dtype} {mode} {rows}x{cols} 2^{expo}", flush=True)
    x = _qdata(9900 + i, (rows, cols), expo)
    mc = MODE_CODE[mode]

    if op == "requant":
        q_in, s_in = oq.quant_1x128(x, "pow2" if i % 2 else "maxabs")
        qbuf, qv = _guarded((rows, cols), torch.uint8, 16 * xo, 16 * xp, NAN_CODE)
        _put(qv, q_in)
        sbuf, sv = _guarded_dense(s_in.shape, 4, float("nan"))
        _put(sv, s_in)
        qt = _Out((cols, rows), True, oo, op16, 0)
        st = _Out((rows // 128, cols), False, 0, 0, 1)
        fp8q.fp8_requant_1x128_to_128x1(qv, sv, mc, q_t=qt.view, scales_t=st.view)
        qt_ref, st_ref = oq.requant_1x128_to_128x1(q_in, s_in, mode)
        qt.check(qt_ref, "transposed codes")
        st.check(st_ref, "128x1 scales")
        return

    xv, x_ref = _input_view(x, dtype, xo, xp)
    if op == "1x128":
        q = _Out((rows, cols), True, oo, op16, 0)
        s = _Out((cols // 128, rows), False, 0, 0, 2)
        fp8q.fp8_quant_tile(xv, fp8q.TILE_1x128, mc, q=q.view, scales=s.view)
        q_ref, s_ref = oq.quant_1x128(x_ref, mode)
        q.check(q_ref, "1x128 codes")
        s.check(s_ref, "1x128 scales")
    elif op == "128x1":
        q = _Out((cols, rows), True, oo, op16, 0)
        s = _Out((rows // 128, cols), False, 0, 0, 1)
        fp8q.fp8_quant_tile(xv, fp8q.TILE_128x1, mc, q=q.view, scales=s.view)
        q_ref, s_ref = oq.quant_128x1(x_ref, mode)
        q.check(q_ref, "128x1 codes")
        s.check(s_ref, "128x1 scales")
    elif op == "dual":
        q = _Out((rows, cols), True, oo, op16, 0)
        s = _Out((cols // 128, rows), False, 0, 0, 1)
        qt = _Out((cols, rows), True, op16, oo, 0)
        st = _Out((rows // 128, cols), False, 0, 0, 2)
        fp8q.fp8_quant_tile_dual(xv, mc, q=q.view, scales=s.view, q_t=qt.view, scales_t=st.view)
        q_ref, s_ref = oq.quant_1x128(x_ref, mode)
        qt_ref, st_ref = oq.quant_128x1(x_ref, mode)
        q.check(q_ref, "1x128 codes")
        s.check(s_ref, "1x128 scales")
        qt.check(qt_ref, "128x1 codes")
        st.check(st_ref, "128x1 scales")
    else:
        q = _Out((rows, cols), True, oo, op16, 0)
        s = _Out((rows // 128, cols // 128), False, 0, 0, 1)
        q_ref, s_ref = oq.quant_128x128(x_ref, mode)
        if op == "block":
            fp8q.fp8_quant_block(xv, mc, False, q=q.view, scales=s.view)
        else:
            qt = _Out((cols, rows), True, op16, oo, 0)
            st = _Out((cols // 128, rows // 128), False, 0, 0, 2)
            fp8q.fp8_quant_block(xv, mc, True, q=q.view, scales=s.view, q_t=qt.view, scales_t=st.view)
            qt.check(np.ascontiguousarray(q_ref.T), "transposed block codes")
            st.check(np.ascontiguousarray(s_ref.T), "transposed block scales")
        q.check(q_ref, "block codes")
        s.check(s_ref, "block scales")
