"""Pins for the oracle's 1x128, 128x1 and 128x128 quantizers (CPU only).

What pins them (none of it retypes the oracle's own formulas):
  * max-abs mode: every tile/block whose max-abs clears the floor has
    max |dec(q)| == 448 exactly (the max-abs is mapped to the FP8 maximum);
  * pow2 mode: s is an integral power of two with a/s in (224, 448], so the
    largest code is in [224, 448]; max-abs and pow2 agree when a/448 is a
    power of two;
  * representable inputs round-trip exactly (pow2 scales make s*dec(q) == x);
  * a closed-form error bound holds for every element;
  * 128x1 == transpose of 1x128 on the transposed input, and block
    quantization commutes with transposition;
  * constant tiles give s = fl(c/448) and all codes at +-448;
  * hand-worked tiles in tests/golden/worked_examples.json;
  * a brute-force per-element loop on a tiny ragged tensor.
"""

import json
import os

import numpy as np
import pytest

from oracle import e4m3, quant
from workloads import add_outliers, normal_f32, tiny_fprop

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")
MODES = [quant.MODE_MAXABS, quant.MODE_POW2]


def _outlier_data(seed, shape, sigma=1.0, frac=0.01, factor=100.0):
    rng = np.random.default_rng(seed)
    return add_outliers(rng, normal_f32(rng, shape, sigma), frac, factor)


def _maxdec_1x128(q):
    r, c = q.shape
    d = np.abs(e4m3.decode(q))
    pad = (-c) % 128
    d = np.pad(d, ((0, 0), (0, pad)))
    return d.reshape(r, -1, 128).max(axis=2)            # [r][g]


def test_maxabs_maps_each_tile_max_to_448():
    x = _outlier_data(1, (64, 640))
    x[3, 128:256] = 0.0                                   # a zero tile
    q, s = quant.quant_1x128(x, quant.MODE_MAXABS)
    m = _maxdec_1x128(q)
    nz = np.abs(x).reshape(64, 5, 128).max(axis=2) > 0
    assert np.all(m[nz] == 448.0)
    assert np.all(m[~nz] == 0.0)


def test_pow2_scale_properties():
    x = _outlier_data(2, (64, 512))
    x[5] *= 2.0 ** 40
    x[6] *= 2.0 ** -40
    q, s = quant.quant_1x128(x, quant.MODE_POW2)
    mant, _ = np.frexp(s.astype(np.float64))
    assert np.all(mant == 0.5)                            # s is a power of two
    amax = np.abs(x.astype(np.float64)).reshape(64, 4, 128).max(axis=2).T   # [g][r]
    ratio = amax / s
    assert np.all(ratio > 224.0) and np.all(ratio <= 448.0)
    m = _maxdec_1x128(q).T
    assert np.all(m >= 224.0) and np.all(m <= 448.0)


def test_pow2_and_maxabs_agree_when_amax_over_448_is_power_of_two():
    rng = np.random.default_rng(3)
    x = rng.uniform(-1, 1, size=(16, 256)).astype(np.float32)
    for r in range(16):                                   # force max-abs = 448 * 2^k
        for g in range(2):
            seg = x[r, g * 128:(g + 1) * 128]
            seg /= np.abs(seg).max()
            seg *= np.float32(448.0 * 2.0 ** (r - 8))
    qa, sa = quant.quant_1x128(x, quant.MODE_MAXABS)
    qp, sp = quant.quant_1x128(x, quant.MODE_POW2)
    assert np.array_equal(qa, qp) and np.array_equal(sa, sp)


def test_representable_round_trip_pow2():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 0x7F, size=(8, 256)).astype(np.uint8)
    codes[:, ::128] = 0x7E                                # max 448 in each tile
    codes |= (rng.integers(0, 2, size=codes.shape) << 7).astype(np.uint8)
    k = rng.integers(-20, 20, size=(8, 2))
    scale = np.repeat(np.ldexp(1.0, k), 128, axis=1)
    x = (e4m3.decode(codes) * scale).astype(np.float32)
    q, s = quant.quant_1x128(x, quant.MODE_POW2)
    back = quant.dequant_1x128(q, s)
    assert np.array_equal(back, x.astype(np.float64))
    assert np.array_equal(q, codes)


def test_representable_round_trip_maxabs_unit_scale():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 0x7F, size=(4, 128)).astype(np.uint8)
    codes[:, 7] = 0x7E
    x = e4m3.decode(codes).astype(np.float32)
    q, s = quant.quant_1x128(x, quant.MODE_MAXABS)
    assert np.all(s == 1.0)
    assert np.array_equal(q, codes)


@pytest.mark.parametrize("mode", MODES)
def test_elementwise_error_bound(mode):
    x = _outlier_data(6, (32, 384), frac=0.02, factor=1000.0)
    q, s = quant.quant_1x128(x, mode)
    srep = np.repeat(s.T.astype(np.float64), 128, axis=1)
    deq = e4m3.decode(q) * srep
    y = np.abs(x.astype(np.float64)) / srep               # ideal scaled magnitude
    ulp = np.where(y >= 2.0 ** -6, np.ldexp(1.0, np.floor(np.log2(np.maximum(y, 2.0 ** -6))).astype(int) - 3), 2.0 ** -9)
    bound = srep * 0.5 * ulp * (1 + 2.0 ** -20) + 2.0 ** -21 * np.abs(x)
    assert np.all(np.abs(x - deq) <= bound)


@pytest.mark.parametrize("mode", MODES)
def test_128x1_is_transposed_1x128(mode):
    x = _outlier_data(7, (384, 200))
    qt, s = quant.quant_128x1(x, mode)
    q2, s2 = quant.quant_1x128(np.ascontiguousarray(x.T), mode)
    assert qt.shape == (200, 384) and s.shape == (3, 200)
    assert np.array_equal(qt, q2) and np.array_equal(s, s2)


@pytest.mark.parametrize("mode", MODES)
def test_block_quant_commutes_with_transpose(mode):
    w = _outlier_data(8, (256, 384), sigma=0.02)
    q, s = quant.quant_128x128(w, mode)
    qt, st = quant.quant_128x128(np.ascontiguousarray(w.T), mode)
    assert np.array_equal(q.T, qt) and np.array_equal(s.T, st)


def test_block_scale_is_block_max():
    w = _outlier_data(9, (256, 384), sigma=0.02)
    q, s = quant.quant_128x128(w, quant.MODE_MAXABS)
    d = np.abs(e4m3.decode(q)).reshape(2, 128, 3, 128).max(axis=(1, 3))
    assert np.all(d == 448.0)
    amax = np.abs(w).reshape(2, 128, 3, 128).max(axis=(1, 3))
    assert np.array_equal(s, (amax / np.float32(448.0)).astype(np.float32))


def test_constant_tiles():
    c = np.float32(0.02)
    x = np.full((4, 256), c, dtype=np.float32)
    x[1] *= -1
    q, s = quant.quant_1x128(x, quant.MODE_MAXABS)
    assert np.all(s == np.float32(c / np.float32(448.0)))
    assert np.all(q[0] == 0x7E) and np.all(q[1] == 0xFE)
    qb, sb = quant.quant_128x128(np.full((128, 128), -c, np.float32), quant.MODE_MAXABS)
    assert np.all(qb == 0xFE) and sb.shape == (1, 1)


def test_zero_and_tiny_tiles():
    x = np.zeros((2, 128), np.float32)
    x[1, 5] = np.float32(1e-40)                           # float32 subnormal max-abs
    q, s = quant.quant_1x128(x, quant.MODE_MAXABS)
    assert np.all(s == np.float32(2.0 ** -126))
    assert np.all(q[0] == 0)
    # float32(1e-40) = 71362 * 2^-149; times inv = 2^126 gives 71362 * 2^-23 = 4.355 * 2^-9,
    # which rounds to the subnormal code 4.
    assert q[1, 5] == 0x04
    qp, sp = quant.quant_1x128(x, quant.MODE_POW2)
    assert np.all(sp == np.float32(2.0 ** -126))


def test_golden_tiles():
    cases = json.load(open(GOLDEN))["tile_cases"]
    for c in cases:
        x = np.zeros((1, 128), np.uint32)
        for i, h in c["x"].items():
            x[0, int(i)] = int(h, 16)
        q, s = quant.quant_1x128(x.view(np.float32), c["mode"])
        assert int(s.view(np.uint32)[0, 0]) == int(c["scale"], 16), c["why"]
        for i, h in c["codes"].items():
            assert int(q[0, int(i)]) == int(h, 16), (c["why"], i)


def _brute_force_1x128(x, mode):
    """Per-element loops over a tiny ragged tensor, one tile at a time."""
    r, cols = x.shape
    ng = -(-cols // 128)
    q = np.zeros((r, cols), np.uint8)
    s = np.zeros((ng, r), np.float32)
    for i in range(r):
        for g in range(ng):
            lo, hi = g * 128, min(cols, (g + 1) * 128)
            amax = np.float32(0.0)
            for j in range(lo, hi):
                amax = max(amax, np.float32(abs(x[i, j])))
            si, inv = quant.scales_from_amax(np.array([amax]), mode)
            s[g, i] = si[0]
            for j in range(lo, hi):
                q[i, j] = e4m3.encode(np.array([np.float32(x[i, j]) * inv[0]], np.float32))[0]
    return q, s


@pytest.mark.parametrize("mode", MODES)
def test_ragged_tensor_against_per_element_loops(mode):
    x = _outlier_data(10, (3, 300))
    q, s = quant.quant_1x128(x, mode)
    qb, sb = _brute_force_1x128(x, mode)
    assert np.array_equal(q, qb) and np.array_equal(s, sb)
    qt, st = quant.quant_128x1(np.ascontiguousarray(x.T), mode)
    assert np.array_equal(qt, q) and np.array_equal(st, s)


def test_ragged_blocks_cover_only_present_elements():
    w = _outlier_data(11, (200, 130), sigma=0.02)
    q, s = quant.quant_128x128(w, quant.MODE_MAXABS)
    assert s.shape == (2, 2)
    for bi in range(2):
        for bj in range(2):
            blk = w[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            a = np.float32(np.abs(blk).max())
            assert s[bi, bj] == np.float32(a / np.float32(448.0))
            assert np.abs(e4m3.decode(q[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128])).max() == 448.0


def test_tiny_config_quantization_shapes():
    d = tiny_fprop()
    qa, sa = quant.quant_1x128(d["a"])
    qb, sb = quant.quant_128x128(d["bt"])
    assert qa.shape == (128, 256) and sa.shape == (2, 128)
    assert qb.shape == (128, 256) and sb.shape == (1, 2)


# ---------------------------------------------------------------------------
# FP8 -> FP8 1x128 -> 128x1 re-quantization (dssusan.co.kr FP8 excerpt,
# paragraph 4 for the conversion, paragraph 1 for its power-of-2 scales).
# ---------------------------------------------------------------------------

def _codes_with_big_entry_per_column_tile(seed, r, c):
    """Random finite codes where every 128x1 column tile holds one |dec| in (224, 448]."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 256, size=(r, c), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] ^= 0x01                           # no NaN codes
    q[(q & 0x7F) > 0x77] &= 0xF7                            # |dec| <= 224 everywhere ...
    for g in range(r // 128):
        rows = g * 128 + rng.integers(0, 128, size=c)
        q[rows, np.arange(c)] = rng.choice([0x78, 0x7A, 0x7E, 0xF9, 0xFE], size=c)   # ... but one > 224
    return q


def test_requant_is_lossless_when_row_scales_align():
    # Every row scale 2^e and every column tile reaching (224, 448]*2^e: the
    # 128x1 tiles get the same scale 2^e and the codes come back unchanged,
    # only transposed (pow2 scales make the re-quantization exact).
    r, c = 256, 384
    q = _codes_with_big_entry_per_column_tile(11, r, c)
    for e in (-20, 0, 7):
        s = np.full((c // 128, r), 2.0 ** e, dtype=np.float32)
        qt, st = quant.requant_1x128_to_128x1(q, s, quant.MODE_POW2)
        assert np.array_equal(qt, q.T)
        assert np.all(st == np.float32(2.0 ** e))


@pytest.mark.parametrize("mode", MODES)
def test_requant_scale_covariance(mode):
    # Multiplying every input scale by 2^j multiplies every output scale by
    # 2^j and leaves the codes alone (both scale rules are invariant under
    # exact power-of-two rescaling away from under/overflow).
    x = _outlier_data(12, (256, 256))
    q, s = quant.quant_1x128(x, mode)
    qt0, st0 = quant.requant_1x128_to_128x1(q, s, mode)
    for j in (-9, 5):
        qt1, st1 = quant.requant_1x128_to_128x1(q, (s * np.float32(2.0 ** j)).astype(np.float32), mode)
        assert np.array_equal(qt1, qt0)
        assert np.array_equal(st1, (st0 * np.float32(2.0 ** j)).astype(np.float32))


def test_requant_maxabs_maps_column_max_to_448():
    x = _outlier_data(13, (256, 384))
    q, s = quant.quant_1x128(x, quant.MODE_POW2)
    qt, st = quant.requant_1x128_to_128x1(q, s, quant.MODE_MAXABS)
    d = np.abs(e4m3.decode(qt)).reshape(384, 2, 128).max(axis=2)
    xh = np.abs(e4m3.decode(q) * np.repeat(s.T, 128, axis=1)).T.reshape(384, 2, 128).max(axis=2)
    assert np.all(d[xh > 0] == 448.0)


@pytest.mark.parametrize("mode", MODES)
def test_requant_error_bound_against_source(mode):
    # Two roundings, each at most half an E4M3 step of its own tile:
    # |dec(q')s' - x| <= |dec(q)s - x| + 2^-4 |xh| + 2^-10 s'  (E4M3 keeps 3
    # mantissa bits; the subnormal step is 2^-9 of the tile scale).
    x = _outlier_data(14, (256, 256))
    q, s = quant.quant_1x128(x, quant.MODE_POW2)
    xh = quant.dequant_1x128(q, s)
    qt, st = quant.requant_1x128_to_128x1(q, s, mode)
    back = e4m3.decode(qt).T * np.repeat(st.astype(np.float64), 128, axis=0)
    bound = np.abs(xh - x) + np.abs(xh) * 2.0 ** -4 + np.repeat(st.astype(np.float64), 128, axis=0) * 2.0 ** -10
    assert np.all(np.abs(back - x) <= bound)


def test_requant_rejects_wrong_scale_shape_and_nan_codes():
    q = np.zeros((128, 256), dtype=np.uint8)
    with pytest.raises(ValueError):
        quant.requant_1x128_to_128x1(q, np.ones((1, 128), np.float32))
    q[5, 7] = 0x7F
    with pytest.raises(ValueError):
        quant.requant_1x128_to_128x1(q, np.ones((2, 128), np.float32))
