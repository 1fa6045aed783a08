"""GPU parity of the HIP quantizers against the CPU oracle: bit-exact FP8 bytes
and FP32 scales, through the C ABI.

Small cases cover several tiles and a ragged tail; edge cases sweep every
BF16 value in range and every float32 value around each E4M3 rounding
midpoint through the hardware converter; the full-size cases run the
quantizer-only workload (activation 8192x7168, weight 18432x7168) and the
Dgrad/Wgrad operands at their real shapes and check sampled rows/columns that
the oracle recomputes.
"""

import numpy as np
import pytest
import torch

from oracle import e4m3, quant as oq
from tests.helpers import assert_bytes_equal, dev, dev_bf16, host, require_gpu
from workloads import add_outliers, linear_layer, normal_f32, output_grad, to_bf16_bits

pytestmark = pytest.mark.gpu

MODES = [("maxabs", 0), ("pow2", 1)]


def _data(seed, shape, sigma=1.0, frac=0.01, factor=100.0):
    rng = np.random.default_rng(seed)
    return add_outliers(rng, normal_f32(rng, shape, sigma), frac, factor)


def _to_dev(x_f32, dtype):
    """Device tensor plus the exact float32 values the oracle must see."""
    if dtype == "bf16":
        bits = to_bf16_bits(x_f32)
        return dev_bf16(bits), oq.bf16_bits_to_f32(bits)
    return dev(x_f32), x_f32


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode_name,mode", MODES)
@pytest.mark.parametrize("shape", [(128, 256), (37, 384), (1, 128), (300, 1024)])
def test_quant_1x128(dtype, mode_name, mode, shape):
    fp8q = require_gpu()
    x_dev, x_ref = _to_dev(_data(hash(shape) % 1000, shape), dtype)
    q, s = fp8q.fp8_quant_tile(x_dev, fp8q.TILE_1x128, mode)
    q_ref, s_ref = oq.quant_1x128(x_ref, mode_name)
    assert_bytes_equal(host(q), q_ref, "codes")
    assert_bytes_equal(host(s), s_ref, "scales")


def _edge_tensor_f32():
    """Rows whose first element is 448*2^k (so inv = 2^-k exactly) followed by
    127 values that sweep the converter's rounding cases."""
    mags = e4m3.decode(np.arange(0x7F, dtype=np.uint8))
    mids = (0.5 * (mags[:-1] + mags[1:])).astype(np.float32)
    pts = np.concatenate([mags.astype(np.float32), mids])
    bits = pts.view(np.int32).astype(np.int64)[:, None] + np.arange(-3, 4)[None, :]
    sweep = bits.reshape(-1)
    sweep = sweep[sweep >= 0].astype(np.int32).view(np.float32)
    sweep = sweep[np.abs(sweep) <= 448.0]
    sweep = np.concatenate([sweep, -sweep, np.array([0.0, -0.0, 1e-45, -1e-45, 1e-39, -1e-39], np.float32)])
    n_rows = -(-sweep.size // 127)
    sweep = np.concatenate([sweep, np.zeros(n_rows * 127 - sweep.size, np.float32)])
    body = sweep.reshape(n_rows, 127)
    rows = []
    for k in (0, -3, 5):
        head = np.full((n_rows, 1), np.float32(448.0 * 2.0 ** k))
        rows.append(np.concatenate([head, body * np.float32(2.0 ** k)], axis=1))
    special = np.zeros((6, 128), np.float32)
    special[1, :] = -0.0                             # all negative zeros
    special[2, 3] = np.float32(1e-40)                # subnormal max-abs
    special[3, :] = np.float32(-0.02)                # constant tile
    special[4, 0] = np.float32(3e38)                 # near FP32 max
    special[4, 1:] = np.float32(1e30)
    special[5, 0] = np.float32(3.6)                  # pow2 rounds the exponent up
    return np.concatenate(rows + [special], axis=0).astype(np.float32)


@pytest.mark.parametrize("mode_name,mode", MODES)
def test_quant_1x128_edge_values_f32(mode_name, mode):
    fp8q = require_gpu()
    x = _edge_tensor_f32()
    q, s = fp8q.fp8_quant_tile(dev(x), fp8q.TILE_1x128, mode)
    q_ref, s_ref = oq.quant_1x128(x, mode_name)
    assert_bytes_equal(host(s), s_ref, "scales")
    assert_bytes_equal(host(q), q_ref, "codes")


@pytest.mark.parametrize("mode_name,mode", MODES)
def test_quant_1x128_every_bf16_pattern(mode_name, mode):
    """All 65536 BF16 patterns that are finite, arranged 127 per tile behind a
    448 (max-abs 448 -> unit scale) and behind 448*2^-20."""
    fp8q = require_gpu()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oq.bf16_bits_to_f32(bits)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448.0)
    bits = bits[keep]
    n_rows = -(-bits.size // 127)
    bits = np.concatenate([bits, np.zeros(n_rows * 127 - bits.size, np.uint16)]).reshape(n_rows, 127)
    head = np.full((n_rows, 1), 0x43E0, np.uint16)                 # 448.0 in BF16
    x_bits = np.concatenate([head, bits], axis=1)
    # second copy scaled by 2^-20 (exact in BF16 for normal values; tiny ones flush as BF16 would not)
    small = oq.bf16_bits_to_f32(x_bits) * np.float32(2.0 ** -20)
    x_bits = np.concatenate([x_bits, to_bf16_bits(small)], axis=0)
    q, s = fp8q.fp8_quant_tile(dev_bf16(x_bits), fp8q.TILE_1x128, mode)
    q_ref, s_ref = oq.quant_1x128(oq.bf16_bits_to_f32(x_bits), mode_name)
    assert_bytes_equal(host(s), s_ref, "scales")
    assert_bytes_equal(host(q), q_ref, "codes")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode_name,mode", MODES)
@pytest.mark.parametrize("shape", [(128, 8), (256, 200), (384, 64), (128, 1000), (256, 512), (384, 264)])
def test_quant_128x1(dtype, mode_name, mode, shape):
    """Column counts that end in a partial 64-column tile (200, 1000, 264) and ones that do not."""
    fp8q = require_gpu()
    x_dev, x_ref = _to_dev(_data(7 + shape[1], shape), dtype)
    qt, s = fp8q.fp8_quant_tile(x_dev, fp8q.TILE_128x1, mode)
    qt_ref, s_ref = oq.quant_128x1(x_ref, mode_name)
    assert_bytes_equal(host(qt), qt_ref, "transposed codes")
    assert_bytes_equal(host(s), s_ref, "scales")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode_name,mode", MODES)
@pytest.mark.parametrize("shape", [(128, 128), (256, 384), (384, 256), (256, 1024)])
def test_quant_block(dtype, mode_name, mode, shape):
    fp8q = require_gpu()
    x_dev, x_ref = _to_dev(_data(11 + shape[0], shape, sigma=0.02), dtype)
    q, s, qt, st = fp8q.fp8_quant_block(x_dev, mode, transposed=True)
    q_ref, s_ref = oq.quant_128x128(x_ref, mode_name)
    assert_bytes_equal(host(q), q_ref, "codes")
    assert_bytes_equal(host(s), s_ref, "scales")
    assert_bytes_equal(host(qt), np.ascontiguousarray(q_ref.T), "transposed codes")
    assert_bytes_equal(host(st), np.ascontiguousarray(s_ref.T), "transposed scales")
    # without the transposed copy (BF16 with cols % 256 == 0 runs the two-block kernel)
    q2, s2 = fp8q.fp8_quant_block(x_dev, mode, transposed=False)
    assert_bytes_equal(host(q2), q_ref, "codes without the transposed copy")
    assert_bytes_equal(host(s2), s_ref, "scales without the transposed copy")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode_name,mode", MODES)
def test_degenerate_groups_128x1_and_blocks(dtype, mode_name, mode):
    """All-zero, negative-zero, constant, lone-subnormal-max and near-FP32-max groups in the 128x1 and the
    128x128 quantizers (the scale floor and the extremes of the scale derivation)."""
    fp8q = require_gpu()
    x = _data(41, (256, 768))
    x[0:128, 0:128] = 0.0                            # a 128x128 block and 128 columns of 128x1 groups: zero
    x[128:256, 0:128] = -0.0
    x[0:128, 128:256] = np.float32(-0.02)            # constant
    x[128:256, 128:256] = 0.0
    x[130, 200] = np.float32(1e-40)                  # lone FP32 subnormal as max-abs (flushes in BF16)
    x[0:128, 256:384] = np.float32(1e30)             # near the top of the FP32 range
    x[5, 300] = np.float32(3e38)
    x_dev, x_ref = _to_dev(x, dtype)
    qt, st = fp8q.fp8_quant_tile(x_dev, fp8q.TILE_128x1, mode)
    qt_ref, st_ref = oq.quant_128x1(x_ref, mode_name)
    assert_bytes_equal(host(st), st_ref, "128x1 scales")
    assert_bytes_equal(host(qt), qt_ref, "128x1 codes")
    q, s, q_t, s_t = fp8q.fp8_quant_block(x_dev, mode, transposed=True)
    q_ref, s_ref = oq.quant_128x128(x_ref, mode_name)
    assert_bytes_equal(host(s), s_ref, "block scales")
    assert_bytes_equal(host(q), q_ref, "block codes")
    assert_bytes_equal(host(q_t), q_ref.T, "transposed block codes")
    assert_bytes_equal(host(s_t), s_ref.T, "transposed block scales")
    # the same blocks without the transposed copy: 768 columns, so BF16 input
    # takes the two-block (128x256 per workgroup) kernel, each degenerate
    # block in either half of a pair
    for cols in (slice(0, 768), slice(128, 640)):
        xs = x_dev[:, cols]
        q2, s2 = fp8q.fp8_quant_block(xs, mode, transposed=False)
        q2_ref, s2_ref = oq.quant_128x128(x_ref[:, cols], mode_name)
        assert_bytes_equal(host(s2), s2_ref, f"block scales, no copy, columns {cols}")
        assert_bytes_equal(host(q2), q2_ref, f"block codes, no copy, columns {cols}")


def test_quant_strided_input_and_outputs():
    """Leading dimensions larger than the logical width (a column slice)."""
    fp8q = require_gpu()
    full = _data(5, (256, 512))
    bits = to_bf16_bits(full)
    x_dev = dev_bf16(bits)[:, 128:384]                       # ld 512, width 256
    q_store = torch.zeros((256, 320), dtype=torch.uint8, device="cuda")
    q, s = fp8q.fp8_quant_tile(x_dev, fp8q.TILE_1x128, 0, q=q_store[:, :256])
    q_ref, s_ref = oq.quant_1x128(oq.bf16_bits_to_f32(bits[:, 128:384]), "maxabs")
    assert_bytes_equal(host(q_store)[:, :256], q_ref, "codes")
    assert np.all(host(q_store)[:, 256:] == 0)
    assert_bytes_equal(host(s), s_ref, "scales")


def test_quant_128x1_strided_input_and_output():
    """128x1 on a column slice of a wider matrix, transposed codes into a wider buffer."""
    fp8q = require_gpu()
    full = _data(6, (256, 768))
    bits = to_bf16_bits(full)
    x_dev = dev_bf16(bits)[:, 128:648]                       # ld 768, width 520
    qt_store = torch.zeros((520, 288), dtype=torch.uint8, device="cuda")
    qt, s = fp8q.fp8_quant_tile(x_dev, fp8q.TILE_128x1, 0, q=qt_store[:, :256])
    qt_ref, s_ref = oq.quant_128x1(oq.bf16_bits_to_f32(bits[:, 128:648]), "maxabs")
    assert_bytes_equal(host(qt_store)[:, :256], qt_ref, "transposed codes")
    assert np.all(host(qt_store)[:, 256:] == 0)
    assert_bytes_equal(host(s), s_ref, "scales")


def test_quantizers_deterministic():
    fp8q = require_gpu()
    x_dev, _ = _to_dev(_data(3, (512, 1024)), "bf16")
    a = [host(t) for t in fp8q.fp8_quant_tile(x_dev, fp8q.TILE_1x128, 0)]
    b = [host(t) for t in fp8q.fp8_quant_tile(x_dev, fp8q.TILE_1x128, 0)]
    assert all(np.array_equal(u, v) for u, v in zip(a, b))


# ----------------------------------------------------------------------------
# Full-size workloads, checked on sampled rows / columns / bands.
# ----------------------------------------------------------------------------

@pytest.fixture(scope="module")
def layer():
    d = linear_layer()
    return d, dev_bf16(d["x"]), dev_bf16(d["wt"])


@pytest.mark.parametrize("mode_name,mode", MODES)
def test_full_activation_1x128_sampled_rows(layer, mode_name, mode):
    fp8q = require_gpu()
    d, x_dev, _ = layer
    q, s = fp8q.fp8_quant_tile(x_dev, fp8q.TILE_1x128, mode)
    rows = np.sort(np.random.default_rng(21).choice(8192, 48, replace=False))
    rows = np.concatenate([rows, [0, 8191]])
    q_ref, s_ref = oq.quant_1x128(oq.bf16_bits_to_f32(d["x"][rows]), mode_name)
    assert_bytes_equal(host(q[torch.as_tensor(rows).cuda()]), q_ref, "codes")
    assert_bytes_equal(host(s)[:, rows], s_ref, "scales")


def test_full_weight_block_sampled_bands(layer):
    fp8q = require_gpu()
    d, _, w_dev = layer
    q, s, qt, st = fp8q.fp8_quant_block(w_dev, 0, transposed=True)
    qh, sh, qth, sth = host(q), host(s), host(qt), host(st)
    for band in (0, 77, 143):                                   # 128-row bands of the [18432][7168] weight
        rs = slice(band * 128, (band + 1) * 128)
        q_ref, s_ref = oq.quant_128x128(oq.bf16_bits_to_f32(d["wt"][rs]), "maxabs")
        assert_bytes_equal(qh[rs], q_ref, f"band {band} codes")
        assert_bytes_equal(sh[band], s_ref[0], f"band {band} scales")
        assert_bytes_equal(qth[:, rs], np.ascontiguousarray(q_ref.T), f"band {band} transposed codes")
        assert_bytes_equal(sth[:, band], s_ref[0], f"band {band} transposed scales")


def test_full_wgrad_operands_128x1_sampled_columns(layer):
    fp8q = require_gpu()
    d, x_dev, _ = layer
    qt, s = fp8q.fp8_quant_tile(x_dev, fp8q.TILE_128x1, 0)
    cols = np.sort(np.random.default_rng(22).choice(7168, 40, replace=False))
    qt_ref, s_ref = oq.quant_128x1(oq.bf16_bits_to_f32(d["x"][:, cols]), "maxabs")
    assert_bytes_equal(host(qt)[cols], qt_ref, "transposed codes")
    assert_bytes_equal(host(s)[:, cols], s_ref, "scales")


def test_full_output_grad_both_tilings_sampled():
    fp8q = require_gpu()
    dy = output_grad()["dy"]
    dy_dev = dev_bf16(dy)
    q, s = fp8q.fp8_quant_tile(dy_dev, fp8q.TILE_1x128, 0)
    rows = np.sort(np.random.default_rng(23).choice(8192, 24, replace=False))
    q_ref, s_ref = oq.quant_1x128(oq.bf16_bits_to_f32(dy[rows]), "maxabs")
    assert_bytes_equal(host(q)[rows], q_ref, "1x128 codes")
    assert_bytes_equal(host(s)[:, rows], s_ref, "1x128 scales")
    del q, s
    qt, s = fp8q.fp8_quant_tile(dy_dev, fp8q.TILE_128x1, 1)
    cols = np.sort(np.random.default_rng(24).choice(18432, 24, replace=False))
    qt_ref, s_ref = oq.quant_128x1(oq.bf16_bits_to_f32(dy[:, cols]), "pow2")
    assert_bytes_equal(host(qt)[cols], qt_ref, "128x1 codes")
    assert_bytes_equal(host(s)[:, cols], s_ref, "128x1 scales")


@pytest.mark.parametrize("mode_name,mode", MODES)
def test_scale_derivation_across_all_binades(mode_name, mode):
    """262144 tiles whose max-abs values cover every float32 binade from the
    floor 448*2^-126 to 2^127 with random mantissas (plus the exact edges); the
    scales (and the codes, which depend on the reciprocal scale) must equal the
    oracle's IEEE-division results bit for bit."""
    fp8q = require_gpu()
    rng = np.random.default_rng(101)
    n_tiles = 262144
    lo, hi = 0x04E00000, 0x7F7FFFFF
    amax_bits = rng.integers(lo, hi + 1, size=n_tiles, dtype=np.int64)
    amax_bits[:8] = [lo, lo + 1, 0x7F000000, hi, 0x43E00000, 0x3F800000, 0x7E800000, 0x72800000]
    amax = amax_bits.astype(np.uint32).view(np.float32)
    body = rng.uniform(-1.0, 1.0, size=(n_tiles, 128)).astype(np.float32)
    x = (body * amax[:, None]).astype(np.float32)
    x[:, 0] = amax
    x = np.where(np.isfinite(x), x, 0).astype(np.float32)
    q, s = fp8q.fp8_quant_tile(dev(x), fp8q.TILE_1x128, mode)
    q_ref, s_ref = oq.quant_1x128(x, mode_name)
    assert_bytes_equal(host(s), s_ref, "scales")
    assert_bytes_equal(host(q), q_ref, "codes")


# ----------------------------------------------------------------------------
# FP8 -> FP8 1x128 -> 128x1 re-quantization.  Every input (codes and scales)
# comes from the oracle's 1x128 quantizer or from a seeded generator.
# ----------------------------------------------------------------------------

def _requant_check(fp8q, q, s, mode_name, mode):
    qt, st = fp8q.fp8_requant_1x128_to_128x1(dev(q), dev(s), mode)
    qt_ref, st_ref = oq.requant_1x128_to_128x1(q, s, mode_name)
    assert_bytes_equal(host(qt), qt_ref, "transposed codes")
    assert_bytes_equal(host(st), st_ref, "128x1 scales")


@pytest.mark.parametrize("in_mode", ["maxabs", "pow2"])
@pytest.mark.parametrize("mode_name,mode", MODES)
@pytest.mark.parametrize("shape", [(128, 128), (256, 384), (384, 256), (1024, 128)])
def test_requant_from_oracle_1x128(in_mode, mode_name, mode, shape):
    fp8q = require_gpu()
    q, s = oq.quant_1x128(_data(sum(shape) + 7, shape), in_mode)
    _requant_check(fp8q, q, s, mode_name, mode)


@pytest.mark.parametrize("mode_name,mode", MODES)
def test_requant_every_code_and_extreme_scales(mode_name, mode):
    # Every finite code (both zeros and all subnormals included) under row
    # scales spread from 2^-126 to 2^100, power-of-2 and not, so the FP32
    # dequantization runs through subnormal and huge products.
    fp8q = require_gpu()
    rng = np.random.default_rng(31)
    rows, cols = 512, 512
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    q = rng.choice(finite, size=(rows, cols)).astype(np.uint8)
    e = rng.integers(-126, 101, size=(cols // 128, rows))
    mant = np.where(rng.random((cols // 128, rows)) < 0.5, 1.0, rng.uniform(1.0, 2.0, (cols // 128, rows)))
    s = (mant * np.exp2(e.astype(np.float64))).astype(np.float32)
    s[0, :4] = [2.0 ** -126, np.float32(1.5 * 2.0 ** -126), 2.0 ** 100, np.float32(1.0 / 448.0)]
    _requant_check(fp8q, q, s, mode_name, mode)


def test_requant_lossless_when_scales_align():
    fp8q = require_gpu()
    rng = np.random.default_rng(32)
    rows, cols = 256, 256
    q = rng.integers(0, 0x78, size=(rows, cols), dtype=np.uint8) | (rng.integers(0, 2, (rows, cols)) << 7).astype(np.uint8)
    q[rng.integers(0, 128, cols), np.arange(cols)] = 0x7E          # every 128x1 tile reaches 448
    q[128 + rng.integers(0, 128, cols), np.arange(cols)] = 0xF8    # ... and -256
    s = np.full((cols // 128, rows), 2.0 ** -5, dtype=np.float32)
    qt, st = fp8q.fp8_requant_1x128_to_128x1(dev(q), dev(s), 1)
    assert_bytes_equal(host(qt), np.ascontiguousarray(q.T), "codes come back transposed and unchanged")
    assert np.all(host(st) == np.float32(2.0 ** -5))


def test_requant_strided_input_and_output():
    fp8q = require_gpu()
    q, s = oq.quant_1x128(_data(33, (256, 256)), "pow2")
    q_big = torch.zeros((256, 384), dtype=torch.uint8, device="cuda")
    q_big[:, :256] = dev(q)
    qt_big = torch.full((256, 320), 0xAB, dtype=torch.uint8, device="cuda")
    st = torch.empty((2, 256), dtype=torch.float32, device="cuda")
    fp8q.fp8_requant_1x128_to_128x1(q_big[:, :256], dev(s), 1, q_t=qt_big[:, :256], scales_t=st)
    qt_ref, st_ref = oq.requant_1x128_to_128x1(q, s, "pow2")
    h = host(qt_big)
    assert_bytes_equal(h[:, :256], qt_ref, "codes")
    assert np.all(h[:, 256:] == 0xAB), "padding columns of the output were written"
    assert_bytes_equal(host(st), st_ref, "scales")


@pytest.fixture(scope="module")
def activation_pow2_1x128(layer):
    d, _, _ = layer
    return oq.quant_1x128(oq.bf16_bits_to_f32(d["x"]), "pow2")


@pytest.mark.parametrize("mode_name,mode", MODES)
def test_full_requant_activation_sampled_groups(activation_pow2_1x128, mode_name, mode):
    # 8192 x 7168 activation, 1x128 pow2 codes as the backward pass caches
    # them; three 128-column groups are recomputed by the oracle.
    fp8q = require_gpu()
    q, s = activation_pow2_1x128
    qt, st = fp8q.fp8_requant_1x128_to_128x1(dev(q), dev(s), mode)
    qth, sth = host(qt), host(st)
    for g in (0, 29, 55):
        cs = slice(g * 128, (g + 1) * 128)
        qt_ref, st_ref = oq.requant_1x128_to_128x1(np.ascontiguousarray(q[:, cs]), s[g:g + 1], mode_name)
        assert_bytes_equal(qth[cs], qt_ref, f"group {g} codes")
        assert_bytes_equal(sth[:, cs], st_ref, f"group {g} scales")
