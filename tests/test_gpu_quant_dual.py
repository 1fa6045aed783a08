"""GPU parity of fp8_quant_tile_dual (1x128 and transposed 128x1 tiles of one
tensor in one pass), through the C ABI: every output bit-exact against the
oracle's 1x128 and 128x1 quantizers, and against the two single-tiling
fp8_quant_tile calls at the full output-gradient size."""

import numpy as np
import pytest
import torch

from oracle import quant as oq
from tests.helpers import assert_bytes_equal, dev, dev_bf16, host, require_gpu
from workloads import add_outliers, linear_layer, normal_f32, output_grad, to_bf16_bits

pytestmark = pytest.mark.gpu

MODES = [("maxabs", 0), ("pow2", 1)]


def _data(seed, shape, sigma=1.0, frac=0.01, factor=100.0):
    rng = np.random.default_rng(seed)
    return add_outliers(rng, normal_f32(rng, shape, sigma), frac, factor)


def _to_dev(x_f32, dtype):
    if dtype == "bf16":
        bits = to_bf16_bits(x_f32)
        return dev_bf16(bits), oq.bf16_bits_to_f32(bits)
    return dev(x_f32), x_f32


def _check_against_oracle(outs, x_ref, mode_name, what=""):
    q, s, qt, st = (host(t) for t in outs)
    q_ref, s_ref = oq.quant_1x128(x_ref, mode_name)
    qt_ref, st_ref = oq.quant_128x1(x_ref, mode_name)
    assert_bytes_equal(s, s_ref, what + "1x128 scales")
    assert_bytes_equal(q, q_ref, what + "1x128 codes")
    assert_bytes_equal(st, st_ref, what + "128x1 scales")
    assert_bytes_equal(qt, qt_ref, what + "128x1 transposed codes")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode_name,mode", MODES)
@pytest.mark.parametrize("shape", [(128, 128), (256, 384), (384, 256), (640, 1152)])
def test_dual_matches_oracle(dtype, mode_name, mode, shape):
    fp8q = require_gpu()
    x_dev, x_ref = _to_dev(_data(50 + shape[0] + shape[1], shape), dtype)
    _check_against_oracle(fp8q.fp8_quant_tile_dual(x_dev, mode), x_ref, mode_name)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode_name,mode", MODES)
def test_dual_degenerate_groups(dtype, mode_name, mode):
    """Zero, negative-zero and constant blocks, a lone FP32 subnormal as a group's max-abs and values near the
    top of the FP32 range, in both tilings at once."""
    fp8q = require_gpu()
    x = _data(42, (256, 768))
    x[0:128, 0:128] = 0.0
    x[128:256, 0:128] = -0.0
    x[0:128, 128:256] = np.float32(-0.02)
    x[128:256, 128:256] = 0.0
    x[130, 200] = np.float32(1e-40)
    x[0:128, 256:384] = np.float32(1e30)
    x[5, 300] = np.float32(3e38)
    x[200, 640:768] = np.float32(7.0)                # a constant 1x128 row inside a varied 128x1 column band
    x_dev, x_ref = _to_dev(x, dtype)
    _check_against_oracle(fp8q.fp8_quant_tile_dual(x_dev, mode), x_ref, mode_name)


@pytest.mark.parametrize("mode_name,mode", MODES)
def test_dual_every_bf16_pattern(mode_name, mode):
    """Every finite BF16 pattern of magnitude <= 448, 127 per row behind a 448 (so each 1x128 tile has unit
    scale), in 128-row bands whose columns then mix all binades for the 128x1 tiles."""
    fp8q = require_gpu()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oq.bf16_bits_to_f32(bits)
    bits = bits[np.isfinite(vals) & (np.abs(vals) <= 448.0)]
    n_rows = -(-bits.size // 127)
    n_rows = -(-n_rows // 128) * 128
    bits = np.concatenate([bits, np.zeros(n_rows * 127 - bits.size, np.uint16)]).reshape(n_rows, 127)
    x_bits = np.concatenate([np.full((n_rows, 1), 0x43E0, np.uint16), bits], axis=1)
    _check_against_oracle(fp8q.fp8_quant_tile_dual(dev_bf16(x_bits), mode), oq.bf16_bits_to_f32(x_bits),
                          mode_name)


def test_dual_strided_input_and_outputs():
    """A column slice of a wider input; both code outputs into wider buffers whose extra bytes stay untouched."""
    fp8q = require_gpu()
    full = _data(8, (384, 768))
    bits = to_bf16_bits(full)
    x_dev = dev_bf16(bits)[:, 128:640]                        # ld 768, width 512
    q_store = torch.zeros((384, 544), dtype=torch.uint8, device="cuda")
    qt_store = torch.zeros((512, 400), dtype=torch.uint8, device="cuda")
    q, s, qt, st = fp8q.fp8_quant_tile_dual(x_dev, 0, q=q_store[:, :512], q_t=qt_store[:, :384])
    x_ref = oq.bf16_bits_to_f32(bits[:, 128:640])
    q_ref, s_ref = oq.quant_1x128(x_ref, "maxabs")
    qt_ref, st_ref = oq.quant_128x1(x_ref, "maxabs")
    assert_bytes_equal(host(q_store)[:, :512], q_ref, "1x128 codes")
    assert_bytes_equal(host(qt_store)[:, :384], qt_ref, "128x1 codes")
    assert np.all(host(q_store)[:, 512:] == 0) and np.all(host(qt_store)[:, 384:] == 0)
    assert_bytes_equal(host(s), s_ref, "1x128 scales")
    assert_bytes_equal(host(st), st_ref, "128x1 scales")


def test_dual_empty_is_noop():
    fp8q = require_gpu()
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda")
    q, s, qt, st = fp8q.fp8_quant_tile_dual(x, 0)
    assert q.shape == (0, 256) and s.shape == (2, 0) and qt.shape == (256, 0) and st.shape == (0, 256)


# ----------------------------------------------------------------------------
# Full size, in the launch configuration the bench times.
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("mode_name,mode", MODES)
def test_full_output_grad_dual_equals_single_tilings_and_oracle(mode_name, mode):
    """dY 8192x18432: every byte of the four outputs equals the two single-tiling calls; sampled rows and
    columns equal the oracle."""
    fp8q = require_gpu()
    dy = output_grad()["dy"]
    dy_dev = dev_bf16(dy)
    q, s, qt, st = fp8q.fp8_quant_tile_dual(dy_dev, mode)
    q1, s1 = fp8q.fp8_quant_tile(dy_dev, fp8q.TILE_1x128, mode)
    assert torch.equal(q, q1) and torch.equal(s.view(torch.int32), s1.view(torch.int32))
    del q1, s1
    qt1, st1 = fp8q.fp8_quant_tile(dy_dev, fp8q.TILE_128x1, mode)
    assert torch.equal(qt, qt1) and torch.equal(st.view(torch.int32), st1.view(torch.int32))
    del qt1, st1
    rows = np.sort(np.concatenate([np.random.default_rng(25).choice(8192, 16, replace=False), [0, 8191]]))
    q_ref, s_ref = oq.quant_1x128(oq.bf16_bits_to_f32(dy[rows]), mode_name)
    assert_bytes_equal(host(q)[rows], q_ref, "1x128 codes")
    assert_bytes_equal(host(s)[:, rows], s_ref, "1x128 scales")
    cols = np.sort(np.concatenate([np.random.default_rng(26).choice(18432, 16, replace=False), [0, 18431]]))
    qt_ref, st_ref = oq.quant_128x1(oq.bf16_bits_to_f32(dy[:, cols]), mode_name)
    assert_bytes_equal(host(qt)[cols], qt_ref, "128x1 codes")
    assert_bytes_equal(host(st)[:, cols], st_ref, "128x1 scales")


def test_full_activation_dual_equals_single_tilings():
    """X 8192x7168 (the activation with outliers), max-abs: the dual call against the two single-tiling calls."""
    fp8q = require_gpu()
    x_dev = dev_bf16(linear_layer()["x"])
    q, s, qt, st = fp8q.fp8_quant_tile_dual(x_dev, 0)
    q1, s1 = fp8q.fp8_quant_tile(x_dev, fp8q.TILE_1x128, 0)
    qt1, st1 = fp8q.fp8_quant_tile(x_dev, fp8q.TILE_128x1, 0)
    assert torch.equal(q, q1) and torch.equal(s.view(torch.int32), s1.view(torch.int32))
    assert torch.equal(qt, qt1) and torch.equal(st.view(torch.int32), st1.view(torch.int32))
