"""The Python binding rejects caller-provided tensors whose device, dtype, shape
or layout does not match what the C ABI will read or write through their
pointers (the ABI sees no sizes).  Every call here raises before any kernel is
launched."""

import pytest
import torch

from tests.helpers import require_gpu

pytestmark = pytest.mark.gpu

U8, F32, BF = torch.uint8, torch.float32, torch.bfloat16


def _t(shape, dtype, device="cuda"):
    return torch.zeros(shape, dtype=dtype, device=device)


def test_quant_tile_outputs_checked():
    fp8q = require_gpu()
    x = _t((256, 384), BF)
    with pytest.raises(ValueError, match="scales has shape"):
        fp8q.fp8_quant_tile(x, fp8q.TILE_1x128, 0, scales=_t((3, 255), F32))
    with pytest.raises(ValueError, match="q has shape"):
        fp8q.fp8_quant_tile(x, fp8q.TILE_128x1, 0, q=_t((256, 384), U8))      # 128x1 codes are [cols][rows]
    with pytest.raises(TypeError, match="scales must be"):
        fp8q.fp8_quant_tile(x, fp8q.TILE_1x128, 0, scales=_t((3, 256), BF))
    with pytest.raises(ValueError, match="contiguous"):
        fp8q.fp8_quant_tile(x, fp8q.TILE_1x128, 0, scales=_t((256, 3), F32).t())
    with pytest.raises(ValueError, match="must be a tensor on"):
        fp8q.fp8_quant_tile(x, fp8q.TILE_1x128, 0, q=_t((256, 384), U8, "cpu"))
    q, s = fp8q.fp8_quant_tile(x, fp8q.TILE_1x128, 0, q=_t((256, 384), torch.float8_e4m3fn))
    assert q.dtype == U8 and s.shape == (3, 256)                              # FP8 codes view is accepted


def test_quant_tile_dual_outputs_checked():
    fp8q = require_gpu()
    x = _t((256, 384), BF)
    with pytest.raises(ValueError, match="q_t has shape"):
        fp8q.fp8_quant_tile_dual(x, 0, q_t=_t((256, 384), U8))                # 128x1 codes are [cols][rows]
    with pytest.raises(ValueError, match="scales_t has shape"):
        fp8q.fp8_quant_tile_dual(x, 0, scales_t=_t((3, 256), F32))            # the 1x128 scale shape
    with pytest.raises(ValueError, match="scales has shape"):
        fp8q.fp8_quant_tile_dual(x, 0, scales=_t((2, 384), F32))              # the 128x1 scale shape
    with pytest.raises(TypeError, match="uint8 E4M3FN codes"):
        fp8q.fp8_quant_tile_dual(x, 0, q=_t((256, 384), BF))
    with pytest.raises(ValueError, match="must be a 2-D row-major"):
        fp8q.fp8_quant_tile_dual(_t((384, 256), BF).t(), 0)


def test_quant_block_and_requant_outputs_checked():
    fp8q = require_gpu()
    w = _t((256, 384), F32)
    with pytest.raises(ValueError, match="scales_t has shape"):
        fp8q.fp8_quant_block(w, 0, True, scales_t=_t((2, 3), F32))
    with pytest.raises(ValueError, match="q_t has shape"):
        fp8q.fp8_quant_block(w, 0, True, q_t=_t((256, 384), U8))
    q = _t((256, 384), U8)
    with pytest.raises(ValueError, match="scales has shape"):
        fp8q.fp8_requant_1x128_to_128x1(q, _t((256, 3), F32))
    with pytest.raises(ValueError, match="scales_t has shape"):
        fp8q.fp8_requant_1x128_to_128x1(q, _t((3, 256), F32), scales_t=_t((2, 256), F32))


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_gemm_operands_checked(kind):
    fp8q = require_gpu()
    m, n, k = 256, 384, 512
    a, b = _t((m, k), U8), _t((n, k), U8)
    sa = _t((k // 128, m), F32)
    sb = _t((k // 128, n), F32) if kind == 2 else _t((n // 128, k // 128), F32)
    bad_sb = _t((n // 128, k // 128), F32) if kind == 2 else _t((k // 128, n), F32)
    with pytest.raises(ValueError, match="b_scales has shape"):
        fp8q.fp8_gemm_blockscaled(kind, a, sa, b, bad_sb)
    with pytest.raises(ValueError, match="a_scales has shape"):
        fp8q.fp8_gemm_blockscaled(kind, a, _t((m, k // 128), F32), b, sb)
    with pytest.raises(ValueError, match="c has shape"):
        fp8q.fp8_gemm_blockscaled(kind, a, sa, b, sb, c=_t((m, n - 128), F32))
    with pytest.raises(TypeError, match="c must be bfloat16 or float32"):
        fp8q.fp8_gemm_blockscaled(kind, a, sa, b, sb, c=_t((m, n), torch.float16))
    with pytest.raises(ValueError, match="a_scales has shape"):
        fp8q.fp8_gemm_blockscaled_pow2(kind, a, _t((k // 128, m + 128), F32), b, sb)


def test_grouped_operands_checked():
    fp8q = require_gpu()
    g, m, n, k = 3, 512, 256, 256
    a, b = _t((m, k), U8), _t((g, n, k), U8)
    sa, sb = _t((k // 128, m), F32), _t((g, n // 128, k // 128), F32)
    gmap = torch.zeros(m // 128, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="group_of_mtile has shape"):
        fp8q.fp8_gemm_blockscaled_grouped(gmap[:3], a, sa, b, sb)
    with pytest.raises(TypeError, match="group_of_mtile must be"):
        fp8q.fp8_gemm_blockscaled_grouped(gmap.to(torch.int64), a, sa, b, sb)
    with pytest.raises(ValueError, match="b_scales has shape"):
        fp8q.fp8_gemm_blockscaled_grouped(gmap, a, sa, b, _t((g, n // 128 + 1, k // 128), F32))
    with pytest.raises(ValueError, match="c has shape"):
        fp8q.fp8_gemm_blockscaled_grouped(gmap, a, sa, b, sb, c=_t((m - 128, n), BF))


def test_stream_on_another_device_is_rejected():
    """Kernels run on the stream's device: a stream object that names another
    device than the tensors' is refused before anything is launched."""
    import types
    fp8q = require_gpu()
    x = _t((128, 128), BF)
    other = types.SimpleNamespace(device=torch.device("cuda", 1), cuda_stream=0)
    with pytest.raises(ValueError, match="stream is on"):
        fp8q.fp8_quant_tile(x, fp8q.TILE_1x128, fp8q.MAXABS, stream=other)
    # the tensors' own device: accepted, on an explicit stream and on the default one
    s = torch.cuda.Stream()
    q, sc = fp8q.fp8_quant_tile(x, fp8q.TILE_1x128, fp8q.MAXABS, stream=s)
    s.synchronize()
    q2, sc2 = fp8q.fp8_quant_tile(x, fp8q.TILE_1x128, fp8q.MAXABS)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(sc, sc2)
