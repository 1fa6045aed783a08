"""Python binding of the fp8q C ABI (include/fp8q.h) for AMD MI355X.

Argument marshalling only: every step of quantization and GEMM runs in the
HIP kernels of ``libfp8q.so``.  torch supplies device memory and the stream.
Importing this package fails loudly if the library has not been built
(``python -c "import __graft_entry__; __graft_entry__.build()"``); there is
no CPU fallback.

Functions keep the C names:
    fp8_quant_tile(x, tile, mode)              -> (q, scales)
    fp8_quant_tile_dual(x, mode)               -> (q, scales, q_t, scales_t)   (1x128 and 128x1 at once)
    fp8_quant_block(w, mode, transposed)       -> (q, scales[, q_t, scales_t])
    fp8_gemm_blockscaled(kind, a, sa, b, sb)   -> c
    fp8_gemm_blockscaled_pow2(kind, a, sa, b, sb, pow2_operands) -> c   (power-of-two scales)
    fp8_gemm_blockscaled_grouped(gmap, a, sa, b, sb) -> c
    fp8_requant_1x128_to_128x1(q, scales, mode) -> (q_t, scales_t)
FP8 tensors are torch.uint8 holding OCP E4M3FN codes.
"""

import ctypes
import os

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libfp8q.so")

# enums of include/fp8q.h
OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_UNSUPPORTED, ERR_ALIAS, ERR_HIP, ERR_ARG = range(8)
BF16, F32 = 0, 1
MAXABS, POW2 = 0, 1
TILE_1x128, TILE_128x1 = 0, 1
FPROP, DGRAD, WGRAD = 0, 1, 2
POW2_A, POW2_B, POW2_AB = 1, 2, 3

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_int = ctypes.c_int
_ptr = ctypes.c_void_p

# (name, argtypes) for every entry point of include/fp8q.h
SIGNATURES = {
    "fp8_quant_tile": [_ptr, _int, _i64, _i64, _i64, _int, _int, _ptr, _i64, _ptr, _ptr],
    "fp8_quant_block": [_ptr, _int, _i64, _i64, _i64, _int, _ptr, _i64, _ptr, _ptr, _i64, _ptr, _ptr],
    "fp8_quant_tile_dual": [_ptr, _int, _i64, _i64, _i64, _int, _ptr, _i64, _ptr, _ptr, _i64, _ptr, _ptr],
    "fp8_gemm_blockscaled": [_int, _i64, _i64, _i64, _ptr, _i64, _ptr, _ptr, _i64, _ptr, _ptr, _int, _i64,
                             _int, _ptr],
    "fp8_gemm_blockscaled_pow2": [_int, _i64, _i64, _i64, _ptr, _i64, _ptr, _ptr, _i64, _ptr, _ptr, _int, _i64,
                                  _int, _int, _ptr],
    "fp8_gemm_blockscaled_grouped": [_i32, _i64, _i64, _i64, _ptr, _ptr, _i64, _ptr, _ptr, _ptr, _ptr, _int,
                                     _i64, _ptr],
    "fp8_requant_1x128_to_128x1": [_ptr, _i64, _i64, _i64, _ptr, _int, _ptr, _i64, _ptr, _ptr],
    "fp8q_status_string": [_int],
    "fp8q_abi_version": [],
}


class Fp8qError(RuntimeError):
    """A non-OK status returned by the C ABI."""

    def __init__(self, status):
        self.status = status
        super().__init__(status_string(status))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, argtypes in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_char_p if name == "fp8q_status_string" else ctypes.c_int
    return lib


lib = _load()


def status_string(status):
    return lib.fp8q_status_string(int(status)).decode()


def _check(status):
    if status != OK:
        raise Fp8qError(status)


def _run(fn, dev, stream, *args):
    """Call entry point `fn` with the tensors' device `dev` current and the stream resolved on it: the kernels run
    on the stream's device, and the NULL stream (torch's default stream) is the current device's."""
    if stream is not None and isinstance(getattr(stream, "device", None), torch.device) and stream.device != dev:
        raise ValueError(f"stream is on {stream.device}, the tensors on {dev}")
    with torch.cuda.device(dev):
        if stream is None:
            handle = torch.cuda.current_stream(dev).cuda_stream
        else:
            handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        _check(fn(*args, handle))


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _codes(t):
    """Accept uint8 or float8_e4m3fn code tensors; return the uint8 view."""
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError(f"FP8 operands are uint8 E4M3FN codes, got {t.dtype}")
    return t


def _rowmajor(t, name):
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be a 2-D row-major tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t


def _ld(t):
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], 1)


def _cdiv(a, b):
    return -(-a // b)


def _expect(t, name, dtype, shape, device, dense=False):
    """Check a caller-provided tensor before its pointer reaches the C ABI, which
    cannot see sizes: device, dtype, exact logical shape, and layout (dense, or
    2-D row-major with a leading dimension the ABI checks)."""
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a tensor on {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dense:
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    else:
        _rowmajor(t, name)
    return t


def fp8_quant_tile(x, tile=TILE_1x128, mode=MAXABS, q=None, scales=None, stream=None):
    """1x128 (q[rows][cols], scales[cols/128][rows]) or 128x1 (q[cols][rows] transposed,
    scales[rows/128][cols]) quantization of a 2-D bf16/fp32 tensor."""
    _rowmajor(x, "x")
    rows, cols = x.shape
    q_shape = (rows, cols) if tile == TILE_1x128 else (cols, rows)
    s_shape = (_cdiv(cols, 128), rows) if tile == TILE_1x128 else (_cdiv(rows, 128), cols)
    if q is None:
        q = torch.empty(q_shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(s_shape, dtype=torch.float32, device=x.device)
    q = _expect(_codes(q), "q", torch.uint8, q_shape, x.device)
    _expect(scales, "scales", torch.float32, s_shape, x.device, dense=True)
    _run(lib.fp8_quant_tile, x.device, stream, x.data_ptr(), _dtype_code(x), rows, cols, _ld(x), tile, mode,
         q.data_ptr(), _ld(q), scales.data_ptr())
    return q, scales


def fp8_quant_tile_dual(x, mode=MAXABS, q=None, scales=None, q_t=None, scales_t=None, stream=None):
    """1x128 (q, scales) and transposed 128x1 (q_t, scales_t) quantization of one
    2-D bf16/fp32 tensor in one pass; the same outputs as the two fp8_quant_tile calls."""
    _rowmajor(x, "x")
    rows, cols = x.shape
    dev = x.device
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((_cdiv(cols, 128), rows), dtype=torch.float32, device=dev)
    if q_t is None:
        q_t = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
    if scales_t is None:
        scales_t = torch.empty((_cdiv(rows, 128), cols), dtype=torch.float32, device=dev)
    q = _expect(_codes(q), "q", torch.uint8, (rows, cols), dev)
    _expect(scales, "scales", torch.float32, (_cdiv(cols, 128), rows), dev, dense=True)
    q_t = _expect(_codes(q_t), "q_t", torch.uint8, (cols, rows), dev)
    _expect(scales_t, "scales_t", torch.float32, (_cdiv(rows, 128), cols), dev, dense=True)
    _run(lib.fp8_quant_tile_dual, dev, stream, x.data_ptr(), _dtype_code(x), rows, cols, _ld(x), mode,
         q.data_ptr(), _ld(q), scales.data_ptr(), q_t.data_ptr(), _ld(q_t), scales_t.data_ptr())
    return q, scales, q_t, scales_t


def fp8_quant_block(w, mode=MAXABS, transposed=False, q=None, scales=None, q_t=None, scales_t=None,
                    stream=None):
    """128x128 block quantization; with transposed=True also the transposed codes
    q_t[cols][rows] and scales_t[cols/128][rows/128] (Dgrad's weight operand)."""
    _rowmajor(w, "w")
    rows, cols = w.shape
    dev = w.device
    if not transposed and (q_t is not None or scales_t is not None):
        raise ValueError("q_t / scales_t are the transposed copy: pass transposed=True")
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows // 128, cols // 128), dtype=torch.float32, device=dev)
    if transposed:
        if q_t is None:
            q_t = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
        if scales_t is None:
            scales_t = torch.empty((cols // 128, rows // 128), dtype=torch.float32, device=dev)
    q = _expect(_codes(q), "q", torch.uint8, (rows, cols), dev)
    _expect(scales, "scales", torch.float32, (_cdiv(rows, 128), _cdiv(cols, 128)), dev, dense=True)
    if q_t is not None:
        q_t = _expect(_codes(q_t), "q_t", torch.uint8, (cols, rows), dev)
    if scales_t is not None:
        _expect(scales_t, "scales_t", torch.float32, (_cdiv(cols, 128), _cdiv(rows, 128)), dev, dense=True)
    qt_ptr = q_t.data_ptr() if q_t is not None else None
    ld_qt = _ld(q_t) if q_t is not None else 0
    st_ptr = scales_t.data_ptr() if scales_t is not None else None
    _run(lib.fp8_quant_block, dev, stream, w.data_ptr(), _dtype_code(w), rows, cols, _ld(w), mode,
         q.data_ptr(), _ld(q), scales.data_ptr(), qt_ptr, ld_qt, st_ptr)
    if transposed:
        return q, scales, q_t, scales_t
    return q, scales


def fp8_gemm_blockscaled(kind, a, a_scales, b, b_scales, out_dtype=torch.bfloat16, c=None,
                         accumulate=False, stream=None):
    """C[M][N] (+)= A . B^T with per-128-K-group scales (see include/fp8q.h)."""
    return _gemm(lib.fp8_gemm_blockscaled, kind, a, a_scales, b, b_scales, out_dtype, c, accumulate, stream)


def fp8_gemm_blockscaled_pow2(kind, a, a_scales, b, b_scales, out_dtype=torch.bfloat16, c=None,
                              accumulate=False, pow2_operands=POW2_AB, stream=None):
    """Same GEMM with the power-of-two scales of A, B or both (pow2_operands)
    applied by the hardware-scaled MFMA."""
    return _gemm(lib.fp8_gemm_blockscaled_pow2, kind, a, a_scales, b, b_scales, out_dtype, c, accumulate, stream,
                 extra=(int(pow2_operands),))


def _gemm(fn, kind, a, a_scales, b, b_scales, out_dtype, c, accumulate, stream, extra=()):
    a, b = _codes(_rowmajor(a, "a")), _codes(_rowmajor(b, "b"))
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k:
        raise ValueError("a and b disagree on K")
    dev = a.device
    _expect(b, "b", torch.uint8, (n, k), dev)
    if kind in (FPROP, DGRAD, WGRAD):              # any other kind is the ABI's FP8Q_ERR_ARG
        _expect(a_scales, "a_scales", torch.float32, (_cdiv(k, 128), m), dev, dense=True)
        sb_shape = (_cdiv(k, 128), n) if kind == WGRAD else (_cdiv(n, 128), _cdiv(k, 128))
        _expect(b_scales, "b_scales", torch.float32, sb_shape, dev, dense=True)
    if c is None:
        c = torch.empty((m, n), dtype=out_dtype, device=dev)
    if c.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"c must be bfloat16 or float32, got {c.dtype}")
    _expect(c, "c", c.dtype, (m, n), dev)
    _run(fn, dev, stream, kind, m, n, k, a.data_ptr(), _ld(a), a_scales.data_ptr(), b.data_ptr(), _ld(b),
         b_scales.data_ptr(), c.data_ptr(), _dtype_code(c), _ld(c), 1 if accumulate else 0, *extra)
    return c


def fp8_gemm_blockscaled_grouped(group_of_mtile, a, a_scales, b, b_scales, out_dtype=torch.bfloat16,
                                 c=None, stream=None):
    """Grouped Fprop: b is [G][N][K] codes, b_scales [G][N/128][K/128], group_of_mtile int32
    [M_total/128] on the device."""
    a = _codes(_rowmajor(a, "a"))
    b = _codes(b)
    if b.dim() != 3 or not b.is_contiguous():
        raise ValueError("b must be a contiguous [G][N][K] tensor")
    g, n, k = b.shape
    m = a.shape[0]
    if a.shape[1] != k:
        raise ValueError("a and b disagree on K")
    dev = a.device
    _expect(b, "b", torch.uint8, (g, n, k), dev, dense=True)
    _expect(group_of_mtile, "group_of_mtile", torch.int32, (_cdiv(m, 128),), dev, dense=True)
    _expect(a_scales, "a_scales", torch.float32, (_cdiv(k, 128), m), dev, dense=True)
    _expect(b_scales, "b_scales", torch.float32, (g, _cdiv(n, 128), _cdiv(k, 128)), dev, dense=True)
    if c is None:
        c = torch.empty((m, n), dtype=out_dtype, device=dev)
    if c.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"c must be bfloat16 or float32, got {c.dtype}")
    _expect(c, "c", c.dtype, (m, n), dev)
    _run(lib.fp8_gemm_blockscaled_grouped, dev, stream, g, m, n, k, group_of_mtile.data_ptr(), a.data_ptr(),
         _ld(a), a_scales.data_ptr(), b.data_ptr(), b_scales.data_ptr(), c.data_ptr(), _dtype_code(c), _ld(c))
    return c


def fp8_requant_1x128_to_128x1(q, scales, mode=POW2, q_t=None, scales_t=None, stream=None):
    """FP8 -> FP8 re-tiling of 1x128 codes q[rows][cols] (scales[cols/128][rows]) into
    128x1 tiles: q_t[cols][rows] transposed, scales_t[rows/128][cols]."""
    q = _codes(_rowmajor(q, "q"))
    rows, cols = q.shape
    dev = q.device
    _expect(scales, "scales", torch.float32, (_cdiv(cols, 128), rows), dev, dense=True)
    if q_t is None:
        q_t = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
    if scales_t is None:
        scales_t = torch.empty((_cdiv(rows, 128), cols), dtype=torch.float32, device=dev)
    q_t = _expect(_codes(q_t), "q_t", torch.uint8, (cols, rows), dev)
    _expect(scales_t, "scales_t", torch.float32, (_cdiv(rows, 128), cols), dev, dense=True)
    _run(lib.fp8_requant_1x128_to_128x1, dev, stream, q.data_ptr(), rows, cols, _ld(q), scales.data_ptr(), mode,
         q_t.data_ptr(), _ld(q_t), scales_t.data_ptr())
    return q_t, scales_t
