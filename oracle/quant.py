"""Fine-grained FP8 quantizers (TEST INFRASTRUCTURE ONLY -- never imported by the product path).

What the pages fix:
    * activations are grouped and scaled per 1x128 tile (per token per 128
      channels) and weights per 128x128 block (per 128 input channels per 128
      output channels) -- dssusan.co.kr FP8 excerpt, paragraph 4; youlimart.com
      FP8 excerpt, paragraph 1; "FP8 mixed precision - где и как DeepSeek
      снизили точность вычислений?", section "Точечное (fine-grained) квантование";
    * the maximum absolute value of each tile/block is computed online, the
      scaling factor is derived from it, and the tensor is quantized to FP8
      online -- dssusan.co.kr FP8 excerpt, paragraph 2;
    * the derivation maps the max-abs onto the largest representable FP8
      value -- "Deepseek - Not For everyone", paragraph 3;
    * some scales are restricted to integral powers of 2 -- dssusan.co.kr FP8
      excerpt, paragraph 1;
    * activations go from 1x128 tiles to 128x1 tiles for the backward pass --
      dssusan.co.kr FP8 excerpt, paragraph 4.

Readings taken where the pages are silent (all pinned in tests/test_oracle_quant.py):
    * the stored scale is the dequantization multiplier s = a / 448 and the
      quantization multiplies by inv = 448 / a, both single correctly-rounded
      float32 divisions; q = E4M3(fl32(x * inv));
    * a = max(max|x|, 448 * 2^-126) so that all-zero or tiny tiles get a
      normal float32 scale (zero tiles quantize to +-0);
    * power-of-2 mode: s = 2^k with k the smallest integer such that
      a <= 448 * 2^k (round the exponent up, so nothing saturates);
      inv = 2^-k exactly;
    * a group that runs past the tensor edge covers only the elements present;
    * 128x1 output is written transposed (QT[c][r]) with scales S[r/128][c];
      1x128 scales are stored group-major, S[c/128][r].

Inputs are float32 arrays (BF16 inputs are widened exactly first with
``bf16_bits_to_f32``). Outputs: uint8 E4M3 codes and float32 scales.
"""

import numpy as np

from . import e4m3

MODE_MAXABS = "maxabs"
MODE_POW2 = "pow2"

GROUP = 128
#: Floor on the group max-abs: 448 * 2^-126 (float32 bits 0x04E00000).
AMAX_FLOOR = np.float32(448.0 * 2.0 ** -126)
_F448 = np.float32(448.0)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening of BF16 bit patterns (uint16) to float32."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def scales_from_amax(amax, mode: str):
    """Return (s, inv) float32 arrays for group max-abs values ``amax``.

    max-abs mode: s = fl32(a/448), inv = fl32(448/a) with a = max(amax, floor).
    pow2 mode:    s = 2^k, inv = 2^-k, k the smallest integer with a <= 448*2^k.
    """
    amax = np.asarray(amax, dtype=np.float32)
    if not np.all(np.isfinite(amax)):
        raise ValueError("non-finite input is not defined for the quantizer")
    a = np.maximum(amax, AMAX_FLOOR)
    if mode == MODE_MAXABS:
        s = (a / _F448).astype(np.float32)          # IEEE float32 division
        inv = (_F448 / a).astype(np.float32)
        return s, inv
    if mode == MODE_POW2:
        a64 = a.astype(np.float64)
        _, e = np.frexp(a64)                          # a = m * 2^e, m in [0.5, 1)
        k = e.astype(np.int64) - 9                    # first guess: 448*2^(e-9) = 0.875*2^e
        k = np.where(a64 > 448.0 * np.ldexp(1.0, k), k + 1, k)
        # k is now the smallest integer with a <= 448 * 2^k:
        assert np.all(a64 <= 448.0 * np.ldexp(1.0, k))
        assert np.all(a64 > 448.0 * np.ldexp(1.0, k - 1))
        s = np.ldexp(np.float32(1.0), k).astype(np.float32)
        inv = np.ldexp(np.float32(1.0), -k).astype(np.float32)
        return s, inv
    raise ValueError(f"unknown scale mode {mode!r}")


def _quantize_groups(g, mode):
    """Quantize an array shaped [..., n] whose last axis is one group.

    Returns (codes with the same shape, scales shaped [...]).
    """
    g = np.asarray(g, dtype=np.float32)
    amax = np.max(np.abs(g), axis=-1)
    s, inv = scales_from_amax(amax, mode)
    scaled = (g * inv[..., None]).astype(np.float32)      # one float32 rounding
    return e4m3.encode(scaled), s


def _pad_to(x, rows, cols):
    """Zero-pad a 2-D float32 array; zeros never change a group's max-abs."""
    out = np.zeros((rows, cols), dtype=np.float32)
    out[: x.shape[0], : x.shape[1]] = x
    return out


def _ceil(n, d):
    return -(-n // d)


def quant_1x128(x, mode=MODE_MAXABS):
    """1x128 tiles along the columns of X[R][C].

    Returns Q[R][C] (uint8) and S[ceil(C/128)][R] (float32, group-major).
    """
    x = np.asarray(x, dtype=np.float32)
    r, c = x.shape
    gc = _ceil(c, GROUP)
    xp = _pad_to(x, r, gc * GROUP).reshape(r, gc, GROUP)
    q, s = _quantize_groups(xp, mode)                # q [r][gc][128], s [r][gc]
    return q.reshape(r, gc * GROUP)[:, :c].copy(), np.ascontiguousarray(s.T)


def quant_128x1(x, mode=MODE_MAXABS):
    """128x1 tiles along the rows of X[R][C], output transposed.

    Returns QT[C][R] (uint8; QT[c][r] is the code of X[r][c]) and
    S[ceil(R/128)][C] (float32).
    """
    x = np.asarray(x, dtype=np.float32)
    r, c = x.shape
    gr = _ceil(r, GROUP)
    xt = _pad_to(x, gr * GROUP, c).T.reshape(c, gr, GROUP)   # [c][gr][128]
    q, s = _quantize_groups(xt, mode)                        # s [c][gr]
    return q.reshape(c, gr * GROUP)[:, :r].copy(), np.ascontiguousarray(s.T)


def quant_128x128(w, mode=MODE_MAXABS):
    """128x128 blocks of W[R][C].

    Returns Q[R][C] (uint8, same layout as W) and S[ceil(R/128)][ceil(C/128)].
    The transposed copies a Dgrad GEMM consumes are simply Q.T and S.T.
    """
    w = np.asarray(w, dtype=np.float32)
    r, c = w.shape
    gr, gc = _ceil(r, GROUP), _ceil(c, GROUP)
    wp = _pad_to(w, gr * GROUP, gc * GROUP)
    blocks = wp.reshape(gr, GROUP, gc, GROUP).transpose(0, 2, 1, 3).reshape(gr, gc, GROUP * GROUP)
    q, s = _quantize_groups(blocks, mode)                    # q [gr][gc][16384]
    q = q.reshape(gr, gc, GROUP, GROUP).transpose(0, 2, 1, 3).reshape(gr * GROUP, gc * GROUP)
    return q[:r, :c].copy(), s.astype(np.float32)


def dequant_1x128(q, s):
    """Dequantized float64 X from 1x128 codes Q[R][C] and scales S[G][R]."""
    q = np.asarray(q)
    r, c = q.shape
    col_scale = np.repeat(np.asarray(s, np.float64).T, GROUP, axis=1)[:, :c]
    return e4m3.decode(q) * col_scale


def dequant_128x128(q, s):
    """Dequantized float64 W from block codes Q[R][C] and scales S[R/128][C/128]."""
    q = np.asarray(q)
    r, c = q.shape
    full = np.repeat(np.repeat(np.asarray(s, np.float64), GROUP, axis=0), GROUP, axis=1)
    return e4m3.decode(q) * full[:r, :c]


def requant_1x128_to_128x1(q, s, mode=MODE_POW2):
    """FP8 -> FP8 re-tiling: 1x128 codes Q[R][C] with scales S[C/128][R] to
    128x1 tiles, output transposed.

    The backward pass converts cached activations from 1x128 tiles to 128x1
    tiles (dssusan.co.kr FP8 excerpt, paragraph 4), and those activations use
    power-of-2 scales (paragraph 1).  Steps, in the pages' order:
      1. dequantize each element in float32: xh = fl32(dec(Q[r][c]) * S[c/128][r])
         (exact when S is a power of 2);
      2. quantize xh in 128x1 tiles exactly as ``quant_128x1`` does.
    Returns QT[C][R] (uint8) and S'[ceil(R/128)][C] (float32).
    """
    q = np.asarray(q, dtype=np.uint8)
    r, c = q.shape
    s = np.asarray(s, dtype=np.float32)
    if s.shape != (_ceil(c, GROUP), r):
        raise ValueError("1x128 scales must be shaped [ceil(C/128)][R]")
    dec = e4m3.decode(q).astype(np.float32)                  # exact: E4M3 values fit float32
    if not np.all(np.isfinite(dec)):
        raise ValueError("NaN codes are not defined for the re-quantizer")
    col_scale = np.repeat(s.T, GROUP, axis=1)[:, :c]         # [R][C] float32
    xh = (dec * col_scale).astype(np.float32)                # one float32 rounding
    return quant_128x1(xh, mode)
