// Device-side building blocks shared by the fp8q kernels (gfx950 only).
//
// Quantization arithmetic follows the rule stated in include/fp8q.h:
// max-abs per group, scale derived from it (max-abs onto E4M3's 448, or the
// smallest power of two that keeps the group in range), multiply, clamp to
// +-448, round to E4M3FN with the hardware converter (v_cvt_pk_fp8_f32 rounds
// to nearest-even under the default round mode).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

// Largest finite OCP E4M3FN magnitude.
constexpr float kE4M3Max = 448.0f;
// Floor applied to a group's max-abs so zero or FP32-subnormal groups still
// get a normal scale: 448 * 2^-126 (bit pattern 0x04E00000).
constexpr uint32_t kAmaxFloorBits = 0x04E00000u;

constexpr int kModeMaxAbs = 0;
constexpr int kModePow2 = 1;

struct ScalePair {
  float s;    // dequantization multiplier (stored)
  float inv;  // quantization multiplier
};

// fl32(a / 448) for a >= 448 * 2^-126.  448 = 7 * 2^6, so a/448 is fl32(a/7)
// scaled exactly by 2^-6.  fl32(a/7) comes from the quotient estimate
// q0 = a * fl32(1/7), its exact residual r = a - 7*q0 (one FMA) and the
// corrected quotient q0 + r * fl32(1/7) (one more FMA): Markstein's
// FMA-based final correction for IEEE division (P. W. Markstein,
// "Computation of elementary functions on the IBM RISC System/6000
// processor", IBM J. Res. Develop. 34(1), 1990).  Checked bit-exact against
// IEEE division for every float32 in [448 * 2^-126, FLT_MAX] on gfx950.
__device__ __forceinline__ float div_by_448(float a) {
  const float c = __uint_as_float(0x3E124925u);          // fl32(1/7)
  const float q0 = a * c;
  const float r = __builtin_fmaf(-q0, 7.0f, a);
  return __builtin_fmaf(r, c, q0) * 0.015625f;
}

// fl32(448 / a) for a >= 448 * 2^-126: the hardware reciprocal estimate
// y ~ 1/a, q0 = 448 * y, then the same Markstein correction q0 + r * y with
// the residual r = 448 - a*q0 formed exactly by an FMA.  For a > 2^100 the
// computation runs on a * 2^-64 (so 1/a stays a normal number) and the
// result is scaled back exactly.  Checked bit-exact against IEEE division for
// every float32 in [448 * 2^-126, FLT_MAX] on gfx950.
__device__ __forceinline__ float div_448_by(float a0) {
  const bool big = a0 > 0x1p+100f;
  const float a = big ? a0 * 0x1p-64f : a0;
  const float y = __builtin_amdgcn_rcpf(a);
  const float q0 = 448.0f * y;
  const float r = __builtin_fmaf(-q0, a, 448.0f);
  return __builtin_fmaf(r, y, q0) * (big ? 0x1p-64f : 1.0f);
}

// Scale pair from a group's max-abs (given as float32 bits of a non-negative
// value).  MAXABS: s = fl32(a/448), inv = fl32(448/a).  POW2: s = 2^k with k
// the least integer such that a <= 448 * 2^k; writing a = 1.f * 2^e with
// 448 = 1.75 * 2^8, k = e - 8 when 1.f <= 1.75 (mantissa field <= 0x600000)
// and k = e - 7 otherwise.  a >= 448*2^-126 keeps k >= -126 and a < 2^128
// keeps k <= 120, so 2^k and 2^-k are normal.
template <int MODE>
__device__ __forceinline__ ScalePair scale_from_amax_bits(uint32_t amax_bits) {
  const uint32_t bits = amax_bits > kAmaxFloorBits ? amax_bits : kAmaxFloorBits;
  ScalePair r;
  if constexpr (MODE == kModePow2) {
    const int e = int(bits >> 23) - 127;
    const int k = ((bits & 0x7FFFFFu) <= 0x600000u) ? (e - 8) : (e - 7);
    r.s = __uint_as_float(uint32_t(127 + k) << 23);
    r.inv = __uint_as_float(uint32_t(127 - k) << 23);
  } else {
    const float a = __uint_as_float(bits);
    r.s = div_by_448(a);
    r.inv = div_448_by(a);
  }
  return r;
}

// Unsigned max across the 16 lanes of a DPP row, broadcast to all 16.
// quad_perm [1,0,3,2] and [2,3,0,1] reduce each quad; row_half_mirror pairs
// the quads of each half-row; row_mirror pairs the two halves.  Every source
// lane is a valid lane of the same row, so each step folds into one
// v_max_u32_dpp.  Must run with all 16 lanes of the row active.
#define FP8Q_DPP_MAX(v, ctrl) \
  ({ const uint32_t o_ = uint32_t(__builtin_amdgcn_mov_dpp(int(v), (ctrl), 0xF, 0xF, true)); (v) > o_ ? (v) : o_; })
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = FP8Q_DPP_MAX(v, 0xB1);
  v = FP8Q_DPP_MAX(v, 0x4E);
  v = FP8Q_DPP_MAX(v, 0x141);
  v = FP8Q_DPP_MAX(v, 0x140);
  return v;
}

__device__ __forceinline__ float clamp448(float v) {
  return __builtin_amdgcn_fmed3f(v, -kE4M3Max, kE4M3Max);
}

}  // namespace fp8q
