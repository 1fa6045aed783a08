// Device-side building blocks shared by the fp8q kernels (gfx950 only).
//
// Quantization arithmetic follows the rule stated in include/fp8q.h:
// max-abs per group, scale derived from it (max-abs onto E4M3's 448, or the
// smallest power of two that keeps the group in range), multiply, clamp to
// +-448, round to E4M3FN with the hardware converter.
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

// MAXABS: s = a/448 and inv = 448/a, each one IEEE-correct FP32 division
// (the library is built without fast-math, so '/' is correctly rounded).
// POW2: s = 2^k with k the least integer such that a <= 448 * 2^k.  Writing
// a = 1.f * 2^e: 448 = 1.75 * 2^8, so k = e - 8 when 1.f <= 1.75 (mantissa
// field <= 0x600000) and k = e - 7 otherwise.  a >= 448*2^-126 keeps
// k >= -126, and a < 2^128 keeps k <= 120, so both 2^k and 2^-k are normal.
__device__ __forceinline__ ScalePair scale_from_amax(float amax, int mode) {
  const float a = fmaxf(amax, __uint_as_float(kAmaxFloorBits));
  ScalePair r;
  if (mode == kModePow2) {
    const uint32_t bits = __float_as_uint(a);
    const int e = int((bits >> 23) & 0xFFu) - 127;
    const uint32_t frac = bits & 0x7FFFFFu;
    const int k = (frac <= 0x600000u) ? (e - 8) : (e - 7);
    r.s = __uint_as_float(uint32_t(127 + k) << 23);
    r.inv = __uint_as_float(uint32_t(127 - k) << 23);
  } else {
    r.s = a / kE4M3Max;
    r.inv = kE4M3Max / a;
  }
  return r;
}

// Max over the 16 lanes of a DPP row (lanes 16r..16r+15), broadcast to all
// 16.  quad_perm [1,0,3,2] and [2,3,0,1] reduce each quad; row_half_mirror
// pairs quad i with quad 1-i of the same 8; row_mirror pairs the two halves.
// Must be called with all 16 lanes of the row active.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}

// Max over a DPP quad (4 consecutive lanes), broadcast to the quad.
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  return v;
}

__device__ __forceinline__ float clamp448(float v) {
  return __builtin_amdgcn_fmed3f(v, -kE4M3Max, kE4M3Max);
}

// Four already-scaled FP32 values -> four E4M3FN bytes (a in byte 0 ... d in
// byte 3).  The clamp makes saturation explicit; v_cvt_pk_fp8_f32 rounds to
// nearest-even under the default FP round mode.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), w, true);
}

// BF16 pairs packed little-endian in a 32-bit word -> two floats (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Load 8 consecutive input elements (16-byte aligned) as floats.
template <typename T> struct Load8;

template <> struct Load8<uint16_t> {   // BF16 bit patterns
  static __device__ __forceinline__ void run(const uint16_t* p, float (&v)[8]) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
    v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  }
};

template <> struct Load8<float> {
  static __device__ __forceinline__ void run(const float* p, float (&v)[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

}  // namespace fp8q
