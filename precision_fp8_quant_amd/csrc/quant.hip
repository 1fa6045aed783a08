// Online fine-grained FP8 quantizers for gfx950.
//
//  * 1x128 tiles (one token x 128 channels), scales [cols/128][rows]
//  * 128x1 tiles (128 tokens x one channel), codes written transposed
//  * 128x128 blocks (weights), optional transposed copy for Dgrad
//  * FP8 -> FP8 re-tiling of 1x128 codes into 128x1 tiles (backward pass)
//
// Tile shapes and the max-abs -> scale -> cast sequence: dssusan.co.kr FP8
// excerpt, paragraphs 2 and 4; "Deepseek - Not For everyone", paragraph 3;
// power-of-2 scales: dssusan.co.kr FP8 excerpt, paragraph 1.
//
// All four kernels are HBM-bound streaming passes: 16-byte coalesced loads,
// max-abs taken on the integer bit patterns of |x| (non-negative floats order
// like their bits; BF16 pairs reduce two at a time with v_pk_max_u16),
// reduced across lanes with DPP (and LDS across waves where a group spans
// waves), one scale pair per group, v_cvt_pk_fp8_f32 for the cast.  The scale
// mode is a template parameter, so each kernel carries only its own rule.
#include "fp8q_device.h"
#include "fp8q_launch.h"

namespace fp8q {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Eight consecutive elements as raw 32-bit words: 4 words of BF16 pairs, or
// 8 words of FP32.
template <typename T> struct Raw8;
template <> struct Raw8<uint16_t> {
  u32x4 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void zero() { w = u32x4{0u, 0u, 0u, 0u}; }
  // float32 bits of max |x| over the 8 elements
  __device__ __forceinline__ uint32_t amax_bits() const {
    const u16x2 a = __builtin_bit_cast(u16x2, w.x & 0x7FFF7FFFu), b = __builtin_bit_cast(u16x2, w.y & 0x7FFF7FFFu);
    const u16x2 c = __builtin_bit_cast(u16x2, w.z & 0x7FFF7FFFu), d = __builtin_bit_cast(u16x2, w.w & 0x7FFF7FFFu);
    const u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
    const uint32_t hi = m.x > m.y ? m.x : m.y;
    return hi << 16;
  }
  __device__ __forceinline__ float get(int i) const {
    const uint32_t x = w[i >> 1];
    return (i & 1) ? __uint_as_float(x & 0xFFFF0000u) : __uint_as_float(x << 16);
  }
};
template <> struct Raw8<float> {
  u32x4 w0, w1;
  __device__ __forceinline__ void load(const float* p) {
    w0 = reinterpret_cast<const u32x4*>(p)[0];
    w1 = reinterpret_cast<const u32x4*>(p)[1];
  }
  __device__ __forceinline__ void zero() { w0 = u32x4{0u, 0u, 0u, 0u}; w1 = w0; }
  __device__ __forceinline__ uint32_t amax_bits() const {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t a = w0[i] & 0x7FFFFFFFu, b = w1[i] & 0x7FFFFFFFu;
      m = a > m ? a : m;
      m = b > m ? b : m;
    }
    return m;
  }
  __device__ __forceinline__ float get(int i) const { return __uint_as_float(i < 4 ? w0[i] : w1[i - 4]); }
};

// Scale, (for max-abs scales) clamp to +-448, and cast four values to E4M3
// (element i0 in byte 0 ... i0+3 in byte 3).  With power-of-2 scales the
// product is exact and already within +-448, so no clamp is needed.
template <int MODE>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d, float inv) {
  a *= inv; b *= inv; c *= inv; d *= inv;
  if constexpr (MODE == kModeMaxAbs) {
    a = clamp448(a); b = clamp448(b); c = clamp448(c); d = clamp448(d);
  }
  const uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// ---------------------------------------------------------------------------
// 1x128: a workgroup is 4 waves; a work unit is 32 consecutive rows x 4
// groups, wave w taking group 4*stripe + w.  A 16-lane DPP row holds one
// 128-element tile row (8 elements per lane), so the four DPP rows of a wave
// cover 4 rows per step and 8 unrolled steps cover 32 rows.  All eight loads
// are issued before any reduction (32 rows measured ~2% faster than 16 on the
// 8192x7168 activation).  FULL: all 32 rows exist (no row masking).
// ---------------------------------------------------------------------------
template <typename T, int MODE, bool FULL>
__device__ __forceinline__ void quant_1x128_body(const T* __restrict__ x, int64_t rows, int64_t ld_x,
                                                 uint8_t* __restrict__ q, int64_t ld_q,
                                                 float* __restrict__ scales, int64_t g, int64_t row0,
                                                 int sub, int seg) {
  const int64_t col = g * 128 + seg * 8;
  Raw8<T> v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = row0 + i * 4 + sub;
    if (FULL || r < rows) v[i].load(x + r * ld_x + col);
    else v[i].zero();
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const ScalePair sp = scale_from_amax_bits<MODE>(row16_max_u32(v[i].amax_bits()));
    const int64_t r = row0 + i * 4 + sub;
    uint2 out;
    out.x = cvt4<MODE>(v[i].get(0), v[i].get(1), v[i].get(2), v[i].get(3), sp.inv);
    out.y = cvt4<MODE>(v[i].get(4), v[i].get(5), v[i].get(6), v[i].get(7), sp.inv);
    if (FULL || r < rows) {
      *reinterpret_cast<uint2*>(q + r * ld_q + col) = out;
      if (seg == 0) scales[g * rows + r] = sp.s;
    }
  }
}

template <typename T, int MODE>
__global__ __launch_bounds__(256) void quant_1x128_kernel(
    const T* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scales) {
  // Work units of 32 rows x 4 groups in row-band-major order, so that
  // concurrently running workgroups stream whole rows (grid-stride loop).
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t groups = cols >> 7;
  const int64_t stripes = (groups + 3) >> 2;
  const int64_t units = ((rows + 31) >> 5) * stripes;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const int64_t g = (u % stripes) * 4 + wave;
    const int64_t row0 = (u / stripes) * 32;
    if (g >= groups) continue;                   // wave-uniform; this kernel has no barriers
    if (row0 + 32 <= rows)
      quant_1x128_body<T, MODE, true>(x, rows, ld_x, q, ld_q, scales, g, row0, lane >> 4, lane & 15);
    else
      quant_1x128_body<T, MODE, false>(x, rows, ld_x, q, ld_q, scales, g, row0, lane >> 4, lane & 15);
  }
}

// ---------------------------------------------------------------------------
// 128x1 with transposed output: a workgroup quantizes a 128-row x 64-column
// tile.  Thread t loads rows 4*(t/8)..+3 of the 8 columns 8*(t%8)..+7.
//   1. per-thread column max (bits of |x|) over its 4 rows; lanes t and t+8
//      of a DPP row share columns and are combined with row_ror:8; the 16
//      partials per column (4 per wave) meet in LDS
//   2. threads 0..63 finish one column each, derive the scale pair, store s
//      and publish inv in LDS
//   3. every thread scales its 4x8 values and packs each column's 4 rows into
//      one dword (the bytes come out already transposed), staged in an LDS
//      tile T[col][row] (pitch 132 bytes: conflict-free dword writes)
//   4. thread t copies 32 bytes of column t/4 (rows 32*(t%4)..+31) to q.
// ---------------------------------------------------------------------------
constexpr int kT1Pitch = 132;   // bytes per LDS row of the transposed tile

template <typename T, int MODE>
__global__ __launch_bounds__(256) void quant_128x1_kernel(
    const T* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scales) {
  __shared__ uint32_t part[16][64];
  __shared__ float inv_s[64];
  __shared__ uint32_t tile[64 * kT1Pitch / 4];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int c8 = t & 7;
  const int q4 = t >> 3;
  const int64_t ctiles = (cols + 63) >> 6;
  const int64_t tiles = ctiles * (rows >> 7);
  for (int64_t u = blockIdx.x; u < tiles; u += gridDim.x) {   // block-uniform: barriers stay matched
  const int64_t col0 = (u % ctiles) * 64;
  const int64_t rblk = u / ctiles;
  const int64_t row0 = rblk * 128;
  const int64_t col = col0 + c8 * 8;
  const bool col_ok = col < cols;                 // cols % 8 == 0: all-or-nothing per thread

  Raw8<T> v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (col_ok) v[j].load(x + (row0 + q4 * 4 + j) * ld_x + col);
    else v[j].zero();
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t b = __float_as_uint(v[j].get(i)) & 0x7FFFFFFFu;
      m = b > m ? b : m;
    }
    m = FP8Q_DPP_MAX(m, 0x128);                   // row_ror:8 -> lanes l and l+8 of a DPP row
    if ((lane & 15) < 8) part[(t >> 6) * 4 + ((lane >> 4) & 3)][c8 * 8 + i] = m;
  }
  __syncthreads();
  if (t < 64) {
    uint32_t m = part[0][t];
#pragma unroll
    for (int p = 1; p < 16; ++p) m = part[p][t] > m ? part[p][t] : m;
    const ScalePair sp = scale_from_amax_bits<MODE>(m);
    inv_s[t] = sp.inv;
    if (col0 + t < cols) scales[rblk * cols + col0 + t] = sp.s;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float inv = inv_s[c8 * 8 + i];
    tile[((c8 * 8 + i) * kT1Pitch + q4 * 4) >> 2] = cvt4<MODE>(v[0].get(i), v[1].get(i), v[2].get(i), v[3].get(i), inv);
  }
  __syncthreads();
  const int cc = t >> 2;
  const int h = t & 3;
  if (col0 + cc < cols) {
    const uint32_t* src = tile + ((cc * kT1Pitch + h * 32) >> 2);
    uint4 lo, hi;
    lo.x = src[0]; lo.y = src[1]; lo.z = src[2]; lo.w = src[3];
    hi.x = src[4]; hi.y = src[5]; hi.z = src[6]; hi.w = src[7];
    uint8_t* dst = q + (col0 + cc) * ld_q + row0 + h * 32;
    reinterpret_cast<uint4*>(dst)[0] = lo;
    reinterpret_cast<uint4*>(dst)[1] = hi;
  }
  __syncthreads();                                // LDS is reused by the next tile
  }
}

// ---------------------------------------------------------------------------
// 128x128 blocks: one workgroup per block.  Thread t owns the 8 columns
// 8*(t%16)..+7 of rows {4*(t/16)+j, 64+4*(t/16)+j : j=0..3}.
//   1. thread max (bits of |x|) -> DPP max over the 16 lanes of a row -> LDS
//      across the 16 row-groups; every thread reads the block max
//   2. row-major codes: 8 bytes per (thread, row), 128-byte runs per row
//   3. optional transposed copy: each column's 4 adjacent rows are packed into
//      one dword, staged in an LDS tile T[col][row] (pitch 132 bytes), and
//      thread t copies 64 bytes of column t/2 (rows 64*(t%2)..+63) to q_t.
// ---------------------------------------------------------------------------
constexpr int kBPitch = 132;

template <typename T, int MODE>
__global__ __launch_bounds__(256) void quant_128x128_kernel(
    const T* __restrict__ w, int64_t rows, int64_t cols, int64_t ld_w,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scales,
    uint8_t* __restrict__ q_t, int64_t ld_qt, float* __restrict__ scales_t) {
  __shared__ uint32_t group_max[16];
  __shared__ uint32_t tile[128 * kBPitch / 4];

  const int t = threadIdx.x;
  const int c16 = t & 15;
  const int rq = t >> 4;                          // 0..15
  const int64_t cblocks = cols >> 7;
  const int64_t nblocks = cblocks * (rows >> 7);
  for (int64_t u = blockIdx.x; u < nblocks; u += gridDim.x) {   // block-uniform: barriers stay matched
  const int64_t bc = u % cblocks, br = u / cblocks;
  const int64_t col = bc * 128 + c16 * 8;
  const int64_t row_base = br * 128 + rq * 4;

  Raw8<T> v[8];                                   // [j]: row (j/4)*64 + 4*rq + j%4, cols 8*c16..+7
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j].load(w + (row_base + (j >> 2) * 64 + (j & 3)) * ld_w + col);

  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t b = v[j].amax_bits();
    m = b > m ? b : m;
  }
  m = row16_max_u32(m);
  if (c16 == 0) group_max[rq] = m;
  __syncthreads();
  m = group_max[0];
#pragma unroll
  for (int p = 1; p < 16; ++p) m = group_max[p] > m ? group_max[p] : m;
  const ScalePair sp = scale_from_amax_bits<MODE>(m);
  if (t == 0) {
    scales[br * (cols >> 7) + bc] = sp.s;
    if (scales_t) scales_t[bc * (rows >> 7) + br] = sp.s;
  }

#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint2 out;
    out.x = cvt4<MODE>(v[j].get(0), v[j].get(1), v[j].get(2), v[j].get(3), sp.inv);
    out.y = cvt4<MODE>(v[j].get(4), v[j].get(5), v[j].get(6), v[j].get(7), sp.inv);
    *reinterpret_cast<uint2*>(q + (row_base + (j >> 2) * 64 + (j & 3)) * ld_q + col) = out;
  }
  if (q_t != nullptr) {                            // block-uniform: no barrier is skipped by part of the block

#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      tile[((c16 * 8 + i) * kBPitch + h * 64 + rq * 4) >> 2] =
          cvt4<MODE>(v[4 * h].get(i), v[4 * h + 1].get(i), v[4 * h + 2].get(i), v[4 * h + 3].get(i), sp.inv);
  __syncthreads();
  const int cc = t >> 1;
  const int hh = t & 1;
  const uint32_t* src = tile + ((cc * kBPitch + hh * 64) >> 2);
  uint8_t* dst = q_t + (bc * 128 + cc) * ld_qt + br * 128 + hh * 64;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint4 o;
    o.x = src[4 * k]; o.y = src[4 * k + 1]; o.z = src[4 * k + 2]; o.w = src[4 * k + 3];
    reinterpret_cast<uint4*>(dst)[k] = o;
  }
  }
  __syncthreads();                                // group_max / tile are reused by the next block
  }
}

// ---------------------------------------------------------------------------
// FP8 -> FP8 re-tiling of 1x128 codes into 128x1 tiles (output transposed),
// the backward-pass conversion of cached activations: dssusan.co.kr FP8
// excerpt, paragraph 4 (with power-of-2 scales, paragraph 1).  A workgroup
// handles a 128-row x 128-column tile, i.e. exactly one 1x128 group per row.
// Thread t holds rows 4*(t/8)..+3 of the 16 columns 16*(t%8)..+15.
//   1. 16-byte code loads, one 16-byte load of its 4 row scales; decode with
//      v_cvt_pk_f32_fp8 and dequantize in FP32 (exact for power-of-2 scales)
//   2. column max on the bits of |x|: 4 rows in registers, lanes t and t+8
//      via DPP row_ror:8, 16 partials per column through LDS
//   3. threads 0..127 finish one column each (scale pair, store s, publish inv)
//   4. scale + cast; each column's 4 rows pack into one dword, staged in an
//      LDS tile T[col][row] (pitch 132 bytes); thread t then copies 64 bytes
//      of column t/2 (rows 64*(t%2)..+63) to the output.
// ---------------------------------------------------------------------------
constexpr int kRqPartPitch = 132;   // dwords per LDS row of column partials

template <int MODE>
__global__ __launch_bounds__(256) void requant_128x1_kernel(
    const uint8_t* __restrict__ q, int64_t rows, int64_t cols, int64_t ld_q,
    const float* __restrict__ s_in, uint8_t* __restrict__ q_t, int64_t ld_qt, float* __restrict__ s_out) {
  // The column partials (steps 2-3) and the transposed tile (step 4) are live
  // at different times, between barriers, and share one LDS buffer.
  constexpr int kPartWords = 16 * kRqPartPitch;
  constexpr int kTileWords = 128 * kT1Pitch / 4;
  __shared__ uint32_t buf[kPartWords > kTileWords ? kPartWords : kTileWords];
  __shared__ float inv_s[128];
  uint32_t* const part = buf;
  uint32_t* const tile = buf;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int c8 = t & 7;
  const int q4 = t >> 3;
  const int64_t ctiles = cols >> 7;
  const int64_t tiles = ctiles * (rows >> 7);
  for (int64_t u = blockIdx.x; u < tiles; u += gridDim.x) {   // block-uniform: barriers stay matched
  const int64_t cg = u % ctiles;
  const int64_t rblk = u / ctiles;
  const int64_t row0 = rblk * 128;
  const int64_t col0 = cg * 128;

  u32x4 w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w[j] = *reinterpret_cast<const u32x4*>(q + (row0 + q4 * 4 + j) * ld_q + col0 + c8 * 16);
  const v4f sr = *reinterpret_cast<const v4f*>(s_in + cg * rows + row0 + q4 * 4);

  // Dequantized value i (column c8*16 + i) of row j: decoded again where it is
  // needed instead of held (keeps the kernel at 8 waves per SIMD).
  auto deq = [&](int j, int i) {
    const int word = int(w[j][i >> 2]);
    const auto pr = ((i >> 1) & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(word, true)
                                   : __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
    return pr[i & 1] * sr[j];
  };
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t b = __float_as_uint(deq(j, i)) & 0x7FFFFFFFu;
      m = b > m ? b : m;
    }
    m = FP8Q_DPP_MAX(m, 0x128);                   // row_ror:8 -> lanes l and l+8 of a DPP row
    if ((lane & 15) < 8) part[((t >> 6) * 4 + ((lane >> 4) & 3)) * kRqPartPitch + c8 * 16 + i] = m;
  }
  __syncthreads();
  if (t < 128) {
    uint32_t m = part[t];
#pragma unroll
    for (int p = 1; p < 16; ++p) {
      const uint32_t b = part[p * kRqPartPitch + t];
      m = b > m ? b : m;
    }
    const ScalePair sp = scale_from_amax_bits<MODE>(m);
    inv_s[t] = sp.inv;
    s_out[rblk * cols + col0 + t] = sp.s;
  }
  __syncthreads();                                // partials consumed: the buffer becomes the tile
  // Opaque to the compiler: the decode below is recomputed from the 16 code
  // registers rather than the 64 values of the first pass kept alive.
#pragma unroll
  for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(w[j]));
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float inv = inv_s[c8 * 16 + i];
    tile[((c8 * 16 + i) * kT1Pitch + q4 * 4) >> 2] = cvt4<MODE>(deq(0, i), deq(1, i), deq(2, i), deq(3, i), inv);
  }
  __syncthreads();
  const int cc = t >> 1;
  const int hh = t & 1;
  const uint32_t* src = tile + ((cc * kT1Pitch + hh * 64) >> 2);
  uint8_t* dst = q_t + (col0 + cc) * ld_qt + row0 + hh * 64;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    reinterpret_cast<u32x4*>(dst)[k] = u32x4{src[4 * k], src[4 * k + 1], src[4 * k + 2], src[4 * k + 3]};
  __syncthreads();                                // LDS is reused by the next tile
  }
}

// ---------------------------------------------------------------------------
// Launchers (shapes already validated by the ABI layer).
// ---------------------------------------------------------------------------
#define FP8Q_DISPATCH(KERNEL, bf16, mode, grid, st, ...)                                  \
  do {                                                                                    \
    if (bf16) {                                                                           \
      if (mode == kModePow2)                                                              \
        hipLaunchKernelGGL((KERNEL<uint16_t, kModePow2>), grid, dim3(256), 0, st,         \
                           static_cast<const uint16_t*>(x_), __VA_ARGS__);                \
      else                                                                                \
        hipLaunchKernelGGL((KERNEL<uint16_t, kModeMaxAbs>), grid, dim3(256), 0, st,       \
                           static_cast<const uint16_t*>(x_), __VA_ARGS__);                \
    } else {                                                                              \
      if (mode == kModePow2)                                                              \
        hipLaunchKernelGGL((KERNEL<float, kModePow2>), grid, dim3(256), 0, st,            \
                           static_cast<const float*>(x_), __VA_ARGS__);                   \
      else                                                                                \
        hipLaunchKernelGGL((KERNEL<float, kModeMaxAbs>), grid, dim3(256), 0, st,          \
                           static_cast<const float*>(x_), __VA_ARGS__);                   \
    }                                                                                     \
  } while (0)

// One work unit per workgroup (measured fastest on MI355X against 2, 4, 6, 8
// and 12 persistent workgroups per CU); the kernels' grid-stride loops only
// matter for grids beyond the 2^31-1 limit.
static unsigned unit_grid(int64_t units) {
  const int64_t cap = 0x7FFFFFFF;
  return unsigned(units < cap ? units : cap);
}

hipError_t launch_quant_1x128(const void* x_, bool bf16, int64_t rows, int64_t cols, int64_t ld_x,
                              int mode, uint8_t* q, int64_t ld_q, float* scales, hipStream_t st) {
  const dim3 grid(unit_grid(((rows + 31) / 32) * ((cols / 128 + 3) / 4)));
  FP8Q_DISPATCH(quant_1x128_kernel, bf16, mode, grid, st, rows, cols, ld_x, q, ld_q, scales);
  return hipGetLastError();
}

hipError_t launch_quant_128x1(const void* x_, bool bf16, int64_t rows, int64_t cols, int64_t ld_x,
                              int mode, uint8_t* q, int64_t ld_q, float* scales, hipStream_t st) {
  const dim3 grid(unit_grid(((cols + 63) / 64) * (rows / 128)));
  FP8Q_DISPATCH(quant_128x1_kernel, bf16, mode, grid, st, rows, cols, ld_x, q, ld_q, scales);
  return hipGetLastError();
}

hipError_t launch_quant_128x128(const void* x_, bool bf16, int64_t rows, int64_t cols, int64_t ld_w,
                                int mode, uint8_t* q, int64_t ld_q, float* scales,
                                uint8_t* q_t, int64_t ld_qt, float* scales_t, hipStream_t st) {
  const dim3 grid(unit_grid((cols / 128) * (rows / 128)));
  FP8Q_DISPATCH(quant_128x128_kernel, bf16, mode, grid, st, rows, cols, ld_w, q, ld_q, scales, q_t, ld_qt,
                scales_t);
  return hipGetLastError();
}

#undef FP8Q_DISPATCH

hipError_t launch_requant_128x1(const uint8_t* q, int64_t rows, int64_t cols, int64_t ld_q, const float* s_in,
                                int mode, uint8_t* q_t, int64_t ld_qt, float* s_out, hipStream_t st) {
  const dim3 grid(unit_grid((cols / 128) * (rows / 128)));
  if (mode == kModePow2)
    hipLaunchKernelGGL((requant_128x1_kernel<kModePow2>), grid, dim3(256), 0, st, q, rows, cols, ld_q, s_in,
                       q_t, ld_qt, s_out);
  else
    hipLaunchKernelGGL((requant_128x1_kernel<kModeMaxAbs>), grid, dim3(256), 0, st, q, rows, cols, ld_q, s_in,
                       q_t, ld_qt, s_out);
  return hipGetLastError();
}

}  // namespace fp8q
