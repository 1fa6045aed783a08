// Online fine-grained FP8 quantizers for gfx950.
//
//  * 1x128 tiles (one token x 128 channels), scales [cols/128][rows]
//  * 128x1 tiles (128 tokens x one channel), codes written transposed
//  * 128x128 blocks (weights), optional transposed copy for Dgrad; without
//    it, BF16 weights go two blocks per workgroup
//  * 1x128 and 128x1 tiles of one tensor in one pass
//  * FP8 -> FP8 re-tiling of 1x128 codes into 128x1 tiles (backward pass),
//    by the 128x1 kernel reading codes and their row scales
//
// Tile shapes and the max-abs -> scale -> cast sequence: dssusan.co.kr FP8
// excerpt, paragraphs 2 and 4; "Deepseek - Not For everyone", paragraph 3;
// power-of-2 scales: dssusan.co.kr FP8 excerpt, paragraph 1.
//
// All five kernels are HBM-bound streaming passes: 16-byte coalesced loads,
// max-abs taken on the integer bit patterns of |x| (non-negative floats order
// like their bits; BF16 pairs reduce two at a time with v_pk_max_u16),
// reduced across lanes with DPP and the gfx950 permlane swaps (and LDS across
// waves where a group spans waves), one scale pair per group,
// v_cvt_pk_fp8_f32 for the cast.  The scale
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
  __device__ __forceinline__ void opaque() { asm volatile("" : "+v"(w)); }
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
  __device__ __forceinline__ void opaque() { asm volatile("" : "+v"(w0), "+v"(w1)); }
  __device__ __forceinline__ float get(int i) const { return __uint_as_float(i < 4 ? w0[i] : w1[i - 4]); }
};

// Eight FP8 (E4M3) codes of one row with that row's 1x128 scale: element i
// is the dequantized value fl32(dec(code_i) * s), exact for power-of-2
// scales.  With it the 128x1 kernel below is also the FP8 -> FP8 re-tiling of
// cached 1x128 codes into 128x1 tiles, the backward-pass conversion of
// dssusan.co.kr FP8 excerpt, paragraph 4 (measured 31.6 us on the 8192x7168
// activation against 33.5 us for a dedicated 128x128-tile kernel that decoded
// every code twice).
template <> struct Raw8<uint8_t> {
  uint32_t w0, w1;
  float s;
  __device__ __forceinline__ void load(const uint8_t* p) {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    w0 = x.x;
    w1 = x.y;
  }
  __device__ __forceinline__ void zero() { w0 = w1 = 0u; s = 0.0f; }
  __device__ __forceinline__ void opaque() { asm volatile("" : "+v"(w0), "+v"(w1)); }
  __device__ __forceinline__ float get(int i) const {
    const int word = int(i < 4 ? w0 : w1);
    const auto pr = ((i >> 1) & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(word, true)
                                   : __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
    return pr[i & 1] * s;
  }
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
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scales, const float* __restrict__ s_in = nullptr) {
  __shared__ uint32_t part[16][64];
  __shared__ float inv_s[64];
  __shared__ uint32_t tile[64 * kT1Pitch / 4];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int c8 = t & 7;
  const int q4 = t >> 3;
  const int64_t ctiles = (cols + 63) >> 6;
  const int64_t rtiles = rows >> 7;
  const int64_t tiles = ctiles * rtiles;
  // Column-major tile order: consecutive workgroups take consecutive row
  // blocks of one 64-column strip, so together they write whole runs of each
  // transposed output row (measured on the 8192x18432 gradient: 98.5 -> 87.0
  // us against row-band order, whose neighbours write 128-byte pieces of
  // different output rows).
  for (int64_t u = blockIdx.x; u < tiles; u += gridDim.x) {   // block-uniform: barriers stay matched
  const int64_t col0 = (u / rtiles) * 64;
  const int64_t rblk = u % rtiles;
  const int64_t row0 = rblk * 128;
  const int64_t col = col0 + c8 * 8;
  const bool col_ok = col < cols;                 // cols % 8 == 0: all-or-nothing per thread

  Raw8<T> v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (col_ok) v[j].load(x + (row0 + q4 * 4 + j) * ld_x + col);
    else v[j].zero();
  }
  if constexpr (sizeof(T) == 1) {                 // FP8 codes (cols % 128 == 0): their 1x128 row scales [cols/128][rows]
    const v4f sr = *reinterpret_cast<const v4f*>(s_in + (col0 >> 7) * rows + row0 + q4 * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j].s = sr[j];
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
// 128x128 blocks: one 512-thread workgroup per block.  Thread t owns the 8
// columns 8*(t%16)..+7 of the 4 rows 4*(t/16)..+3.
//   1. thread max (bits of |x|) -> DPP max over the 16 lanes of a row ->
//      v_permlane32_swap / v_permlane16_swap across the wave's 4 DPP rows ->
//      LDS across the 8 waves; every thread reads the block max
//   2. row-major codes: 8 bytes per (thread, row), 128-byte runs per row
//   3. optional transposed copy: each column's 4 adjacent rows are packed into
//      one dword, staged in an LDS tile T[col][row] (pitch 132 bytes), and
//      thread t copies 32 bytes of column t/4 (rows 32*(t%4)..+31) to q_t.
// BF16 input is held to 64 VGPRs (8 waves per SIMD): measured 5% faster on
// the 18432x7168 weight with its transposed copy than 256 threads with 8 rows
// each at 4 waves per SIMD (the same on the 131072x7168 expert weights).
// ---------------------------------------------------------------------------
constexpr int kBPitch = 132;

// Block (row, column) of work unit u for the kernels that write row-major and
// transposed codes of 128x128 blocks: 2x2 groups of blocks in row-band order,
// column-major inside a group, so both outputs leave in 256-byte runs of
// neighbouring workgroups rather than one of them in 128-byte pieces.
// Measured against row-band order: the 18432x7168 weight with its transposed
// copy 93.0 -> 90.4 us, the one-pass 1x128 + 128x1 quantizer of the 8192x18432
// gradient 113.7 -> 111.0 us (4x4 and 8x1 groups gained nothing).  Row-band
// order where the block counts are odd.
__device__ __forceinline__ void order_2x2(int64_t u, int64_t rblocks, int64_t cblocks, int64_t& br, int64_t& bc) {
  if (((rblocks | cblocks) & 1) == 0) {
    const int64_t grp = u >> 2, w = u & 3, gcols = cblocks >> 1;
    br = (grp / gcols) * 2 + (w & 1);
    bc = (grp % gcols) * 2 + (w >> 1);
  } else {
    br = u / cblocks;
    bc = u % cblocks;
  }
}


template <typename T, int MODE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 8 : 4, 8)))
void quant_128x128_kernel(
    const T* __restrict__ w, int64_t rows, int64_t cols, int64_t ld_w,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scales,
    uint8_t* __restrict__ q_t, int64_t ld_qt, float* __restrict__ scales_t) {
  __shared__ uint32_t wave_max[8];
  __shared__ uint32_t tile[128 * kBPitch / 4];
  const int t = threadIdx.x;
  const int c16 = t & 15;
  const int rq = t >> 4;                          // 0..31: rows 4*rq..+3
  const int64_t cblocks = cols >> 7;
  const int64_t nblocks = cblocks * (rows >> 7);
  for (int64_t u = blockIdx.x; u < nblocks; u += gridDim.x) {   // block-uniform: barriers stay matched
  int64_t bc, br;                                 // block-uniform
  if (q_t) order_2x2(u, rows >> 7, cblocks, br, bc);
  else { bc = u % cblocks; br = u / cblocks; }   // row-major codes only: row-band order
  const int64_t col = bc * 128 + c16 * 8;
  const int64_t row_base = br * 128 + rq * 4;
  Raw8<T> v[4];                                   // [j]: row 4*rq + j, cols 8*c16..+7
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j].load(w + (row_base + j) * ld_w + col);
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t b = v[j].amax_bits();
    m = b > m ? b : m;
  }
  m = row16_max_u32(m);
  {                                               // lanes l, l^16, l^32, l^48
    const auto a = __builtin_amdgcn_permlane32_swap(m, m, false, false);
    const uint32_t y = uint32_t(a[0]) > uint32_t(a[1]) ? uint32_t(a[0]) : uint32_t(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(y, y, false, false);
    m = uint32_t(b[0]) > uint32_t(b[1]) ? uint32_t(b[0]) : uint32_t(b[1]);
  }
  if ((t & 63) == 0) wave_max[t >> 6] = m;
  __syncthreads();
  m = wave_max[0];
#pragma unroll
  for (int p = 1; p < 8; ++p) m = wave_max[p] > m ? wave_max[p] : m;
  const ScalePair sp = scale_from_amax_bits<MODE>(m);
  if (t == 0) {
    scales[br * cblocks + bc] = sp.s;
    if (scales_t) scales_t[bc * (rows >> 7) + br] = sp.s;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint2 out;
    out.x = cvt4<MODE>(v[j].get(0), v[j].get(1), v[j].get(2), v[j].get(3), sp.inv);
    out.y = cvt4<MODE>(v[j].get(4), v[j].get(5), v[j].get(6), v[j].get(7), sp.inv);
    *reinterpret_cast<uint2*>(q + (row_base + j) * ld_q + col) = out;
  }
  if (q_t != nullptr) {                            // block-uniform: no barrier is skipped by part of the block
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j].opaque();      // unpack again rather than hold the unpacked values
#pragma unroll
  for (int i = 0; i < 8; ++i)
    tile[((c16 * 8 + i) * kBPitch + rq * 4) >> 2] =
        cvt4<MODE>(v[0].get(i), v[1].get(i), v[2].get(i), v[3].get(i), sp.inv);
  __syncthreads();
  const int cc = t >> 2;
  const int hh = t & 3;
  const uint32_t* src = tile + ((cc * kBPitch + hh * 32) >> 2);
  uint8_t* dst = q_t + (bc * 128 + cc) * ld_qt + br * 128 + hh * 32;
#pragma unroll
  for (int k = 0; k < 2; ++k)
    reinterpret_cast<u32x4*>(dst)[k] = u32x4{src[4 * k], src[4 * k + 1], src[4 * k + 2], src[4 * k + 3]};
  }
  __syncthreads();                                // wave_max / tile are reused by the next block
  }
}


// BF16 128x128 blocks, row-major codes only, two horizontally adjacent blocks
// per 512-thread workgroup (128 rows x 256 columns): thread t owns the 16
// columns 16*(t%16)..+15 of rows 4*(t/16)..+3, so lanes 0-7 of a DPP row hold
// the left block and lanes 8-15 the right one; each block's max goes over
// its 8 lanes (quad permutes + row_half_mirror), across the wave's 4 DPP rows
// with the permlane swaps and across the 8 waves through LDS.  Each thread
// keeps two 16-byte loads per row in flight (64 VGPRs, still 8 waves per
// SIMD), twice the one-block kernel's, and the codes leave as 512-byte row
// pieces: measured on the 131072x7168 expert weights 527 -> 508 us.
template <int MODE>
__global__ __launch_bounds__(512) void quant_128x256_kernel(
    const uint16_t* __restrict__ w, int64_t rows, int64_t cols, int64_t ld_w,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scales) {
  __shared__ uint32_t wave_max[8][2];
  const int t = threadIdx.x;
  const int c16 = t & 15;
  const int rq = t >> 4;
  const int half = c16 >> 3;
  const int64_t cpairs = cols >> 8;
  const int64_t cblocks = cols >> 7;
  const int64_t nunits = cpairs * (rows >> 7);
  for (int64_t u = blockIdx.x; u < nunits; u += gridDim.x) {   // block-uniform: barriers stay matched
  const int64_t bp = u % cpairs, br = u / cpairs;
  const int64_t col = bp * 256 + c16 * 16;
  const int64_t row_base = br * 128 + rq * 4;
  Raw8<uint16_t> v[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j][0].load(w + (row_base + j) * ld_w + col);
    v[j][1].load(w + (row_base + j) * ld_w + col + 8);
  }
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t b = v[j][h].amax_bits();
      m = b > m ? b : m;
    }
  m = FP8Q_DPP_MAX(m, 0xB1);
  m = FP8Q_DPP_MAX(m, 0x4E);
  m = FP8Q_DPP_MAX(m, 0x141);                     // max over the 8 lanes of this block
  {                                               // lanes l, l^16, l^32, l^48
    const auto a = __builtin_amdgcn_permlane32_swap(m, m, false, false);
    const uint32_t y = uint32_t(a[0]) > uint32_t(a[1]) ? uint32_t(a[0]) : uint32_t(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(y, y, false, false);
    m = uint32_t(b[0]) > uint32_t(b[1]) ? uint32_t(b[0]) : uint32_t(b[1]);
  }
  if ((t & 55) == 0) wave_max[t >> 6][(t >> 3) & 1] = m;   // lanes 0 and 8 of each wave
  __syncthreads();
  m = wave_max[0][half];
#pragma unroll
  for (int p = 1; p < 8; ++p) m = wave_max[p][half] > m ? wave_max[p][half] : m;
  const ScalePair sp = scale_from_amax_bits<MODE>(m);
  if (t == 0 || t == 8) scales[br * cblocks + bp * 2 + half] = sp.s;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 out = {cvt4<MODE>(v[j][0].get(0), v[j][0].get(1), v[j][0].get(2), v[j][0].get(3), sp.inv),
                       cvt4<MODE>(v[j][0].get(4), v[j][0].get(5), v[j][0].get(6), v[j][0].get(7), sp.inv),
                       cvt4<MODE>(v[j][1].get(0), v[j][1].get(1), v[j][1].get(2), v[j][1].get(3), sp.inv),
                       cvt4<MODE>(v[j][1].get(4), v[j][1].get(5), v[j][1].get(6), v[j][1].get(7), sp.inv)};
    *reinterpret_cast<u32x4*>(q + (row_base + j) * ld_q + col) = out;
  }
  __syncthreads();                                // wave_max is reused by the next unit
  }
}

// ---------------------------------------------------------------------------
// Both tilings of one tensor in one pass (dssusan.co.kr FP8 excerpt,
// paragraph 4: the backward pass needs the output gradient in 1x128 tiles for
// Dgrad and in 128x1 tiles for Wgrad).  The codes and scales are exactly those
// of the 1x128 and 128x1 kernels; the input is read once instead of twice.
// One 512-thread workgroup per 128x128 block; thread t owns the 8 columns
// 8*(t%16)..+7 of the 4 rows 4*(t/16)..+3.
//   1. 1x128: each of the thread's 4 rows reduces over the 16 lanes of its DPP
//      row; scale, cast and store the row-major codes and the row scales
//   2. 128x1: per-column max over the thread's 4 rows (BF16 pairs two at a
//      time), across the 4 DPP rows of the wave with v_permlane32_swap and
//      v_permlane16_swap, across the 8 waves through LDS; every thread then
//      derives the scale pairs of its own 8 columns (no second barrier)
//   3. transposed codes staged in an LDS tile T[col][row] (pitch 132 bytes)
//      and copied out 32 bytes per thread.
// BF16 input is held to 64 VGPRs (8 waves per SIMD, 4 workgroups per CU):
// measured 8% faster on the 8192x18432 output gradient than 256 threads with
// 8 rows each at 5 waves per SIMD.
// ---------------------------------------------------------------------------
template <typename T> struct ColAmax;
template <> struct ColAmax<uint16_t> {            // 4 words, each the max bits of two BF16 columns
  u16x2 m[4];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int k = 0; k < 4; ++k) m[k] = u16x2{0, 0};
  }
  __device__ __forceinline__ void add(const Raw8<uint16_t>& v) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      m[k] = __builtin_elementwise_max(m[k], __builtin_bit_cast(u16x2, v.w[k] & 0x7FFF7FFFu));
  }
  __device__ __forceinline__ void wave_reduce() {   // lanes l, l^16, l^32, l^48 hold the same columns
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t x = __builtin_bit_cast(uint32_t, m[k]);
      const auto a = __builtin_amdgcn_permlane32_swap(x, x, false, false);
      u16x2 y = __builtin_elementwise_max(__builtin_bit_cast(u16x2, uint32_t(a[0])),
                                          __builtin_bit_cast(u16x2, uint32_t(a[1])));
      const uint32_t z = __builtin_bit_cast(uint32_t, y);
      const auto b = __builtin_amdgcn_permlane16_swap(z, z, false, false);
      m[k] = __builtin_elementwise_max(__builtin_bit_cast(u16x2, uint32_t(b[0])),
                                       __builtin_bit_cast(u16x2, uint32_t(b[1])));
    }
  }
  __device__ __forceinline__ uint32_t bits(int i) const {   // float32 bits of column i's max |x|
    return uint32_t((i & 1) ? m[i >> 1].y : m[i >> 1].x) << 16;
  }
};
template <> struct ColAmax<float> {
  uint32_t m[8];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = 0;
  }
  __device__ __forceinline__ void add(const Raw8<float>& v) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t b = __float_as_uint(v.get(i)) & 0x7FFFFFFFu;
      m[i] = b > m[i] ? b : m[i];
    }
  }
  __device__ __forceinline__ void wave_reduce() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const auto a = __builtin_amdgcn_permlane32_swap(m[i], m[i], false, false);
      const uint32_t y = uint32_t(a[0]) > uint32_t(a[1]) ? uint32_t(a[0]) : uint32_t(a[1]);
      const auto b = __builtin_amdgcn_permlane16_swap(y, y, false, false);
      m[i] = uint32_t(b[0]) > uint32_t(b[1]) ? uint32_t(b[0]) : uint32_t(b[1]);
    }
  }
  __device__ __forceinline__ uint32_t bits(int i) const { return m[i]; }
};

template <typename T, int MODE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 8 : 4, 8)))
void quant_dual_kernel(
    const T* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scales,
    uint8_t* __restrict__ q_t, int64_t ld_qt, float* __restrict__ scales_t) {
  __shared__ uint32_t col_part[8][128];           // per-wave column max bits
  __shared__ uint32_t tile[128 * kBPitch / 4];
  const int t = threadIdx.x;
  const int c16 = t & 15;
  const int rq = t >> 4;                          // 0..31: rows 4*rq..+3
  const int wave = t >> 6;
  const int64_t cblocks = cols >> 7;
  const int64_t nblocks = cblocks * (rows >> 7);
  for (int64_t u = blockIdx.x; u < nblocks; u += gridDim.x) {   // block-uniform: barriers stay matched
  int64_t bc, br;
  order_2x2(u, rows >> 7, cblocks, br, bc);
  const int64_t col = bc * 128 + c16 * 8;
  const int64_t row_base = br * 128 + rq * 4;
  Raw8<T> v[4];                                   // [j]: row 4*rq + j, cols 8*c16..+7
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j].load(x + (row_base + j) * ld_x + col);
  ColAmax<T> cm;
  cm.init();
#pragma unroll
  for (int j = 0; j < 4; ++j) cm.add(v[j]);
  cm.wave_reduce();
  if ((t & 63) < 16) {
#pragma unroll
    for (int i = 0; i < 8; ++i) col_part[wave][c16 * 8 + i] = cm.bits(i);
  }

  // 1x128: a tile row is one row of this block.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const ScalePair sp = scale_from_amax_bits<MODE>(row16_max_u32(v[j].amax_bits()));
    const int64_t r = row_base + j;
    uint2 out;
    out.x = cvt4<MODE>(v[j].get(0), v[j].get(1), v[j].get(2), v[j].get(3), sp.inv);
    out.y = cvt4<MODE>(v[j].get(4), v[j].get(5), v[j].get(6), v[j].get(7), sp.inv);
    *reinterpret_cast<uint2*>(q + r * ld_q + col) = out;
    if (c16 == 0) scales[bc * rows + r] = sp.s;
  }
  __syncthreads();

  // 128x1: a tile is one column of this block, written transposed.
  float inv_col[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = c16 * 8 + i;
    uint32_t m = col_part[0][c];
#pragma unroll
    for (int w = 1; w < 8; ++w) m = col_part[w][c] > m ? col_part[w][c] : m;
    const ScalePair sp = scale_from_amax_bits<MODE>(m);
    inv_col[i] = sp.inv;
    if (rq == 0) scales_t[br * cols + bc * 128 + c] = sp.s;
  }
  // Opaque raw words: the values are unpacked again here instead of the first
  // pass's unpacked values being held across the barrier.
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j].opaque();
#pragma unroll
  for (int i = 0; i < 8; ++i)
    tile[((c16 * 8 + i) * kBPitch + rq * 4) >> 2] =
        cvt4<MODE>(v[0].get(i), v[1].get(i), v[2].get(i), v[3].get(i), inv_col[i]);
  __syncthreads();
  const int cc = t >> 2;
  const int hh = t & 3;
  const uint32_t* src = tile + ((cc * kBPitch + hh * 32) >> 2);
  uint8_t* dst = q_t + (bc * 128 + cc) * ld_qt + br * 128 + hh * 32;
#pragma unroll
  for (int k = 0; k < 2; ++k)
    reinterpret_cast<u32x4*>(dst)[k] = u32x4{src[4 * k], src[4 * k + 1], src[4 * k + 2], src[4 * k + 3]};
  __syncthreads();                                // col_part / tile are reused by the next block
  }
}

// ---------------------------------------------------------------------------
// Launchers (shapes already validated by the ABI layer).
// ---------------------------------------------------------------------------
#define FP8Q_DISPATCH_T(KERNEL, threads, bf16, mode, grid, st, ...)                       \
  do {                                                                                    \
    if (bf16) {                                                                           \
      if (mode == kModePow2)                                                              \
        hipLaunchKernelGGL((KERNEL<uint16_t, kModePow2>), grid, dim3(threads), 0, st,     \
                           static_cast<const uint16_t*>(x_), __VA_ARGS__);                \
      else                                                                                \
        hipLaunchKernelGGL((KERNEL<uint16_t, kModeMaxAbs>), grid, dim3(threads), 0, st,   \
                           static_cast<const uint16_t*>(x_), __VA_ARGS__);                \
    } else {                                                                              \
      if (mode == kModePow2)                                                              \
        hipLaunchKernelGGL((KERNEL<float, kModePow2>), grid, dim3(threads), 0, st,        \
                           static_cast<const float*>(x_), __VA_ARGS__);                   \
      else                                                                                \
        hipLaunchKernelGGL((KERNEL<float, kModeMaxAbs>), grid, dim3(threads), 0, st,      \
                           static_cast<const float*>(x_), __VA_ARGS__);                   \
    }                                                                                     \
  } while (0)
#define FP8Q_DISPATCH(KERNEL, bf16, mode, grid, st, ...) \
  FP8Q_DISPATCH_T(KERNEL, 256, bf16, mode, grid, st, __VA_ARGS__)

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
  if (bf16 && q_t == nullptr && cols % 256 == 0) {
    const dim3 grid2(unit_grid((cols / 256) * (rows / 128)));
    const uint16_t* w = static_cast<const uint16_t*>(x_);
    if (mode == kModePow2)
      hipLaunchKernelGGL((quant_128x256_kernel<kModePow2>), grid2, dim3(512), 0, st, w, rows, cols, ld_w, q, ld_q, scales);
    else
      hipLaunchKernelGGL((quant_128x256_kernel<kModeMaxAbs>), grid2, dim3(512), 0, st, w, rows, cols, ld_w, q, ld_q,
                         scales);
    return hipGetLastError();
  }
  const dim3 grid(unit_grid((cols / 128) * (rows / 128)));
  FP8Q_DISPATCH_T(quant_128x128_kernel, 512, bf16, mode, grid, st, rows, cols, ld_w, q, ld_q, scales, q_t, ld_qt,
                scales_t);
  return hipGetLastError();
}

hipError_t launch_quant_dual(const void* x_, bool bf16, int64_t rows, int64_t cols, int64_t ld_x,
                             int mode, uint8_t* q, int64_t ld_q, float* scales,
                             uint8_t* q_t, int64_t ld_qt, float* scales_t, hipStream_t st) {
  const dim3 grid(unit_grid((cols / 128) * (rows / 128)));
  FP8Q_DISPATCH_T(quant_dual_kernel, 512, bf16, mode, grid, st, rows, cols, ld_x, q, ld_q, scales, q_t, ld_qt,
                  scales_t);
  return hipGetLastError();
}

#undef FP8Q_DISPATCH
#undef FP8Q_DISPATCH_T

// FP8 -> FP8 re-tiling: the 128x1 kernel reading 1x128 codes and their scales.
hipError_t launch_requant_128x1(const uint8_t* q, int64_t rows, int64_t cols, int64_t ld_q, const float* s_in,
                                int mode, uint8_t* q_t, int64_t ld_qt, float* s_out, hipStream_t st) {
  const dim3 grid(unit_grid((cols / 64) * (rows / 128)));
  if (mode == kModePow2)
    hipLaunchKernelGGL((quant_128x1_kernel<uint8_t, kModePow2>), grid, dim3(256), 0, st, q, rows, cols, ld_q,
                       q_t, ld_qt, s_out, s_in);
  else
    hipLaunchKernelGGL((quant_128x1_kernel<uint8_t, kModeMaxAbs>), grid, dim3(256), 0, st, q, rows, cols, ld_q,
                       q_t, ld_qt, s_out, s_in);
  return hipGetLastError();
}

}  // namespace fp8q
