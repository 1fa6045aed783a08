// Online fine-grained FP8 quantizers for gfx950.
//
//  * 1x128 tiles (one token x 128 channels), scales [cols/128][rows]
//  * 128x1 tiles (128 tokens x one channel), codes written transposed
//  * 128x128 blocks (weights), optional transposed copy for Dgrad
//
// Tile shapes and the max-abs -> scale -> cast sequence: dssusan.co.kr FP8
// excerpt, paragraphs 2 and 4; "Deepseek - Not For everyone", paragraph 3;
// power-of-2 scales: dssusan.co.kr FP8 excerpt, paragraph 1.
//
// All three kernels are HBM-bound streaming passes: 16-byte coalesced loads,
// max-abs reduced across lanes with DPP (and LDS across waves where a group
// spans waves), one scale pair per group, v_cvt_pk_fp8_f32 for the cast.
#include "fp8q_device.h"
#include "fp8q_launch.h"

namespace fp8q {

// ---------------------------------------------------------------------------
// 1x128: a workgroup is 4 waves; wave w quantizes group (4*blockIdx.y + w) of
// 16 consecutive rows starting at 16*blockIdx.x.  A 16-lane DPP row holds one
// 128-element tile row (8 elements per lane), so the four DPP rows of a wave
// cover 4 rows per step and 4 unrolled steps cover 16 rows.  All loads are
// issued before any reduction.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void quant_1x128_kernel(
    const T* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x, int mode,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t groups = cols >> 7;
  const int64_t g = int64_t(blockIdx.y) * 4 + wave;
  if (g >= groups) return;                       // wave-uniform; no barriers below
  const int sub = lane >> 4;                      // DPP row = tile row within a step
  const int seg = lane & 15;                      // 8-element segment of the tile
  const int64_t row0 = int64_t(blockIdx.x) * 16;
  const int64_t col = g * 128 + seg * 8;

  float v[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = row0 + i * 4 + sub;
    if (r < rows) {
      Load8<T>::run(x + r * ld_x + col, v[i]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i][j] = 0.0f;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float m = fabsf(v[i][0]);
#pragma unroll
    for (int j = 1; j < 8; ++j) m = fmaxf(m, fabsf(v[i][j]));
    m = row16_max(m);
    const ScalePair sp = scale_from_amax(m, mode);
    const int64_t r = row0 + i * 4 + sub;
    uint2 out;
    out.x = pack4_e4m3(v[i][0] * sp.inv, v[i][1] * sp.inv, v[i][2] * sp.inv, v[i][3] * sp.inv);
    out.y = pack4_e4m3(v[i][4] * sp.inv, v[i][5] * sp.inv, v[i][6] * sp.inv, v[i][7] * sp.inv);
    if (r < rows) {
      *reinterpret_cast<uint2*>(q + r * ld_q + col) = out;
      if (seg == 0) scales[g * rows + r] = sp.s;
    }
  }
}

// ---------------------------------------------------------------------------
// 128x1 with transposed output: a workgroup quantizes a 128-row x 64-column
// tile.  Thread t loads rows 4*(t/8)..+3 of the 8 columns 8*(t%8)..+7.
//   1. per-thread column max over its 4 rows -> LDS [32][64]
//   2. wave 0 finishes each column's max over the 32 partials, derives the
//      scale pair, stores s and publishes inv in LDS
//   3. every thread scales its 4x8 values and packs each column's 4 rows into
//      one dword (so the bytes are already in transposed order), stores them
//      into an LDS tile T[col][row] (pitch 132 bytes: conflict-free writes)
//   4. thread t copies 32 bytes of column t/4 (rows 32*(t%4)..+31) to q.
// ---------------------------------------------------------------------------
constexpr int kT1Pitch = 132;   // bytes per LDS row of the transposed tile

template <typename T>
__global__ __launch_bounds__(256) void quant_128x1_kernel(
    const T* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x, int mode,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scales) {
  __shared__ float part[32][64];
  __shared__ float inv_s[64];
  __shared__ uint32_t tile[64 * kT1Pitch / 4];

  const int t = threadIdx.x;
  const int c8 = t & 7;
  const int q4 = t >> 3;
  const int64_t col0 = int64_t(blockIdx.x) * 64;
  const int64_t row0 = int64_t(blockIdx.y) * 128;
  const int64_t col = col0 + c8 * 8;
  const bool col_ok = col < cols;                 // cols % 8 == 0: all-or-nothing per thread

  float v[4][8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (col_ok) {
      Load8<T>::run(x + (row0 + q4 * 4 + j) * ld_x + col, v[j]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[j][i] = 0.0f;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float m = fabsf(v[0][i]);
#pragma unroll
    for (int j = 1; j < 4; ++j) m = fmaxf(m, fabsf(v[j][i]));
    part[q4][c8 * 8 + i] = m;
  }
  __syncthreads();
  if (t < 64) {
    float m = part[0][t];
#pragma unroll
    for (int p = 1; p < 32; ++p) m = fmaxf(m, part[p][t]);
    const ScalePair sp = scale_from_amax(m, mode);
    inv_s[t] = sp.inv;
    if (col0 + t < cols) scales[int64_t(blockIdx.y) * cols + col0 + t] = sp.s;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float inv = inv_s[c8 * 8 + i];
    const uint32_t w = pack4_e4m3(v[0][i] * inv, v[1][i] * inv, v[2][i] * inv, v[3][i] * inv);
    tile[((c8 * 8 + i) * kT1Pitch + q4 * 4) >> 2] = w;
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
}

// ---------------------------------------------------------------------------
// 128x128 blocks: one workgroup per block.  Thread t owns the 8 columns
// 8*(t%16)..+7 of rows {4*(t/16)+j, 64+4*(t/16)+j : j=0..3}.
//   1. thread max -> DPP max over the 16 lanes of a row -> LDS across the 4
//      rows of a wave and the 4 waves; every thread reads the block max
//   2. row-major codes: 8 bytes per (thread, row), 128-byte runs per row
//   3. optional transposed copy: each column's 4 adjacent rows are packed into
//      one dword, staged in an LDS tile T[col][row] (pitch 132 bytes), and
//      thread t copies 64 bytes of column t/2 (rows 64*(t%2)..+63) to q_t.
// ---------------------------------------------------------------------------
constexpr int kBPitch = 132;

template <typename T>
__global__ __launch_bounds__(256) void quant_128x128_kernel(
    const T* __restrict__ w, int64_t rows, int64_t cols, int64_t ld_w, int mode,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scales,
    uint8_t* __restrict__ q_t, int64_t ld_qt, float* __restrict__ scales_t) {
  __shared__ float wave_max[16];
  __shared__ uint32_t tile[128 * kBPitch / 4];

  const int t = threadIdx.x;
  const int c16 = t & 15;
  const int rq = t >> 4;                          // 0..15
  const int64_t bc = blockIdx.x, br = blockIdx.y;
  const int64_t col = bc * 128 + c16 * 8;
  const int64_t row_base = br * 128 + rq * 4;

  float v[8][8];                                  // [j][i]: row (j/4)*64 + 4*rq + j%4, col 8*c16 + i
#pragma unroll
  for (int j = 0; j < 8; ++j)
    Load8<T>::run(w + (row_base + (j >> 2) * 64 + (j & 3)) * ld_w + col, v[j]);

  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[j][i]));
  m = row16_max(m);
  if (c16 == 0) wave_max[rq] = m;
  __syncthreads();
  m = wave_max[0];
#pragma unroll
  for (int p = 1; p < 16; ++p) m = fmaxf(m, wave_max[p]);
  const ScalePair sp = scale_from_amax(m, mode);
  if (t == 0) {
    scales[br * (cols >> 7) + bc] = sp.s;
    if (scales_t) scales_t[bc * (rows >> 7) + br] = sp.s;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) v[j][i] *= sp.inv;

#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint2 out;
    out.x = pack4_e4m3(v[j][0], v[j][1], v[j][2], v[j][3]);
    out.y = pack4_e4m3(v[j][4], v[j][5], v[j][6], v[j][7]);
    *reinterpret_cast<uint2*>(q + (row_base + (j >> 2) * 64 + (j & 3)) * ld_q + col) = out;
  }
  if (q_t == nullptr) return;                      // block-uniform: no barrier is skipped by part of the block

#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t wcol = pack4_e4m3(v[4 * h][i], v[4 * h + 1][i], v[4 * h + 2][i], v[4 * h + 3][i]);
      tile[((c16 * 8 + i) * kBPitch + h * 64 + rq * 4) >> 2] = wcol;
    }
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

// ---------------------------------------------------------------------------
// Launchers (shapes already validated by the ABI layer).
// ---------------------------------------------------------------------------
hipError_t launch_quant_1x128(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld_x,
                              int mode, uint8_t* q, int64_t ld_q, float* scales, hipStream_t st) {
  const int64_t groups = cols / 128;
  dim3 grid(unsigned((rows + 15) / 16), unsigned((groups + 3) / 4));
  if (bf16)
    hipLaunchKernelGGL(quant_1x128_kernel<uint16_t>, grid, dim3(256), 0, st,
                       static_cast<const uint16_t*>(x), rows, cols, ld_x, mode, q, ld_q, scales);
  else
    hipLaunchKernelGGL(quant_1x128_kernel<float>, grid, dim3(256), 0, st,
                       static_cast<const float*>(x), rows, cols, ld_x, mode, q, ld_q, scales);
  return hipGetLastError();
}

hipError_t launch_quant_128x1(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld_x,
                              int mode, uint8_t* q, int64_t ld_q, float* scales, hipStream_t st) {
  dim3 grid(unsigned((cols + 63) / 64), unsigned(rows / 128));
  if (bf16)
    hipLaunchKernelGGL(quant_128x1_kernel<uint16_t>, grid, dim3(256), 0, st,
                       static_cast<const uint16_t*>(x), rows, cols, ld_x, mode, q, ld_q, scales);
  else
    hipLaunchKernelGGL(quant_128x1_kernel<float>, grid, dim3(256), 0, st,
                       static_cast<const float*>(x), rows, cols, ld_x, mode, q, ld_q, scales);
  return hipGetLastError();
}

hipError_t launch_quant_128x128(const void* w, bool bf16, int64_t rows, int64_t cols, int64_t ld_w,
                                int mode, uint8_t* q, int64_t ld_q, float* scales,
                                uint8_t* q_t, int64_t ld_qt, float* scales_t, hipStream_t st) {
  dim3 grid(unsigned(cols / 128), unsigned(rows / 128));
  if (bf16)
    hipLaunchKernelGGL(quant_128x128_kernel<uint16_t>, grid, dim3(256), 0, st,
                       static_cast<const uint16_t*>(w), rows, cols, ld_w, mode, q, ld_q, scales,
                       q_t, ld_qt, scales_t);
  else
    hipLaunchKernelGGL(quant_128x128_kernel<float>, grid, dim3(256), 0, st,
                       static_cast<const float*>(w), rows, cols, ld_w, mode, q, ld_q, scales,
                       q_t, ld_qt, scales_t);
  return hipGetLastError();
}

}  // namespace fp8q
