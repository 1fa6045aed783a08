// Block-scaled FP8 GEMMs for gfx950: Fprop, Dgrad, Wgrad and grouped Fprop.
//
//   C[m][n] = sum_g  sa(g,m) * sb(g,n) * P_g[m][n],
//   P_g[m][n] = sum_{k in K-group g} dec(A[m][k]) * dec(B[n][k])
//
// Per-group scales along K, multiplied in as the dequantization step, with
// the partial products promoted to FP32 accumulation once per group:
// dssusan.co.kr FP8 excerpt, paragraph 3; "Deepseek - Not For everyone",
// paragraph 4; youlimart.com FP8 excerpt, paragraphs 2 and 3.
//
// CDNA4 mapping.  One v_mfma_f32_16x16x128_f8f6f4 consumes exactly one
// 128-deep K-group of a 16x16 output tile, so every MFMA result is a complete
// group partial P_g for its tile: it is produced with a zero accumulator and
// folded into the FP32 accumulators by one VALU FMA per element with the
// combined scale.  The promotion interval is therefore one K-group (128).
//
// The MFMA is issued "swapped": the B fragment (16 rows of N) is source A and
// the A fragment (16 rows of M) is source B, so a lane's four results lie in
// one row m and four columns n.  The 16 rows of each B fragment are drawn from
// a 64-column panel in the order n = 16*(r/4) + 4*js + r%4 (js = subtile),
// which leaves every lane with 16 consecutive columns of one output row after
// the four subtiles of a panel: 32-byte (BF16) or 64-byte (FP32) row runs.
//
// Data path per K-group: global -> registers (16-byte loads, issued one group
// ahead) -> LDS (double-buffered, 16-byte chunks XOR-swizzled by row) ->
// ds_read_b128 fragments -> MFMA -> FMA into FP32 accumulators.
#include "fp8q_launch.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

enum { kScaleBlock = 0, kScaleRow = 1 };   // B scales: 128x128 blocks, or per-row (128x1 tiles)
enum { kOutBF16 = 0, kOutF32 = 1, kOutF32Acc = 2 };

struct GemmArgs {
  const uint8_t* a; int64_t lda; const float* sa;
  const uint8_t* b; int64_t ldb; const float* sb;
  void* c; int64_t ldc;
  int64_t M, N, K;
  // grouped variant
  const int32_t* group_of_mtile; int32_t num_groups; int64_t b_group_stride; int64_t sb_group_stride;
};

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// LDS address (bytes) of 16-byte chunk `chunk` (0..7) of tile row `row`.
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}

template <int BM, int BN, int WM, int WN, int BSCALE, int OUT, bool GROUPED>
__global__ __launch_bounds__(WM * WN * 64) void gemm_blockscaled_kernel(GemmArgs p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM;          // wave tile rows (M)
  constexpr int TN = BN / WN;          // wave tile cols (N)
  constexpr int SM = TM / 16;          // M subtiles per wave
  constexpr int PN = TN / 64;          // 64-column panels per wave
  static_assert(TM % 16 == 0 && TN % 64 == 0, "wave tile shape");
  static_assert(BSCALE == kScaleRow || 128 % TN == 0, "block-scaled B needs a wave inside one 128-column block");
  constexpr int A_CHUNKS = BM * 8 / NT;  // 16-byte chunks per thread per group
  constexpr int B_CHUNKS = BN * 8 / NT;
  static_assert(A_CHUNKS * NT == BM * 8 && B_CHUNKS * NT == BN * 8, "load split");
  constexpr int STAGE = (BM + BN) * 128;

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;

  // ---- tile scheduling: XCD-aware remap, then grouped-M ordering ----------
  const int64_t tiles_m = p.M / BM;
  const int64_t tiles_n = p.N / BN;
  const int64_t ntiles = tiles_m * tiles_n;
  int64_t bid = blockIdx.x;
  if ((ntiles & 7) == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);   // consecutive tiles share an XCD
  constexpr int64_t GROUP_M = 8;
  const int64_t per_group = GROUP_M * tiles_n;
  const int64_t first_m = (bid / per_group) * GROUP_M;
  const int64_t gsize = (tiles_m - first_m) < GROUP_M ? (tiles_m - first_m) : GROUP_M;
  const int64_t mt = first_m + (bid % per_group) % gsize;
  const int64_t nt = (bid % per_group) / gsize;
  const int64_t m0 = mt * BM;
  const int64_t n0 = nt * BN;

  const uint8_t* bptr = p.b;
  const float* sbptr = p.sb;
  if constexpr (GROUPED) {
    const int32_t grp = p.group_of_mtile[mt];
    if (grp < 0 || grp >= p.num_groups) return;     // block-uniform, before any barrier
    bptr += int64_t(grp) * p.b_group_stride;
    sbptr += int64_t(grp) * p.sb_group_stride;
  }

  const int64_t KG = p.K >> 7;

  // ---- global -> register staging (thread t moves chunks t, t+NT, ...) ----
  u32x4 ra[A_CHUNKS], rb[B_CHUNKS];
#define FP8Q_LOAD_GLOBAL(g)                                                                       \
  do {                                                                                            \
    _Pragma("unroll") for (int i = 0; i < A_CHUNKS; ++i) {                                        \
      const int idx = tid + i * NT;                                                               \
      ra[i] = *reinterpret_cast<const u32x4*>(p.a + (m0 + (idx >> 3)) * p.lda + (g) * 128 +        \
                                              (idx & 7) * 16);                                    \
    }                                                                                             \
    _Pragma("unroll") for (int i = 0; i < B_CHUNKS; ++i) {                                        \
      const int idx = tid + i * NT;                                                               \
      rb[i] = *reinterpret_cast<const u32x4*>(bptr + (n0 + (idx >> 3)) * p.ldb + (g) * 128 +       \
                                              (idx & 7) * 16);                                    \
    }                                                                                             \
  } while (0)
#define FP8Q_STORE_LDS(stage)                                                                     \
  do {                                                                                            \
    uint8_t* base_ = smem + (stage) * STAGE;                                                      \
    _Pragma("unroll") for (int i = 0; i < A_CHUNKS; ++i) {                                        \
      const int idx = tid + i * NT;                                                               \
      *reinterpret_cast<u32x4*>(base_ + lds_off(idx >> 3, idx & 7)) = ra[i];                      \
    }                                                                                             \
    _Pragma("unroll") for (int i = 0; i < B_CHUNKS; ++i) {                                        \
      const int idx = tid + i * NT;                                                               \
      *reinterpret_cast<u32x4*>(base_ + BM * 128 + lds_off(idx >> 3, idx & 7)) = rb[i];           \
    }                                                                                             \
  } while (0)

  // ---- per-lane output coordinates ----------------------------------------
  const int lr = lane & 15;          // m within a subtile / source row of a fragment
  const int lq = lane >> 4;          // K quarter of a fragment; 16-column run of a panel
  const int64_t m_lane = m0 + wm * TM + lr;                 // + 16*ms
  const int64_t n_wave = n0 + wn * TN;                      // + 64*pn + 16*lq + 4*js + j

  float acc[SM][PN][4][4];
#pragma unroll
  for (int a = 0; a < SM; ++a)
#pragma unroll
    for (int b = 0; b < PN; ++b)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int d = 0; d < 4; ++d) acc[a][b][c][d] = 0.0f;

  if (KG > 0) {
    FP8Q_LOAD_GLOBAL(0);
    FP8Q_STORE_LDS(0);
  }
  __syncthreads();

  for (int64_t g = 0; g < KG; ++g) {
    const int stage = int(g & 1);
    if (g + 1 < KG) FP8Q_LOAD_GLOBAL(g + 1);

    // scales for this group
    float sa_v[SM];
#pragma unroll
    for (int ms = 0; ms < SM; ++ms) sa_v[ms] = p.sa[g * p.M + m_lane + 16 * ms];
    float sb_blk = 0.0f;
    float sb_col[PN][4][4];
    if constexpr (BSCALE == kScaleBlock) {
      sb_blk = sbptr[(n_wave >> 7) * KG + g];
#pragma unroll
      for (int ms = 0; ms < SM; ++ms) sa_v[ms] *= sb_blk;
    } else {
#pragma unroll
      for (int pn = 0; pn < PN; ++pn) {
        const v4f* src = reinterpret_cast<const v4f*>(sbptr + g * p.N + n_wave + 64 * pn + 16 * lq);
#pragma unroll
        for (int js = 0; js < 4; ++js) {
          const v4f s4 = src[js];
          sb_col[pn][js][0] = s4.x; sb_col[pn][js][1] = s4.y;
          sb_col[pn][js][2] = s4.z; sb_col[pn][js][3] = s4.w;
        }
      }
    }

    // fragments
    const uint8_t* sbase = smem + stage * STAGE;
    v8i afrag[SM];
#pragma unroll
    for (int ms = 0; ms < SM; ++ms) {
      const int row = wm * TM + 16 * ms + lr;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(sbase + lds_off(row, 2 * lq));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(sbase + lds_off(row, 2 * lq + 1));
      afrag[ms] = v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
    }
#pragma unroll
    for (int pn = 0; pn < PN; ++pn) {
#pragma unroll
      for (int js = 0; js < 4; ++js) {
        const int row = wn * TN + 64 * pn + 16 * (lr >> 2) + 4 * js + (lr & 3);
        const uint8_t* bb = sbase + BM * 128;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(bb + lds_off(row, 2 * lq));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(bb + lds_off(row, 2 * lq + 1));
        const v8i bfrag = v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
#pragma unroll
        for (int ms = 0; ms < SM; ++ms) {
          const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
          const v4f d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfrag, afrag[ms], zero,
                                                                        0, 0, 0, 0, 0, 0);
          if constexpr (BSCALE == kScaleBlock) {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[ms][pn][js][j] = __builtin_fmaf(d[j], sa_v[ms], acc[ms][pn][js][j]);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[ms][pn][js][j] = __builtin_fmaf(d[j] * sb_col[pn][js][j], sa_v[ms], acc[ms][pn][js][j]);
          }
        }
      }
    }

    if (g + 1 < KG) FP8Q_STORE_LDS(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: each lane writes 16 consecutive columns of SM*PN rows ----
#pragma unroll
  for (int ms = 0; ms < SM; ++ms) {
    const int64_t m = m_lane + 16 * ms;
#pragma unroll
    for (int pn = 0; pn < PN; ++pn) {
      const int64_t n = n_wave + 64 * pn + 16 * lq;
      if constexpr (OUT == kOutBF16) {
        uint32_t w[8];
#pragma unroll
        for (int js = 0; js < 4; ++js) {
          w[2 * js] = bf16_rne_bits(acc[ms][pn][js][0]) | (bf16_rne_bits(acc[ms][pn][js][1]) << 16);
          w[2 * js + 1] = bf16_rne_bits(acc[ms][pn][js][2]) | (bf16_rne_bits(acc[ms][pn][js][3]) << 16);
        }
        u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.c) + m * p.ldc + n);
        dst[0] = u32x4{w[0], w[1], w[2], w[3]};
        dst[1] = u32x4{w[4], w[5], w[6], w[7]};
      } else {
        v4f* dst = reinterpret_cast<v4f*>(static_cast<float*>(p.c) + m * p.ldc + n);
#pragma unroll
        for (int js = 0; js < 4; ++js) {
          v4f o = {acc[ms][pn][js][0], acc[ms][pn][js][1], acc[ms][pn][js][2], acc[ms][pn][js][3]};
          if constexpr (OUT == kOutF32Acc) o += dst[js];
          dst[js] = o;
        }
      }
    }
  }
}

#undef FP8Q_LOAD_GLOBAL
#undef FP8Q_STORE_LDS

// ---------------------------------------------------------------------------
// Launch configurations.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int BSCALE, int OUT, bool GROUPED>
static hipError_t launch_cfg(const GemmArgs& a, hipStream_t st) {
  const int64_t tiles = (a.M / BM) * (a.N / BN);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_blockscaled_kernel<BM, BN, WM, WN, BSCALE, OUT, GROUPED>),
                     dim3(unsigned(tiles)), dim3(WM * WN * 64), 0, st, a);
  return hipGetLastError();
}

template <int BSCALE, bool GROUPED>
static hipError_t launch_out(const GemmArgs& a, int out, hipStream_t st) {
  // 128x128 workgroup tile, 2x2 waves of 64x64.
  switch (out) {
    case kOutBF16: return launch_cfg<128, 128, 2, 2, BSCALE, kOutBF16, GROUPED>(a, st);
    case kOutF32: return launch_cfg<128, 128, 2, 2, BSCALE, kOutF32, GROUPED>(a, st);
    default: return launch_cfg<128, 128, 2, 2, BSCALE, kOutF32Acc, GROUPED>(a, st);
  }
}

static int out_code(bool out_bf16, bool accumulate) {
  return out_bf16 ? kOutBF16 : (accumulate ? kOutF32Acc : kOutF32);
}

hipError_t launch_gemm(int kind, int64_t M, int64_t N, int64_t K,
                       const uint8_t* a, int64_t lda, const float* sa,
                       const uint8_t* b, int64_t ldb, const float* sb,
                       void* c, bool out_bf16, int64_t ldc, bool accumulate, hipStream_t st) {
  GemmArgs args{a, lda, sa, b, ldb, sb, c, ldc, M, N, K, nullptr, 0, 0, 0};
  const int out = out_code(out_bf16, accumulate);
  if (kind == 2) return launch_out<kScaleRow, false>(args, out, st);
  return launch_out<kScaleBlock, false>(args, out, st);
}

hipError_t launch_gemm_grouped(int32_t num_groups, int64_t M_total, int64_t N, int64_t K,
                               const int32_t* group_of_mtile,
                               const uint8_t* a, int64_t lda, const float* sa,
                               const uint8_t* b, const float* sb,
                               void* c, bool out_bf16, int64_t ldc, hipStream_t st) {
  GemmArgs args{a, lda, sa, b, K, sb, c, ldc, M_total, N, K,
                group_of_mtile, num_groups, N * K, (N / 128) * (K / 128)};
  return launch_out<kScaleBlock, true>(args, out_code(out_bf16, false), st);
}

}  // namespace fp8q
