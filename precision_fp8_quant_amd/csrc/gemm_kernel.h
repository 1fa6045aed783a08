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
// Data path per K-group: global -> LDS by LDS DMA (buffer_load_dwordx4 ...
// lds, issued one group ahead into the other of two stages; 16-byte chunks
// XOR-swizzled by row) -> ds_read_b128 fragments -> MFMA -> FMA into FP32
// accumulators.
//
// The template parameter HW says which operands' scales are powers of two
// and applied by the matrix core itself (v_mfma_scale_f32_16x16x128_f8f6f4
// takes them as E8M0 exponents): kHwNone, kHwA, kHwB, or kHwAB.  With both,
// every group accumulates in place in the MFMA and the loop carries no VALU
// work (instantiated in gemm_pow2.hip); with one, the other operand's scale
// is the only factor left for the promotion FMA, which for Wgrad saves the
// per-element multiply.
#pragma once

#include "fp8q_launch.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

enum { kScaleBlock = 0, kScaleRow = 1 };   // B scales: 128x128 blocks, or per-row (128x1 tiles)
enum { kOutBF16 = 0, kOutF32 = 1, kOutF32Acc = 2 };
enum { kHwNone = 0, kHwA = 1, kHwB = 2, kHwAB = 3 };   // power-of-two scales applied in the MFMA

struct GemmArgs {
  const uint8_t* a; int64_t lda; const float* sa;
  const uint8_t* b; int64_t ldb; const float* sb;
  void* c; int64_t ldc;
  int64_t M, N, K;
  // grouped variant
  const int32_t* group_of_mtile; int32_t num_groups; int64_t b_group_stride; int64_t sb_group_stride;
  // leading dimension of the A scales [K/128][sa_ld] (the full M; a grid
  // that covers a band of rows gets sa offset to its first row)
  int64_t sa_ld;
  // K-split grids (KSPLIT > 1, FP32 output): elements between the output
  // matrices of consecutive K ranges
  int64_t split_c_off;
};

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// LDS tile rows are 128 bytes (one K-group) in eight 16-byte chunks; chunk c
// of row r is stored at position c ^ (r & 7).  The K order inside one MFMA
// is free as long as both operands use the same one, so lane quarter q
// (lanes 16q..16q+15) feeds its fragment from chunks q and q+4.  The LDS
// serves a ds_read_b128 in four passes of 16 lanes -- lanes whose 4-lane
// group index has even / odd bit parity, per half-wave -- over 64 four-byte
// banks (256 bytes); with this chunk assignment and swizzle every pass of both
// fragment reads touches 16 distinct 16-byte bank groups (no conflicts),
// while the DMA still moves whole 128-byte rows.
__device__ __forceinline__ int swz(int row) { return row & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * 128 + ((chunk ^ swz(row)) << 4); }

// B tiles are stored in LDS in fragment order: LDS row rho = 64*p + 16*js + r
// holds global row 64*p + 16*(r/4) + 4*js + r%4, so the 16 rows a fragment
// needs are consecutive in LDS while a lane still ends up owning 16
// consecutive output columns (the B DMA below writes this order).

typedef const __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// 16 bytes per lane from global memory straight into LDS at dst + 16*lane
// (dst is wave-uniform).  Completion is tracked by vmcnt.
__device__ __forceinline__ void dma16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)dst, 16, 0, 0);
}
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int row, int lq) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(tile + lds_off(row, lq));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(tile + lds_off(row, lq + 4));
  return v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
}

// KSPLIT > 1: every tile is computed KSPLIT times, each over its share of the
// K-groups, into its own FP32 output (p.c + part * p.split_c_off); a second
// kernel adds the parts.
template <int BM, int BN, int WM, int WN, int BSCALE, int OUT, bool GROUPED, int HW, int KSPLIT = 1>
__global__ __launch_bounds__(WM * WN * 64) void gemm_blockscaled_kernel(GemmArgs p) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM;          // wave tile rows (M)
  constexpr int TN = BN / WN;          // wave tile cols (N)
  constexpr int SM = TM / 16;          // M subtiles per wave
  constexpr int PN = TN / 64;          // 64-column panels per wave
  static_assert(TM % 16 == 0 && TN % 64 == 0, "wave tile shape");
  static_assert(BSCALE == kScaleRow || 128 % TN == 0, "block-scaled B needs a wave inside one 128-column block");
  constexpr int A_BYTES = BM * 128;
  constexpr int B_BYTES = BN * 128;
  constexpr int SB_BYTES = BSCALE == kScaleRow ? BN * 4 : 0;   // one group's per-column B scales
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int SB_SLOTS = 2;           // per-column B scales of groups g and g+1, beside the stages
  constexpr int A_DMA = A_BYTES / 1024 / NW;     // 1 KB wave-wide DMA instructions per wave per stage
  constexpr int B_DMA = B_BYTES / 1024 / NW;
  static_assert(A_DMA * 1024 * NW == A_BYTES && B_DMA * 1024 * NW == B_BYTES, "DMA split");
  static_assert(BSCALE != kScaleRow || BN <= 256, "row scales: one DMA of at most 64 lanes x 4 floats");

  // K-group stages (and Wgrad's per-column B scales), reused by the epilogue
  // to stage the output tile (TM rows of 64 columns per wave, padded rows)
  constexpr int LOOP_LDS = 2 * STAGE + SB_SLOTS * SB_BYTES;
  constexpr int EPI_LDS = NW * TM * (64 * (OUT == kOutBF16 ? 2 : 4) + 16);
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LOOP_LDS > EPI_LDS ? LOOP_LDS : EPI_LDS];
  uint8_t* const sb_ring = smem + 2 * STAGE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;

  // ---- tile scheduling: XCD-aware remap, then grouped-M ordering ----------
  static_assert(KSPLIT == 1 || (OUT == kOutF32 && !GROUPED), "K-split grids write FP32 parts");
  const int64_t tiles_m = p.M / BM;
  const int64_t tiles_n = p.N / BN;
  const int64_t ntiles = tiles_m * tiles_n * KSPLIT;    // with K split: (tile, part) pairs, parts adjacent
  // Workgroup i runs on XCD i % 8.  Plain GEMMs: give every XCD one
  // contiguous range of tiles (ceil or floor of ntiles/8), so neighbouring
  // tiles share its L2.  Grouped GEMMs: deal the 32-tile runs of the
  // grouped-M order (8 M-tiles x 4 N-tiles when N = 2048) to the XCDs in turn.
  // A contiguous eighth of a grouped problem is one kind of group: with groups
  // of very different sizes, one XCD got all the small groups, whose weight
  // panels are read by one or two M-tiles each, and streamed them through its
  // own link to memory while the XCDs of the largest group reused theirs from
  // L2 (measured on 64 Zipf(1.1)-sized experts: 1120 -> 1076 us).  The runs
  // keep each XCD's concurrent tiles on shared A and B panels.
  int64_t bid = blockIdx.x;
  if constexpr (GROUPED) {
    const int64_t full = (ntiles >> 8) << 8;    // whole rounds of 8 runs; the rest keep their order
    if (bid < full) {
      const int64_t x = bid & 7, l = bid >> 3;
      bid = (((l >> 5) << 3) + x) * 32 + (l & 31);
    }
  } else {
    const int64_t q = ntiles >> 3, r = ntiles & 7, x = bid & 7, l = bid >> 3;
    bid = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + l;
  }
  const int part = KSPLIT > 1 ? int(bid % KSPLIT) : 0;
  if constexpr (KSPLIT > 1) bid /= KSPLIT;
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
  const int64_t KG = p.K >> 7;                 // K-groups of the whole problem (scale indexing)
  const int64_t kg0 = KSPLIT > 1 ? (KG * part) / KSPLIT : 0;          // this block's range of them
  const int64_t kg1 = KSPLIT > 1 ? (KG * (part + 1)) / KSPLIT : KG;

  // ---- DMA addressing ------------------------------------------------------
  // Wave-wide DMA instruction `blk` fills LDS rows 8*blk .. 8*blk+7; lane l
  // lands at row 8*blk + l/8, physical chunk l%8, i.e. logical chunk
  // (l%8) ^ swz(row) = (l%8) ^ (l/8).  The per-lane byte offset is the same
  // for every blk and everything else is wave-uniform (SGPRs).  For B the LDS
  // row rho maps to global row 64*(blk/8) + 32*(blk&1) + 4*((blk/2)&3)
  // [uniform] + 16*(l/32) + (l/8)%4 [per lane].
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int lchunk = ((lane & 7) ^ (lane >> 3)) << 4;
  const uint32_t a_off = uint32_t((lane >> 3) * p.lda + lchunk);
  const uint32_t b_off = uint32_t((16 * (lane >> 5) + ((lane >> 3) & 3)) * p.ldb + lchunk);
  const uint8_t* a_base = p.a + m0 * p.lda;
  const uint8_t* b_base = bptr + n0 * p.ldb;

  // The DMA goes through buffer resources based at the tile's first A and B
  // rows (records = the tile's bytes, so nothing outside the tile is read):
  // the per-lane byte offset is a constant VGPR and the wave-uniform row and
  // K-group offset an SGPR, so the loop spends no VALU instruction on
  // addresses (with 64-bit global addresses it spent 12-18 per group; Fprop
  // 2% faster).  The 32-bit offsets need a tile's rows of A and B (up to 512)
  // to span less than 2^31 bytes, which the C ABI checks (leading dimensions
  // below 4 MiB).
  // 0x00020000: the buffer descriptor's fourth word for untyped 32-bit
  // accesses on gfx9-family devices.
  const __amdgpu_buffer_rsrc_t rsrc_a =
      __builtin_amdgcn_make_buffer_rsrc((void*)a_base, (short)0, int((BM - 1) * p.lda + p.K), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsrc_b =
      __builtin_amdgcn_make_buffer_rsrc((void*)b_base, (short)0, int((BN - 1) * p.ldb + p.K), 0x00020000);
  // DMA instruction i (0 .. A_DMA+B_DMA-1) of this wave's share of group g.
  auto issue_dma = [&](int64_t g, int stage, int i) {
    uint8_t* base = smem + stage * STAGE;
    if (i < A_DMA) {
      const int blk = wave_u * A_DMA + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_a, (lptr_t)(base + blk * 1024), 16, int(a_off),
                                               int(8 * blk * p.lda + g * 128), 0, 0);
    } else {
      const int blk = wave_u * B_DMA + (i - A_DMA);
      const int row_u = 64 * (blk >> 3) + 32 * (blk & 1) + 4 * ((blk >> 1) & 3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_b, (lptr_t)(base + A_BYTES + blk * 1024), 16, int(b_off),
                                               int(row_u * p.ldb + g * 128), 0, 0);
    }
  };
  auto issue_stage = [&](int64_t g, int stage) {
#pragma unroll
    for (int i = 0; i < A_DMA + B_DMA; ++i) issue_dma(g, stage, i);
  };
  // Per-column B scales of group g into slot `slot` (issued at the top of an
  // iteration, where a wave-uniform branch splits no MFMA/FMA block).
  auto issue_scales = [&](int64_t g, int slot) {
    if constexpr (BSCALE == kScaleRow) {
      if (wave_u == NW - 1 && lane < BN / 4)
        dma16(sbptr + g * p.N + n0 + lane * 4, sb_ring + slot * SB_BYTES);
    }
  };

  // ---- per-lane output coordinates ----------------------------------------
  const int lr = lane & 15;
  const int lq = lane >> 4;
  const int64_t m_lane = m0 + wm * TM + lr;                 // + 16*ms
  const int64_t n_wave = n0 + wn * TN;                      // + 64*pn + 16*lq + 4*js + j

  // Promoted path: FP32 accumulators updated by VALU FMAs once per group.
  // Both scales in hardware (kHwAB): the MFMA applies both power-of-two
  // scales itself and accumulates every group into accv (no VALU work).
  constexpr bool IN_MFMA = HW == kHwAB;           // accumulate inside the MFMA
  constexpr bool A_HW = (HW & kHwA) != 0;         // A-row scale applied by the MFMA
  constexpr bool B_HW = (HW & kHwB) != 0;         // B-row / block scale applied by the MFMA
  float acc[SM][PN][4][4];
  v4f accv[SM][PN][4];
#pragma unroll
  for (int a = 0; a < SM; ++a)
#pragma unroll
    for (int b = 0; b < PN; ++b)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if constexpr (IN_MFMA) accv[a][b][c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int d = 0; d < 4; ++d) acc[a][b][c][d] = 0.0f;
      }

  // Per K-group: the group's MFMAs run from LDS fragments while the DMA of
  // group g+1 into the other stage is issued between its first MFMAs, then
  // one barrier.  Inside the group a software pipeline over its NT = NB*SM
  // MFMAs (step t: B fragment bi = t/SM against A fragment ms = t%SM):
  //  * promoted path: MFMA t writes result slot t%3 and the promotion FMAs of
  //    MFMA t-2 follow it, so a VALU op never waits on the MFMA just issued;
  //  * kHwAB: the MFMA takes both E8M0 scales and accumulates in place;
  //    nothing else runs (kHwA / kHwB: the MFMA takes one scale, the FMA the
  //    other);
  //  * fragment reads run ahead of their MFMAs: the group's A fragments and B
  //    fragments 0-1 up front, then B fragment bi+2 (with the per-column
  //    Wgrad scales it needs) right after the first MFMA of block bi, never
  //    just before a fragment's first use: where the compiler cannot count
  //    the LDS reads exactly (Wgrad, whose per-column scales come by a 64-bit
  //    global DMA), it waits for all of them (lgkmcnt(0)) before a use.
  // A scheduling barrier after every step pins this interleave (left alone,
  // the compiler places each FMA right behind its own MFMA and pads the
  // hazard with s_nop).
  constexpr int NB = PN * 4;            // B fragments per group
  constexpr int NT = NB * SM;           // MFMAs per group
  constexpr int LAG = IN_MFMA ? 0 : 2;
  static_assert(HW == kHwNone || !GROUPED, "the hardware-scaled paths cover the plain GEMMs");
  static_assert(A_DMA + B_DMA <= NT, "the next group's DMA rides on this group's first MFMA steps");

  auto frag_row_b = [&](int bi) { return wn * TN + 16 * bi + lr; };
  auto sbq_off = [&](int bi) { return (wn * TN + 64 * (bi >> 2) + 16 * lq + 4 * (bi & 3)) * 4; };
  // B_HW: the source-A row this lane feeds in B fragment bi is the LDS row
  // frag_row_b(bi), i.e. tile column wn*TN + 64*(bi/4) + 16*(lr/4) + 4*(bi%4) + lr%4.
  // A power-of-two float's E8M0 code is its biased exponent field.
  auto sbe_read = [&](const uint8_t* ring, int bi) {
    const int col = wn * TN + 64 * (bi >> 2) + 16 * (lr >> 2) + 4 * (bi & 3) + (lr & 3);
    return reinterpret_cast<const uint32_t*>(ring)[col] >> 23;
  };

  float sa_cur[SM], sa_nxt[SM];
  float sb_cur = 0.0f, sb_nxt = 0.0f;
  if (kg1 > kg0) {
    issue_stage(kg0, 0);
    issue_scales(kg0, 0);
#pragma unroll
    for (int ms = 0; ms < SM; ++ms) sa_cur[ms] = p.sa[kg0 * p.sa_ld + m_lane + 16 * ms];
    if constexpr (BSCALE == kScaleBlock) sb_cur = sbptr[(n_wave >> 7) * KG + kg0];
    wait_vmem_all();
  }
  __syncthreads();

  // One basic block per iteration (no branches between the MFMAs and their
  // promotion FMAs): the last iteration simply re-fetches its own group into
  // the idle stage, which nobody reads.
  for (int64_t g = kg0; g < kg1; ++g) {
    const int stage = int((g - kg0) & 1);
    const int64_t gn = g + 1 < kg1 ? g + 1 : g;
    issue_scales(gn, stage ^ 1);
#pragma unroll
    for (int ms = 0; ms < SM; ++ms) sa_nxt[ms] = p.sa[gn * p.sa_ld + m_lane + 16 * ms];
    if constexpr (BSCALE == kScaleBlock) sb_nxt = sbptr[(n_wave >> 7) * KG + gn];

    const uint8_t* ta = smem + stage * STAGE;
    const uint8_t* tb = ta + A_BYTES;
    const uint8_t* ts = sb_ring + stage * SB_BYTES;
    // cs: the promotion factor of A fragment ms (everything the MFMA does not
    // apply, except Wgrad's per-column B scale, which sbq carries)
    float cs[SM];
    uint32_t sae[SM];                                   // A_HW: E8M0 codes of the A-row scales
#pragma unroll
    for (int ms = 0; ms < SM; ++ms) {
      const float fa = A_HW ? 1.0f : sa_cur[ms];
      cs[ms] = (BSCALE == kScaleBlock && !B_HW) ? fa * sb_cur : fa;
      sae[ms] = A_HW ? __float_as_uint(sa_cur[ms]) >> 23 : 127u;   // 127: E8M0 code of 1.0
    }
    const uint32_t sbe_blk = __float_as_uint(sb_cur) >> 23;

    v8i af[SM];
    v8i bfb[3];
    v4f sbq[3];                             // Wgrad, B promoted: slot b%3 holds block b's column scales
    uint32_t sbe[3];                        // Wgrad, B in the MFMA: slot b%3 holds this lane's B-row code
#pragma unroll
    for (int ms = 0; ms < SM; ++ms) af[ms] = read_frag(ta, wm * TM + 16 * ms + lr, lq);
    bfb[0] = read_frag(tb, frag_row_b(0), lq);
    if (NB > 1) bfb[1] = read_frag(tb, frag_row_b(1), lq);
    if constexpr (BSCALE == kScaleRow) {
      if constexpr (B_HW) {
        sbe[0] = sbe_read(ts, 0);
        if (NB > 1) sbe[1] = sbe_read(ts, 1);
      } else {
        sbq[0] = *reinterpret_cast<const v4f*>(ts + sbq_off(0));
      }
    }
    v4f dq[3];
#pragma unroll
    for (int t = 0; t < NT + LAG; ++t) {
      if (t < NT) {
        const int bi = t / SM, ms = t % SM;
        if constexpr (IN_MFMA) {
          // v_mfma_scale_f32_16x16x128_f8f6f4: E8M0 scale of source A (this
          // lane's B row) and of source B (this lane's A row) applied in the
          // matrix core, result accumulated in place
          const uint32_t sb_e = BSCALE == kScaleRow ? sbe[bi % 3] : sbe_blk;
          accv[ms][bi >> 2][bi & 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              bfb[bi % 3], af[ms], accv[ms][bi >> 2][bi & 3], 0, 0, 0, sb_e, 0, sae[ms]);
        } else if constexpr (HW != kHwNone) {
          // one operand's scale in the matrix core (the other's is 2^0), the
          // partial then promoted like below
          const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
          const uint32_t sb_e = !B_HW ? 127u : (BSCALE == kScaleRow ? sbe[bi % 3] : sbe_blk);
          dq[t % 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfb[bi % 3], af[ms], zero, 0, 0, 0, sb_e, 0,
                                                                      sae[ms]);
        } else {
          const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
          dq[t % 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfb[bi % 3], af[ms], zero, 0, 0, 0, 0, 0, 0);
        }
        if (ms == 0) {
          if (bi + 2 < NB) {
            bfb[(bi + 2) % 3] = read_frag(tb, frag_row_b(bi + 2), lq);
            if constexpr (B_HW && BSCALE == kScaleRow) sbe[(bi + 2) % 3] = sbe_read(ts, bi + 2);
          }
          if constexpr (!B_HW && BSCALE == kScaleRow)
            if (bi + 1 < NB) sbq[(bi + 1) % 3] = *reinterpret_cast<const v4f*>(ts + sbq_off(bi + 1));
        }
        // the next group's DMA, one instruction after each of the group's
        // first MFMAs: issued all at the top of the group it held back the
        // first MFMAs (measured 3-6% slower; one every 2 MFMAs sat in between,
        // spread over the whole group it was 5% slower still, the last
        // instructions then landing late for the end-of-group wait)
        if (t < A_DMA + B_DMA) issue_dma(gn, stage ^ 1, t);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (!IN_MFMA && t >= LAG) {
        const int u = t - LAG;
        const int bu = u / SM, mu = u % SM;
        const int pn = bu >> 2, js = bu & 3;
        const v4f d = dq[u % 3];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (BSCALE == kScaleRow && !B_HW && A_HW) {
            acc[mu][pn][js][j] = __builtin_fmaf(d[j], sbq[bu % 3][j], acc[mu][pn][js][j]);
          } else {
            // the combined scale sa*sb first, then one fused multiply-add of
            // the partial: no intermediate depends on the partial's size
            const float cj = (BSCALE == kScaleRow && !B_HW) ? cs[mu] * sbq[bu % 3][j] : cs[mu];
            acc[mu][pn][js][j] = __builtin_fmaf(d[j], cj, acc[mu][pn][js][j]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // keep step t's MFMA and step t-2's FMAs together
    }
#pragma unroll
    for (int ms = 0; ms < SM; ++ms) sa_cur[ms] = sa_nxt[ms];
    sb_cur = sb_nxt;
    wait_vmem_all();
    __syncthreads();
  }
  if constexpr (IN_MFMA) {
#pragma unroll
    for (int a = 0; a < SM; ++a)
#pragma unroll
      for (int b = 0; b < PN; ++b)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int d = 0; d < 4; ++d) acc[a][b][c][d] = accv[a][b][c][d];
  }

  // ---- epilogue ----------------------------------------------------------
  // A lane holds 16 consecutive columns of one row per (ms, pn).  Stored as
  // they are, one store instruction wrote 16-byte pieces of 32 (BF16) or 64
  // (FP32) different 128-byte lines, and writing the output was the costliest
  // part of a tile (measured on the bench shapes: full-line stores made Fprop
  // 6% and, non-temporal, the FP32 Wgrad 9% faster).  So the tile leaves
  // through LDS, which the last K-group's barrier has freed: each wave writes
  // one 64-column panel at a time into its own region (rows padded by 16
  // bytes, which keeps both the writes and the read-back free of bank
  // conflicts) and reads it back so that 8 lanes hold one whole line; every
  // store instruction then writes whole lines of 8 (BF16) or 4 (FP32) rows.
  // A wave's LDS instructions run in order, so it reuses its region for the
  // next panel without a wait.  Non-temporal stores: the output goes to HBM
  // while the GEMM, which is MFMA-bound, still runs, instead of lingering
  // dirty in the memory-side cache for the next kernel to write back
  // (measured: the 1x128 + 128x1 quantizer of an 8192x18432 gradient after
  // Fprop, 126 -> 113 us).
  constexpr int ESZ = OUT == kOutBF16 ? 2 : 4;
  constexpr int PITCH = 64 * ESZ + 16;                  // bytes per staged row
  constexpr int LPR = 64 * ESZ / 16;                     // lanes per 64-column row: 8 or 16
  constexpr int RPI = 64 / LPR;                          // rows per store instruction: 8 or 4
  static_assert(NW * TM * PITCH <= int(sizeof(smem)), "epilogue staging fits the LDS");
  uint8_t* const stg = smem + wave * (TM * PITCH);
#pragma unroll
  for (int pn = 0; pn < PN; ++pn) {
#pragma unroll
    for (int ms = 0; ms < SM; ++ms) {
      uint8_t* row = stg + (16 * ms + lr) * PITCH;
      if constexpr (OUT == kOutBF16) {
        uint32_t w[8];
#pragma unroll
        for (int js = 0; js < 4; ++js) {
          w[2 * js] = bf16_rne_bits(acc[ms][pn][js][0]) | (bf16_rne_bits(acc[ms][pn][js][1]) << 16);
          w[2 * js + 1] = bf16_rne_bits(acc[ms][pn][js][2]) | (bf16_rne_bits(acc[ms][pn][js][3]) << 16);
        }
        *reinterpret_cast<u32x4*>(row + 32 * lq) = u32x4{w[0], w[1], w[2], w[3]};
        *reinterpret_cast<u32x4*>(row + 32 * lq + 16) = u32x4{w[4], w[5], w[6], w[7]};
      } else {
#pragma unroll
        for (int js = 0; js < 4; ++js)
          *reinterpret_cast<v4f*>(row + 64 * lq + 16 * js) =
              v4f{acc[ms][pn][js][0], acc[ms][pn][js][1], acc[ms][pn][js][2], acc[ms][pn][js][3]};
      }
    }
    const int chunk = lane % LPR;
#pragma unroll
    for (int sr = 0; sr < TM / RPI; ++sr) {
      const int r = sr * RPI + lane / LPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * PITCH + 16 * chunk);
      const int64_t m = m0 + wm * TM + r;
      const int64_t n = n_wave + 64 * pn + chunk * (16 / ESZ);
      if constexpr (OUT == kOutBF16) {
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.c) + m * p.ldc + n));
      } else {
        float* const c = static_cast<float*>(p.c) + (KSPLIT > 1 ? part * p.split_c_off : 0);
        v4f* dst = reinterpret_cast<v4f*>(c + m * p.ldc + n);
        v4f o = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
        if constexpr (OUT == kOutF32Acc) o += *dst;
        __builtin_nontemporal_store(o, dst);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launch configurations.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int BSCALE, int OUT, bool GROUPED, int HW, int KSPLIT = 1>
static hipError_t launch_cfg(const GemmArgs& a, hipStream_t st) {
  const int64_t tiles = (a.M / BM) * (a.N / BN) * KSPLIT;
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_blockscaled_kernel<BM, BN, WM, WN, BSCALE, OUT, GROUPED, HW, KSPLIT>),
                     dim3(unsigned(tiles)), dim3(WM * WN * 64), 0, st, a);
  return hipGetLastError();
}

namespace {
// The BF16 columns of a GEMM whose K was split in two:
//   c[m][n] = RNE(p[m][n] + p[m][half + n]),  n < cols,
// p holding the two FP32 parts side by side in rows of ldp floats.  Eight
// columns per thread (cols % 8 == 0), 16-byte loads and stores; rows
// blockIdx.y, blockIdx.y + gridDim.y, ...
__global__ __launch_bounds__(128) void ksplit_sum_bf16_kernel(const float* __restrict__ p, int64_t ldp, int64_t half,
                                                              uint16_t* __restrict__ c, int64_t ldc, int64_t rows,
                                                              int64_t cols) {
  const int64_t n = (int64_t(blockIdx.x) * 128 + threadIdx.x) * 8;
  if (n >= cols) return;
  for (int64_t m = blockIdx.y; m < rows; m += gridDim.y) {
    const v4f* a = reinterpret_cast<const v4f*>(p + m * ldp + n);
    const v4f* b = reinterpret_cast<const v4f*>(p + m * ldp + half + n);
    const v4f lo = a[0] + b[0], hi = a[1] + b[1];
    u32x4 w;
    w.x = bf16_rne_bits(lo[0]) | (bf16_rne_bits(lo[1]) << 16);
    w.y = bf16_rne_bits(lo[2]) | (bf16_rne_bits(lo[3]) << 16);
    w.z = bf16_rne_bits(hi[0]) | (bf16_rne_bits(hi[1]) << 16);
    w.w = bf16_rne_bits(hi[2]) | (bf16_rne_bits(hi[3]) << 16);
    *reinterpret_cast<u32x4*>(c + m * ldc + n) = w;
  }
}
}  // namespace

// Tile configurations, largest that divides the problem:
//   256x256, 8 waves (4 along M x 2 along N) of 64x128
//   grouped GEMMs (one group per 128-row tile): 128x512, 8 waves (2x4) of
//   64x128 -- the same wave tile as 256x256, with both stages filling the
//   160 KB of LDS (measured 25% faster than 128x256 on the MoE layer); else
//   128x256, 8 waves (2x4) of 64x64
//   128x256, 4 waves (2x2) of 64x128
//   256x128, 4 waves (4x1) of 64x128
//   128x128, 4 waves (2x2) of 64x64
template <int BSCALE, int OUT, bool GROUPED, int HW>
static hipError_t launch_tiles(const GemmArgs& a, hipStream_t st) {
  if (!GROUPED && a.M % 256 == 0 && a.N % 256 == 0) return launch_cfg<256, 256, 4, 2, BSCALE, OUT, GROUPED, HW>(a, st);
  if constexpr (GROUPED) {
    if (a.N % 512 == 0) return launch_cfg<128, 512, 2, 4, BSCALE, OUT, GROUPED, HW>(a, st);
    if (a.N % 256 == 0) return launch_cfg<128, 256, 2, 4, BSCALE, OUT, GROUPED, HW>(a, st);
  }
  if (a.N % 256 == 0) return launch_cfg<128, 256, 2, 2, BSCALE, OUT, GROUPED, HW>(a, st);
  if (!GROUPED && a.M % 256 == 0) return launch_cfg<256, 128, 4, 1, BSCALE, OUT, GROUPED, HW>(a, st);
  return launch_cfg<128, 128, 2, 2, BSCALE, OUT, GROUPED, HW>(a, st);
}

// Balance the last wave of tiles (256 CUs): a 256x256 grid whose last wave
// is at most half full leaves half the chip idle for a whole tile time.  When
// those tail tiles form whole 256-column bands (block-scaled B only), the bands
// run either as whole tiles with K split in two (BF16 output, below) or as a
// second grid of 128x256 tiles -- two per 256x256 tile, one full wave --
// right behind the first (an 8192x7168 output: 768 + 256 tiles instead of
// 896 in 3.5 waves).
template <int BSCALE, int OUT, bool GROUPED, int HW>
static hipError_t launch_balanced(const GemmArgs& a, hipStream_t st) {
  constexpr int64_t kCUs = 256;
  // Grouped GEMM: the same for a last wave of 128x512 tiles, split off along
  // M instead (whole 128-row tiles, each in one group), e.g. the 64-expert MoE
  // layer with 543 M-tiles: 2048 + 248 tiles (8 waves + one of 128x256)
  // instead of 2172 in 8.5 waves.
  if constexpr (GROUPED) {
    if (a.N % 512 == 0) {
      const int64_t tn = a.N / 512, tiles = (a.M / 128) * tn;
      const int64_t tail = tiles % kCUs;
      if (tiles > kCUs && tail != 0 && 2 * tail <= kCUs && tail % tn == 0) {
        GemmArgs head = a, rest = a;
        rest.M = (tail / tn) * 128;
        head.M = a.M - rest.M;
        rest.a = a.a + head.M * a.lda;
        rest.sa = a.sa + head.M;
        rest.group_of_mtile = a.group_of_mtile + head.M / 128;
        rest.c = static_cast<uint8_t*>(a.c) + head.M * a.ldc * (OUT == kOutBF16 ? 2 : 4);
        const hipError_t e = launch_cfg<128, 512, 2, 4, BSCALE, OUT, true, HW>(head, st);
        if (e != hipSuccess) return e;
        return launch_cfg<128, 256, 2, 4, BSCALE, OUT, true, HW>(rest, st);
      }
    }
  }
  if constexpr (BSCALE == kScaleBlock && !GROUPED) {
    if (a.M % 256 == 0 && a.N % 256 == 0) {
      const int64_t tm = a.M / 256, tiles = tm * (a.N / 256);
      const int64_t tail = tiles % kCUs;
      if (tiles > kCUs && tail != 0 && 2 * tail <= kCUs && tail % tm == 0) {
        GemmArgs head = a, rest = a;
        rest.N = (tail / tm) * 256;
        head.N = a.N - rest.N;
        rest.b = a.b + head.N * a.ldb;
        rest.sb = a.sb + (head.N / 128) * (a.K / 128);
        rest.c = static_cast<uint8_t*>(a.c) + head.N * (OUT == kOutBF16 ? 2 : 4);
        // BF16 output with room for two FP32 copies of the tail in the head
        // columns of C (which the head grid writes afterwards): the tail runs
        // as whole 256x256 tiles, each as two K halves in one wave of
        // 2 x tail workgroups, into that scratch, and a third kernel adds the
        // halves into the tail columns (Dgrad 8192x7168x18432: 905 -> 860 us).
        // Otherwise the tail bands run as 128x256 tiles over the whole K,
        // which read more LDS bytes per MFMA.
        if constexpr (OUT == kOutBF16) {
          if (a.K >= 256 && head.N >= 4 * rest.N) {
            GemmArgs part = rest;
            part.c = a.c;                        // FP32 rows of ldc / 2 floats over C's head columns
            part.ldc = a.ldc / 2;
            part.split_c_off = rest.N;
            hipError_t e = launch_cfg<256, 256, 4, 2, BSCALE, kOutF32, false, HW, 2>(part, st);
            if (e != hipSuccess) return e;
            const dim3 sum_grid(unsigned((rest.N / 8 + 127) / 128), unsigned(a.M < 65535 ? a.M : 65535));
            hipLaunchKernelGGL(ksplit_sum_bf16_kernel, sum_grid, dim3(128), 0, st, static_cast<const float*>(a.c),
                               a.ldc / 2, rest.N, static_cast<uint16_t*>(rest.c), a.ldc, a.M, rest.N);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
            return launch_cfg<256, 256, 4, 2, BSCALE, OUT, false, HW>(head, st);
          }
        }
        const hipError_t e = launch_cfg<256, 256, 4, 2, BSCALE, OUT, false, HW>(head, st);
        if (e != hipSuccess) return e;
        return launch_cfg<128, 256, 2, 4, BSCALE, OUT, false, HW>(rest, st);
      }
    }
  }
  return launch_tiles<BSCALE, OUT, GROUPED, HW>(a, st);
}

template <int BSCALE, bool GROUPED, int HW>
static hipError_t launch_out(const GemmArgs& a, int out, hipStream_t st) {
  switch (out) {
    case kOutBF16: return launch_balanced<BSCALE, kOutBF16, GROUPED, HW>(a, st);
    case kOutF32: return launch_balanced<BSCALE, kOutF32, GROUPED, HW>(a, st);
    default: return launch_balanced<BSCALE, kOutF32Acc, GROUPED, HW>(a, st);
  }
}

static int out_code(bool out_bf16, bool accumulate) {
  return out_bf16 ? kOutBF16 : (accumulate ? kOutF32Acc : kOutF32);
}

}  // namespace fp8q
