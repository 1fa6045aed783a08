// C ABI of fp8q: argument validation, then dispatch to the HIP launchers.
// Every check runs on the host before anything is enqueued; the first
// violation returns its status and nothing is launched.
#include "../../include/fp8q.h"
#include "fp8q_launch.h"

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace {

constexpr int64_t kMaxGridX = 0x7FFFFFFF;
// GEMM operands are read through buffer resources with 32-bit offsets within
// a tile of up to 512 rows: leading dimensions of A and B must stay below
// 2^31 / 512 bytes (4 MiB), with K <= ld.
constexpr int64_t kMaxGemmLd = (int64_t(1) << 31) / 512 - 128;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;   // [lo, hi)
  bool ok;            // false: the extent overflows 64 bits or the address space
};

// Bytes spanned by a row-major matrix with `rows` rows of `cols` elements,
// ((rows - 1) * ld + cols) * esize, with every step checked for overflow
// (the sizes are non-negative here: negative ones were rejected before).
Range span(const void* p, int64_t rows, int64_t cols, int64_t ld, int64_t esize) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  if (rows <= 0 || cols <= 0) return {lo, lo, true};
  int64_t elems = 0, bytes = 0;
  uintptr_t hi = 0;
  if (__builtin_mul_overflow(rows - 1, ld, &elems) || __builtin_add_overflow(elems, cols, &elems) ||
      __builtin_mul_overflow(elems, esize, &bytes) || __builtin_add_overflow(lo, uintptr_t(bytes), &hi))
    return {lo, lo, false};
  return {lo, hi, true};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

// a * b for non-negative a, b; false on overflow
bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

// A leading dimension of `ld` elements of `esize` (2 or 4) bytes is a multiple
// of 16 bytes (without forming ld * esize, which could overflow).
bool ld16(int64_t ld, int64_t esize) { return ld % (16 / esize) == 0; }

int64_t dtype_size(int dt) { return dt == FP8Q_BF16 ? 2 : 4; }
bool dtype_ok(int dt) { return dt == FP8Q_BF16 || dt == FP8Q_F32; }

int from_hip(hipError_t e) { return e == hipSuccess ? FP8Q_OK : FP8Q_ERR_HIP; }

// Shared validation of the two plain GEMM entry points; on success the
// caller launches.
int check_gemm(int kind, int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda,
                      const float* a_scales, const uint8_t* b, int64_t ldb, const float* b_scales, void* c,
                      int c_dtype, int64_t ldc, int accumulate, bool* nothing_to_do) {
  *nothing_to_do = false;
  if (kind != FP8Q_FPROP && kind != FP8Q_DGRAD && kind != FP8Q_WGRAD) return FP8Q_ERR_ARG;
  if (!dtype_ok(c_dtype) || (accumulate != 0 && accumulate != 1)) return FP8Q_ERR_ARG;
  if (M < 0 || N < 0 || K < 0) return FP8Q_ERR_SHAPE;
  if (M == 0 || N == 0) {
    *nothing_to_do = true;
    return FP8Q_OK;
  }
  if (!c) return FP8Q_ERR_NULL;
  if (K > 0 && (!a || !b || !a_scales || !b_scales)) return FP8Q_ERR_NULL;
  if (ldc < N || (K > 0 && (lda < K || ldb < K))) return FP8Q_ERR_SHAPE;
  const int64_t es = dtype_size(c_dtype);
  if (!aligned16(c) || !ld16(ldc, es)) return FP8Q_ERR_ALIGN;
  if (K > 0 && (!aligned16(a) || !aligned16(b) || !aligned16(a_scales) || !aligned16(b_scales) ||
                lda % 16 || ldb % 16))
    return FP8Q_ERR_ALIGN;
  if (M % 128 || N % 128 || K % 128) return FP8Q_ERR_UNSUPPORTED;
  if (accumulate && c_dtype != FP8Q_F32) return FP8Q_ERR_UNSUPPORTED;
  if (K > 0 && (lda > kMaxGemmLd || ldb > kMaxGemmLd)) return FP8Q_ERR_UNSUPPORTED;
  if (N / 128 > kMaxGridX / (M / 128)) return FP8Q_ERR_UNSUPPORTED;   // tiles beyond one grid
  int64_t nsa = 0, nsb = 0;
  if (!mul_ok(K / 128, M, &nsa) || !mul_ok(K / 128, N, &nsb)) return FP8Q_ERR_SHAPE;
  if (kind != FP8Q_WGRAD) nsb = (N / 128) * (K / 128);
  const Range rc = span(c, M, N, ldc, es);
  const Range ins[4] = {span(a, M, K, lda, 1), span(b, N, K, ldb, 1),
                        span(a_scales, 1, nsa, nsa, 4), span(b_scales, 1, nsb, nsb, 4)};
  if (!rc.ok) return FP8Q_ERR_SHAPE;
  for (int i = 0; i < 4; ++i)
    if (!ins[i].ok) return FP8Q_ERR_SHAPE;
  for (int i = 0; i < 4; ++i)
    if (overlap(rc, ins[i])) return FP8Q_ERR_ALIAS;
  return FP8Q_OK;
}

}  // namespace

extern "C" {

int fp8q_abi_version(void) { return 104; }

const char* fp8q_status_string(int s) {
  switch (s) {
    case FP8Q_OK: return "FP8Q_OK";
    case FP8Q_ERR_NULL: return "FP8Q_ERR_NULL: a required pointer is NULL";
    case FP8Q_ERR_SHAPE: return "FP8Q_ERR_SHAPE: negative size or leading dimension too small";
    case FP8Q_ERR_ALIGN: return "FP8Q_ERR_ALIGN: pointer or leading dimension not 16-byte aligned";
    case FP8Q_ERR_UNSUPPORTED: return "FP8Q_ERR_UNSUPPORTED: shape or dtype outside the supported set";
    case FP8Q_ERR_ALIAS: return "FP8Q_ERR_ALIAS: an output overlaps an input or another output";
    case FP8Q_ERR_HIP: return "FP8Q_ERR_HIP: kernel launch failed";
    case FP8Q_ERR_ARG: return "FP8Q_ERR_ARG: unknown enum value";
    default: return "unknown fp8q status";
  }
}

int fp8_quant_tile(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                   int tile, int mode, uint8_t* q, int64_t ld_q, float* scales, void* stream) {
  if (!dtype_ok(x_dtype)) return FP8Q_ERR_ARG;
  if (tile != FP8Q_TILE_1x128 && tile != FP8Q_TILE_128x1) return FP8Q_ERR_ARG;
  if (mode != FP8Q_SCALE_MAXABS && mode != FP8Q_SCALE_POW2) return FP8Q_ERR_ARG;
  if (rows < 0 || cols < 0) return FP8Q_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP8Q_OK;
  if (!x || !q || !scales) return FP8Q_ERR_NULL;
  const int64_t es = dtype_size(x_dtype);
  if (ld_x < cols) return FP8Q_ERR_SHAPE;
  const bool t1x128 = tile == FP8Q_TILE_1x128;
  if (ld_q < (t1x128 ? cols : rows)) return FP8Q_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(q) || !aligned16(scales) || !ld16(ld_x, es) || ld_q % 16)
    return FP8Q_ERR_ALIGN;
  if (t1x128) {
    if (cols % 128) return FP8Q_ERR_UNSUPPORTED;
  } else {
    if (rows % 128 || cols % 8) return FP8Q_ERR_UNSUPPORTED;
  }
  int64_t nscale = 0;
  if (!(t1x128 ? mul_ok(cols / 128, rows, &nscale) : mul_ok(rows / 128, cols, &nscale))) return FP8Q_ERR_SHAPE;
  const Range rx = span(x, rows, cols, ld_x, es);
  const Range rq = t1x128 ? span(q, rows, cols, ld_q, 1) : span(q, cols, rows, ld_q, 1);
  const Range rs = span(scales, 1, nscale, nscale, 4);
  if (!rx.ok || !rq.ok || !rs.ok) return FP8Q_ERR_SHAPE;
  if (overlap(rx, rq) || overlap(rx, rs) || overlap(rq, rs)) return FP8Q_ERR_ALIAS;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool bf16 = x_dtype == FP8Q_BF16;
  return from_hip(t1x128 ? fp8q::launch_quant_1x128(x, bf16, rows, cols, ld_x, mode, q, ld_q, scales, st)
                         : fp8q::launch_quant_128x1(x, bf16, rows, cols, ld_x, mode, q, ld_q, scales, st));
}

int fp8_quant_block(const void* w, int w_dtype, int64_t rows, int64_t cols, int64_t ld_w, int mode,
                    uint8_t* q, int64_t ld_q, float* scales,
                    uint8_t* q_t, int64_t ld_qt, float* scales_t, void* stream) {
  if (!dtype_ok(w_dtype)) return FP8Q_ERR_ARG;
  if (mode != FP8Q_SCALE_MAXABS && mode != FP8Q_SCALE_POW2) return FP8Q_ERR_ARG;
  if (rows < 0 || cols < 0) return FP8Q_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP8Q_OK;
  if (!w || !q || !scales) return FP8Q_ERR_NULL;
  if (q_t && !scales_t) return FP8Q_ERR_NULL;
  if (scales_t && !q_t) return FP8Q_ERR_ARG;         // the transposed pair comes together
  const int64_t es = dtype_size(w_dtype);
  if (ld_w < cols || ld_q < cols || (q_t && ld_qt < rows)) return FP8Q_ERR_SHAPE;
  if (!aligned16(w) || !aligned16(q) || !aligned16(scales) || !ld16(ld_w, es) || ld_q % 16)
    return FP8Q_ERR_ALIGN;
  if (q_t && (!aligned16(q_t) || !aligned16(scales_t) || ld_qt % 16)) return FP8Q_ERR_ALIGN;
  if (rows % 128 || cols % 128) return FP8Q_ERR_UNSUPPORTED;

  int64_t nscale = 0;
  if (!mul_ok(rows / 128, cols / 128, &nscale)) return FP8Q_ERR_SHAPE;
  const Range rw = span(w, rows, cols, ld_w, es);
  const Range rq = span(q, rows, cols, ld_q, 1);
  const Range rs = span(scales, 1, nscale, nscale, 4);
  const Range rqt = q_t ? span(q_t, cols, rows, ld_qt, 1) : Range{0, 0, true};
  const Range rst = scales_t ? span(scales_t, 1, nscale, nscale, 4) : Range{0, 0, true};
  const Range outs[4] = {rq, rs, rqt, rst};
  if (!rw.ok) return FP8Q_ERR_SHAPE;
  for (int i = 0; i < 4; ++i)
    if (!outs[i].ok) return FP8Q_ERR_SHAPE;
  for (int i = 0; i < 4; ++i) {
    if (overlap(rw, outs[i])) return FP8Q_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return FP8Q_ERR_ALIAS;
  }
  return from_hip(fp8q::launch_quant_128x128(w, w_dtype == FP8Q_BF16, rows, cols, ld_w, mode, q, ld_q,
                                             scales, q_t, ld_qt, scales_t,
                                             reinterpret_cast<hipStream_t>(stream)));
}

int fp8_quant_tile_dual(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x, int mode,
                        uint8_t* q, int64_t ld_q, float* scales,
                        uint8_t* q_t, int64_t ld_qt, float* scales_t, void* stream) {
  if (!dtype_ok(x_dtype)) return FP8Q_ERR_ARG;
  if (mode != FP8Q_SCALE_MAXABS && mode != FP8Q_SCALE_POW2) return FP8Q_ERR_ARG;
  if (rows < 0 || cols < 0) return FP8Q_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP8Q_OK;
  if (!x || !q || !scales || !q_t || !scales_t) return FP8Q_ERR_NULL;
  const int64_t es = dtype_size(x_dtype);
  if (ld_x < cols || ld_q < cols || ld_qt < rows) return FP8Q_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(q) || !aligned16(scales) || !aligned16(q_t) || !aligned16(scales_t) ||
      !ld16(ld_x, es) || ld_q % 16 || ld_qt % 16)
    return FP8Q_ERR_ALIGN;
  if (rows % 128 || cols % 128) return FP8Q_ERR_UNSUPPORTED;
  int64_t n1 = 0, n2 = 0;
  if (!mul_ok(cols / 128, rows, &n1) || !mul_ok(rows / 128, cols, &n2)) return FP8Q_ERR_SHAPE;
  const Range rx = span(x, rows, cols, ld_x, es);
  const Range outs[4] = {span(q, rows, cols, ld_q, 1), span(scales, 1, n1, n1, 4),
                         span(q_t, cols, rows, ld_qt, 1), span(scales_t, 1, n2, n2, 4)};
  if (!rx.ok) return FP8Q_ERR_SHAPE;
  for (int i = 0; i < 4; ++i)
    if (!outs[i].ok) return FP8Q_ERR_SHAPE;
  for (int i = 0; i < 4; ++i) {
    if (overlap(rx, outs[i])) return FP8Q_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return FP8Q_ERR_ALIAS;
  }
  return from_hip(fp8q::launch_quant_dual(x, x_dtype == FP8Q_BF16, rows, cols, ld_x, mode, q, ld_q, scales,
                                          q_t, ld_qt, scales_t, reinterpret_cast<hipStream_t>(stream)));
}

int fp8_requant_1x128_to_128x1(const uint8_t* q, int64_t rows, int64_t cols, int64_t ld_q,
                               const float* scales, int mode,
                               uint8_t* q_t, int64_t ld_qt, float* scales_t, void* stream) {
  if (mode != FP8Q_SCALE_MAXABS && mode != FP8Q_SCALE_POW2) return FP8Q_ERR_ARG;
  if (rows < 0 || cols < 0) return FP8Q_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP8Q_OK;
  if (!q || !scales || !q_t || !scales_t) return FP8Q_ERR_NULL;
  if (ld_q < cols || ld_qt < rows) return FP8Q_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(scales) || !aligned16(q_t) || !aligned16(scales_t) || ld_q % 16 ||
      ld_qt % 16)
    return FP8Q_ERR_ALIGN;
  if (rows % 128 || cols % 128) return FP8Q_ERR_UNSUPPORTED;
  int64_t nscale = 0;                           // same count on both sides
  if (!mul_ok(rows / 128, cols, &nscale)) return FP8Q_ERR_SHAPE;
  const Range ins[2] = {span(q, rows, cols, ld_q, 1), span(scales, 1, nscale, nscale, 4)};
  const Range outs[2] = {span(q_t, cols, rows, ld_qt, 1), span(scales_t, 1, nscale, nscale, 4)};
  if (!ins[0].ok || !ins[1].ok || !outs[0].ok || !outs[1].ok) return FP8Q_ERR_SHAPE;
  if (overlap(outs[0], outs[1])) return FP8Q_ERR_ALIAS;
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j)
      if (overlap(ins[i], outs[j])) return FP8Q_ERR_ALIAS;
  return from_hip(fp8q::launch_requant_128x1(q, rows, cols, ld_q, scales, mode, q_t, ld_qt, scales_t,
                                             reinterpret_cast<hipStream_t>(stream)));
}

int fp8_gemm_blockscaled(int kind, int64_t M, int64_t N, int64_t K,
                         const uint8_t* a, int64_t lda, const float* a_scales,
                         const uint8_t* b, int64_t ldb, const float* b_scales,
                         void* c, int c_dtype, int64_t ldc, int accumulate, void* stream) {
  bool nothing = false;
  const int st = check_gemm(kind, M, N, K, a, lda, a_scales, b, ldb, b_scales, c, c_dtype, ldc, accumulate,
                            &nothing);
  if (st != FP8Q_OK || nothing) return st;
  return from_hip(fp8q::launch_gemm(kind, M, N, K, a, lda, a_scales, b, ldb, b_scales, c,
                                    c_dtype == FP8Q_BF16, ldc, accumulate != 0,
                                    reinterpret_cast<hipStream_t>(stream)));
}

int fp8_gemm_blockscaled_pow2(int kind, int64_t M, int64_t N, int64_t K,
                              const uint8_t* a, int64_t lda, const float* a_scales,
                              const uint8_t* b, int64_t ldb, const float* b_scales,
                              void* c, int c_dtype, int64_t ldc, int accumulate, int pow2_operands,
                              void* stream) {
  if (pow2_operands != FP8Q_POW2_A && pow2_operands != FP8Q_POW2_B && pow2_operands != FP8Q_POW2_AB)
    return FP8Q_ERR_ARG;
  bool nothing = false;
  const int st = check_gemm(kind, M, N, K, a, lda, a_scales, b, ldb, b_scales, c, c_dtype, ldc, accumulate,
                            &nothing);
  if (st != FP8Q_OK || nothing) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (pow2_operands == FP8Q_POW2_AB)
    return from_hip(fp8q::launch_gemm_pow2(kind, M, N, K, a, lda, a_scales, b, ldb, b_scales, c,
                                           c_dtype == FP8Q_BF16, ldc, accumulate != 0, s));
  return from_hip(fp8q::launch_gemm_pow2_one(kind, pow2_operands, M, N, K, a, lda, a_scales, b, ldb, b_scales,
                                             c, c_dtype == FP8Q_BF16, ldc, accumulate != 0, s));
}

int fp8_gemm_blockscaled_grouped(int32_t num_groups, int64_t M_total, int64_t N, int64_t K,
                                 const int32_t* group_of_mtile,
                                 const uint8_t* a, int64_t lda, const float* a_scales,
                                 const uint8_t* b, const float* b_scales,
                                 void* c, int c_dtype, int64_t ldc, void* stream) {
  if (!dtype_ok(c_dtype)) return FP8Q_ERR_ARG;
  if (num_groups < 1 || M_total < 0 || N < 0 || K < 0) return FP8Q_ERR_SHAPE;
  if (M_total == 0 || N == 0) return FP8Q_OK;
  if (!c || !group_of_mtile) return FP8Q_ERR_NULL;
  if (K > 0 && (!a || !b || !a_scales || !b_scales)) return FP8Q_ERR_NULL;
  if (ldc < N || (K > 0 && lda < K)) return FP8Q_ERR_SHAPE;
  const int64_t es = dtype_size(c_dtype);
  if (!aligned16(c) || (reinterpret_cast<uintptr_t>(group_of_mtile) & 3u) || !ld16(ldc, es))
    return FP8Q_ERR_ALIGN;
  if (K > 0 && (!aligned16(a) || !aligned16(b) || !aligned16(a_scales) || !aligned16(b_scales) || lda % 16))
    return FP8Q_ERR_ALIGN;
  if (M_total % 128 || N % 128 || K % 128) return FP8Q_ERR_UNSUPPORTED;
  if (K > 0 && (lda > kMaxGemmLd || K > kMaxGemmLd)) return FP8Q_ERR_UNSUPPORTED;
  if (N / 128 > kMaxGridX / (M_total / 128)) return FP8Q_ERR_UNSUPPORTED;   // tiles beyond one grid
  int64_t nsa = 0, nsb = 0, brows = 0;
  if (!mul_ok(K / 128, M_total, &nsa) || !mul_ok(N / 128, K / 128, &nsb) ||
      !mul_ok(int64_t(num_groups), nsb, &nsb) || !mul_ok(int64_t(num_groups), N, &brows))
    return FP8Q_ERR_SHAPE;
  const Range rc = span(c, M_total, N, ldc, es);
  const Range ins[5] = {span(a, M_total, K, lda, 1), span(b, brows, K, K, 1),
                        span(a_scales, 1, nsa, nsa, 4), span(b_scales, 1, nsb, nsb, 4),
                        span(group_of_mtile, 1, M_total / 128, M_total / 128, 4)};
  if (!rc.ok) return FP8Q_ERR_SHAPE;
  for (int i = 0; i < 5; ++i)
    if (!ins[i].ok) return FP8Q_ERR_SHAPE;
  for (int i = 0; i < 5; ++i)
    if (overlap(rc, ins[i])) return FP8Q_ERR_ALIAS;
  return from_hip(fp8q::launch_gemm_grouped(num_groups, M_total, N, K, group_of_mtile, a, lda, a_scales,
                                            b, b_scales, c, c_dtype == FP8Q_BF16, ldc,
                                            reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
