// Block-scaled FP8 GEMMs with FP32 promotion once per K-group: Fprop, Dgrad,
// Wgrad and grouped Fprop, plus the variants with one operand's power-of-two
// scales applied by the MFMA (the kernel itself is in gemm_kernel.h).
// Compiled with MFMA results in VGPRs, where the promotion FMAs read them.
#include "gemm_kernel.h"

namespace fp8q {

hipError_t launch_gemm(int kind, int64_t M, int64_t N, int64_t K,
                       const uint8_t* a, int64_t lda, const float* sa,
                       const uint8_t* b, int64_t ldb, const float* sb,
                       void* c, bool out_bf16, int64_t ldc, bool accumulate, hipStream_t st) {
  GemmArgs args{a, lda, sa, b, ldb, sb, c, ldc, M, N, K, nullptr, 0, 0, 0, M};
  const int out = out_code(out_bf16, accumulate);
  if (kind == 2) return launch_out<kScaleRow, false, kHwNone>(args, out, st);
  return launch_out<kScaleBlock, false, kHwNone>(args, out, st);
}

// One operand's power-of-two scales applied by the MFMA, the other's by the
// promotion FMA (pow2_operands 1: A, 2: B).
hipError_t launch_gemm_pow2_one(int kind, int pow2_operands, int64_t M, int64_t N, int64_t K,
                                const uint8_t* a, int64_t lda, const float* sa,
                                const uint8_t* b, int64_t ldb, const float* sb,
                                void* c, bool out_bf16, int64_t ldc, bool accumulate, hipStream_t st) {
  GemmArgs args{a, lda, sa, b, ldb, sb, c, ldc, M, N, K, nullptr, 0, 0, 0, M};
  const int out = out_code(out_bf16, accumulate);
  if (pow2_operands == kHwA) {
    if (kind == 2) return launch_out<kScaleRow, false, kHwA>(args, out, st);
    return launch_out<kScaleBlock, false, kHwA>(args, out, st);
  }
  if (kind == 2) return launch_out<kScaleRow, false, kHwB>(args, out, st);
  return launch_out<kScaleBlock, false, kHwB>(args, out, st);
}

hipError_t launch_gemm_grouped(int32_t num_groups, int64_t M_total, int64_t N, int64_t K,
                               const int32_t* group_of_mtile,
                               const uint8_t* a, int64_t lda, const float* sa,
                               const uint8_t* b, const float* sb,
                               void* c, bool out_bf16, int64_t ldc, hipStream_t st) {
  GemmArgs args{a, lda, sa, b, K, sb, c, ldc, M_total, N, K,
                group_of_mtile, num_groups, N * K, (N / 128) * (K / 128), M_total};
  return launch_out<kScaleBlock, true, kHwNone>(args, out_code(out_bf16, false), st);
}

}  // namespace fp8q
