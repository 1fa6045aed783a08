// Block-scaled FP8 GEMMs for power-of-two scales on the hardware-scaled MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4): the A-row and B-row/block scales are
// E8M0 operands of the instruction, so the per-group dequantization happens
// inside the matrix core and every K-group accumulates in the MFMA
// accumulators -- no VALU promotion at all.  Group scaling applied by the
// MMA itself is what the pages recommend for future hardware (dssusan.co.kr
// FP8 excerpt, paragraph 3; "Deepseek - Not For everyone", paragraph 4); the
// scales must be integral powers of two (dssusan.co.kr, paragraph 1).
// Compiled with MFMA accumulators in AGPRs: they are never touched by VALU
// code until the epilogue.
#include "gemm_kernel.h"

namespace fp8q {

hipError_t launch_gemm_pow2(int kind, int64_t M, int64_t N, int64_t K,
                            const uint8_t* a, int64_t lda, const float* sa,
                            const uint8_t* b, int64_t ldb, const float* sb,
                            void* c, bool out_bf16, int64_t ldc, bool accumulate, hipStream_t st) {
  GemmArgs args{a, lda, sa, b, ldb, sb, c, ldc, M, N, K, nullptr, 0, 0, 0, M};
  const int out = out_bf16 ? kOutBF16 : (accumulate ? kOutF32Acc : kOutF32);
  if (kind == 2) return launch_out<kScaleRow, false, kHwAB>(args, out, st);
  return launch_out<kScaleBlock, false, kHwAB>(args, out, st);
}

}  // namespace fp8q
