// Internal launchers behind the C ABI.  Arguments are validated by abi.cpp
// before any of these is called; each enqueues on `st` and returns the launch
// status (hipGetLastError) without synchronising.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fp8q {

hipError_t launch_quant_1x128(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld_x,
                              int mode, uint8_t* q, int64_t ld_q, float* scales, hipStream_t st);

hipError_t launch_quant_128x1(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld_x,
                              int mode, uint8_t* q, int64_t ld_q, float* scales, hipStream_t st);

hipError_t launch_quant_128x128(const void* w, bool bf16, int64_t rows, int64_t cols, int64_t ld_w,
                                int mode, uint8_t* q, int64_t ld_q, float* scales,
                                uint8_t* q_t, int64_t ld_qt, float* scales_t, hipStream_t st);

// 1x128 (q, scales) and 128x1 (q_t, scales_t) tiles of the same input in one pass.
hipError_t launch_quant_dual(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld_x,
                             int mode, uint8_t* q, int64_t ld_q, float* scales,
                             uint8_t* q_t, int64_t ld_qt, float* scales_t, hipStream_t st);

hipError_t launch_requant_128x1(const uint8_t* q, int64_t rows, int64_t cols, int64_t ld_q, const float* s_in,
                                int mode, uint8_t* q_t, int64_t ld_qt, float* s_out, hipStream_t st);

// kind: 0 Fprop, 1 Dgrad (block-scaled B), 2 Wgrad (per-row B scales)
hipError_t launch_gemm(int kind, int64_t M, int64_t N, int64_t K,
                       const uint8_t* a, int64_t lda, const float* sa,
                       const uint8_t* b, int64_t ldb, const float* sb,
                       void* c, bool out_bf16, int64_t ldc, bool accumulate, hipStream_t st);

// Same operands; both operands' power-of-two scales applied by the hardware-scaled MFMA.
hipError_t launch_gemm_pow2(int kind, int64_t M, int64_t N, int64_t K,
                            const uint8_t* a, int64_t lda, const float* sa,
                            const uint8_t* b, int64_t ldb, const float* sb,
                            void* c, bool out_bf16, int64_t ldc, bool accumulate, hipStream_t st);

// One operand power-of-two (1: A, 2: B) applied by the MFMA, the other promoted.
hipError_t launch_gemm_pow2_one(int kind, int pow2_operands, int64_t M, int64_t N, int64_t K,
                                const uint8_t* a, int64_t lda, const float* sa,
                                const uint8_t* b, int64_t ldb, const float* sb,
                                void* c, bool out_bf16, int64_t ldc, bool accumulate, hipStream_t st);

hipError_t launch_gemm_grouped(int32_t num_groups, int64_t M_total, int64_t N, int64_t K,
                               const int32_t* group_of_mtile,
                               const uint8_t* a, int64_t lda, const float* sa,
                               const uint8_t* b, const float* sb,
                               void* c, bool out_bf16, int64_t ldc, hipStream_t st);

}  // namespace fp8q
