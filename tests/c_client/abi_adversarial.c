/*
 * Argument validation of the fp8q C ABI (include/fp8q.h) against adversarial
 * sizes, leading dimensions and addresses: sizes whose byte extents overflow
 * 64 bits, buffers that would wrap past the top of the address space, tile
 * counts beyond one launch grid.  Linked with abi.cpp and host stand-ins for
 * the launchers (no GPU); every call must return its documented status, and a
 * request that passes validation must reach exactly one launcher.
 */
#include <stdint.h>
#include <stdio.h>

#include "fp8q.h"

extern int fp8q_stub_launches;

static int failures = 0;

#define EXPECT(call, want)                                                                      \
  do {                                                                                          \
    const int got_ = (call);                                                                    \
    if (got_ != (want)) {                                                                       \
      fprintf(stderr, "line %d: %s returned %s, expected %s\n", __LINE__, #call,                \
              fp8q_status_string(got_), fp8q_status_string(want));                              \
      ++failures;                                                                               \
    }                                                                                           \
  } while (0)

#define LAUNCHES(call, n)                                                                       \
  do {                                                                                          \
    const int before_ = fp8q_stub_launches;                                                     \
    EXPECT(call, FP8Q_OK);                                                                      \
    if (fp8q_stub_launches - before_ != (n)) {                                                  \
      fprintf(stderr, "line %d: %s launched %d times\n", __LINE__, #call,                      \
              fp8q_stub_launches - before_);                                                    \
      ++failures;                                                                               \
    }                                                                                           \
  } while (0)

int main(void) {
  /* plausible, aligned, disjoint fake device addresses (never dereferenced) */
  void* A = (void*)(uintptr_t)0x100000000ull;
  uint8_t* B = (uint8_t*)(uintptr_t)0x200000000ull;
  float* C = (float*)(uintptr_t)0x300000000ull;
  float* D = (float*)(uintptr_t)0x400000000ull;
  uint8_t* E = (uint8_t*)(uintptr_t)0x500000000ull;
  void* F = (void*)(uintptr_t)0x600000000ull;
  /* 16-byte aligned, 64 bytes below the top of the address space */
  void* TOP = (void*)(uintptr_t)(UINTPTR_MAX - 63u);
  const int64_t BIG = INT64_MAX / 256 * 128;       /* a multiple of 128 near 2^62 */
  const int64_t HUGE_LD = INT64_MAX / 4 / 16 * 16; /* a multiple of 16 near 2^61 */

  /* valid requests reach the launcher */
  LAUNCHES(fp8_quant_tile(A, FP8Q_BF16, 256, 384, 384, FP8Q_TILE_1x128, FP8Q_SCALE_MAXABS, B, 384, C, NULL), 1);
  LAUNCHES(fp8_quant_block(A, FP8Q_F32, 256, 384, 384, FP8Q_SCALE_POW2, B, 384, C, E, 256, D, NULL), 1);
  LAUNCHES(fp8_gemm_blockscaled(FP8Q_WGRAD, 256, 256, 512, B, 512, C, E, 512, D, F, FP8Q_F32, 256, 1, NULL), 1);

  /* fp8_quant_tile: extents that overflow */
  EXPECT(fp8_quant_tile(A, FP8Q_F32, BIG, 128, HUGE_LD, FP8Q_TILE_1x128, FP8Q_SCALE_MAXABS, B, 128, C, NULL),
         FP8Q_ERR_SHAPE);
  EXPECT(fp8_quant_tile(A, FP8Q_BF16, 128, BIG, BIG, FP8Q_TILE_1x128, FP8Q_SCALE_MAXABS, B, BIG, C, NULL),
         FP8Q_ERR_SHAPE);
  EXPECT(fp8_quant_tile(A, FP8Q_BF16, BIG, 128, 128, FP8Q_TILE_128x1, FP8Q_SCALE_POW2, B, BIG, C, NULL),
         FP8Q_ERR_SHAPE);
  EXPECT(fp8_quant_tile(A, FP8Q_BF16, 128, 128, INT64_MAX / 16 * 8, FP8Q_TILE_1x128, FP8Q_SCALE_MAXABS, B, 128, C,
                        NULL),
         FP8Q_ERR_SHAPE);                                     /* ld_x * 2 bytes overflows */
  EXPECT(fp8_quant_tile(TOP, FP8Q_F32, 128, 128, 128, FP8Q_TILE_1x128, FP8Q_SCALE_MAXABS, B, 128, C, NULL),
         FP8Q_ERR_SHAPE);                                     /* input wraps past the top */
  EXPECT(fp8_quant_tile(A, FP8Q_F32, 128, 128, 128, FP8Q_TILE_1x128, FP8Q_SCALE_MAXABS, B, 128, (float*)TOP, NULL),
         FP8Q_ERR_SHAPE);                                     /* scales wrap */

  /* fp8_quant_block / dual / requant */
  EXPECT(fp8_quant_block(A, FP8Q_F32, BIG, 128, 128, FP8Q_SCALE_MAXABS, B, HUGE_LD, C, NULL, 0, NULL, NULL),
         FP8Q_ERR_SHAPE);
  EXPECT(fp8_quant_block(A, FP8Q_F32, 256, 384, 384, FP8Q_SCALE_MAXABS, B, 384, C, E, HUGE_LD, D, NULL),
         FP8Q_ERR_SHAPE);
  EXPECT(fp8_quant_block(A, FP8Q_F32, 256, 384, 384, FP8Q_SCALE_MAXABS, B, 384, C, NULL, 0, D, NULL),
         FP8Q_ERR_ARG);                                       /* scales_t without q_t */
  EXPECT(fp8_quant_tile_dual(A, FP8Q_BF16, BIG, BIG, BIG, FP8Q_SCALE_MAXABS, B, BIG, C, E, BIG, D, NULL),
         FP8Q_ERR_SHAPE);
  EXPECT(fp8_quant_tile_dual(A, FP8Q_BF16, 256, 256, 256, FP8Q_SCALE_MAXABS, B, 256, C, (uint8_t*)TOP, 256, D,
                             NULL),
         FP8Q_ERR_SHAPE);
  EXPECT(fp8_requant_1x128_to_128x1(B, BIG, 128, 128, C, FP8Q_SCALE_POW2, E, BIG, D, NULL), FP8Q_ERR_SHAPE);
  EXPECT(fp8_requant_1x128_to_128x1(B, 256, 256, 256, C, FP8Q_SCALE_POW2, (uint8_t*)TOP, 256, D, NULL),
         FP8Q_ERR_SHAPE);

  /* GEMMs */
  EXPECT(fp8_gemm_blockscaled(FP8Q_FPROP, BIG, 128, 128, B, 128, C, E, 128, D, F, FP8Q_BF16, 128, 0, NULL),
         FP8Q_ERR_UNSUPPORTED);                               /* more tiles than one grid */
  EXPECT(fp8_gemm_blockscaled(FP8Q_FPROP, 128 * 128, 128, BIG, B, BIG, C, E, BIG, D, F, FP8Q_BF16, 128, 0, NULL),
         FP8Q_ERR_UNSUPPORTED);                               /* rows of A and B beyond 32-bit tile offsets */
  EXPECT(fp8_gemm_blockscaled(FP8Q_FPROP, 256, 256, 256, B, HUGE_LD, C, E, 256, D, F, FP8Q_BF16, 256, 0, NULL),
         FP8Q_ERR_UNSUPPORTED);
  EXPECT(fp8_gemm_blockscaled(FP8Q_DGRAD, 256, 256, 256, B, 256, C, E, (int64_t)1 << 22, D, F, FP8Q_BF16, 256, 0,
                              NULL),
         FP8Q_ERR_UNSUPPORTED);                               /* ldb of 4 MiB */
  EXPECT(fp8_gemm_blockscaled(FP8Q_WGRAD, 256, 256, 256, B, 256, C, E, 256, D, F, FP8Q_F32, HUGE_LD, 0, NULL),
         FP8Q_ERR_SHAPE);                                     /* C extent overflows */
  EXPECT(fp8_gemm_blockscaled(FP8Q_WGRAD, 256, 256, 256, B, 256, C, E, 256, D, F, FP8Q_F32, INT64_MAX - 1, 0, NULL),
         FP8Q_ERR_ALIGN);                                     /* ldc * 4 would overflow; not 16-byte rows */
  EXPECT(fp8_gemm_blockscaled(FP8Q_WGRAD, 256, 256, 256, B, 256, C, E, 256, D, F, FP8Q_F32, INT64_MAX - 3, 0, NULL),
         FP8Q_ERR_SHAPE);                                     /* 16-byte rows, but the extent overflows */
  EXPECT(fp8_gemm_blockscaled(FP8Q_FPROP, 256, 256, 256, B, 256, C, E, 256, D, TOP, FP8Q_BF16, 256, 0, NULL),
         FP8Q_ERR_SHAPE);                                     /* C wraps */
  EXPECT(fp8_gemm_blockscaled_pow2(FP8Q_FPROP, 256, 256, 256, (uint8_t*)TOP, 256, C, E, 256, D, F, FP8Q_BF16, 256,
                                   0, FP8Q_POW2_AB, NULL),
         FP8Q_ERR_SHAPE);                                     /* A wraps */
  EXPECT(fp8_gemm_blockscaled_grouped(INT32_MAX, 256, BIG, 128, (const int32_t*)D, B, 128, C, E, (float*)F,
                                      (void*)(uintptr_t)0x700000000ull, FP8Q_BF16, BIG, NULL),
         FP8Q_ERR_UNSUPPORTED);                               /* tiles beyond one grid */
  EXPECT(fp8_gemm_blockscaled_grouped(INT32_MAX, 256, 128 * 1024, 128 * 1024, (const int32_t*)D, B, 128 * 1024, C,
                                      E, (float*)F, (void*)(uintptr_t)0x700000000ull, FP8Q_BF16, 128 * 1024, NULL),
         FP8Q_ERR_SHAPE);                                     /* weight rows x K overflow */
  EXPECT(fp8_gemm_blockscaled_grouped(4, 256, 256, 256, (const int32_t*)D, B, 256, C, E, (float*)F, TOP,
                                      FP8Q_F32, 256, NULL),
         FP8Q_ERR_SHAPE);

  if (failures) {
    fprintf(stderr, "%d adversarial validation failures\n", failures);
    return 1;
  }
  printf("adversarial validation ok (%d launches reached)\n", fp8q_stub_launches);
  return 0;
}
