/*
 * A plain C client of the fp8q C ABI (include/fp8q.h), linked against
 * libfp8q.so: what a non-Python caller does.
 *
 *   fp8q_client check           argument validation only (no GPU needed)
 *   fp8q_client run IN OUT      1x128 quantization of X, 128x128 quantization
 *                               of W and the Fprop GEMM Y = X W^T on the GPU
 *
 * IN : int64 M, N, K, then X as M*K BF16 bit patterns and W as N*K (row-major)
 * OUT: codes(X) M*K, scales(X) (K/128)*M float, codes(W) N*K, scales(W)
 *      (N/128)*(K/128) float, Y as M*N BF16 bit patterns
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fp8q.h"

#define EXPECT(call, want)                                                                   \
  do {                                                                                       \
    const int got_ = (call);                                                                 \
    if (got_ != (want)) {                                                                    \
      fprintf(stderr, "%s:%d: %s returned %s, expected %s\n", __FILE__, __LINE__, #call,     \
              fp8q_status_string(got_), fp8q_status_string(want));                           \
      return 1;                                                                              \
    }                                                                                        \
  } while (0)

#define HIP_OK(call)                                                                         \
  do {                                                                                       \
    if ((call) != hipSuccess) {                                                              \
      fprintf(stderr, "%s:%d: %s failed\n", __FILE__, __LINE__, #call);                      \
      return 2;                                                                              \
    }                                                                                        \
  } while (0)

static int check(void) {
  /* fake 16-byte-aligned device addresses: every call below fails validation
     before anything could dereference them */
  void* A = (void*)0x10000;
  uint8_t* B = (uint8_t*)0x20000000;
  float* C = (float*)0x40000000;
  float* D = (float*)0x60000000;
  if (fp8q_abi_version() != 104) return 3;
  if (strncmp(fp8q_status_string(FP8Q_ERR_ALIAS), "FP8Q_ERR_ALIAS", 14) != 0) return 4;
  EXPECT(fp8_quant_tile(A, FP8Q_BF16, 0, 256, 256, FP8Q_TILE_1x128, FP8Q_SCALE_MAXABS, B, 256, C, NULL), FP8Q_OK);
  EXPECT(fp8_quant_tile(A, FP8Q_BF16, 128, 256, 256, FP8Q_TILE_1x128, 7, B, 256, C, NULL), FP8Q_ERR_ARG);
  EXPECT(fp8_quant_tile(NULL, FP8Q_BF16, 128, 256, 256, FP8Q_TILE_1x128, FP8Q_SCALE_MAXABS, B, 256, C, NULL),
         FP8Q_ERR_NULL);
  EXPECT(fp8_quant_tile(A, FP8Q_BF16, 128, 256, 260, FP8Q_TILE_1x128, FP8Q_SCALE_MAXABS, B, 256, C, NULL),
         FP8Q_ERR_ALIGN);                                  /* 520-byte rows */
  EXPECT(fp8_quant_tile(A, FP8Q_BF16, 128, 200, 200, FP8Q_TILE_1x128, FP8Q_SCALE_MAXABS, B, 208, C, NULL),
         FP8Q_ERR_UNSUPPORTED);                            /* 1x128 needs cols % 128 == 0 */
  EXPECT(fp8_quant_block(A, FP8Q_F32, 200, 384, 384, FP8Q_SCALE_POW2, B, 384, C, NULL, 0, NULL, NULL),
         FP8Q_ERR_UNSUPPORTED);
  EXPECT(fp8_quant_tile_dual(A, FP8Q_BF16, 256, 384, 384, FP8Q_SCALE_MAXABS, B, 384, C, NULL, 256, D, NULL),
         FP8Q_ERR_NULL);                                   /* both tilings' outputs are required */
  EXPECT(fp8_quant_tile_dual(A, FP8Q_BF16, 200, 384, 384, FP8Q_SCALE_MAXABS, B, 384, C, B + 0x100000, 208, D,
                             NULL),
         FP8Q_ERR_UNSUPPORTED);                            /* rows must be whole 128-row tiles */
  EXPECT(fp8_gemm_blockscaled(FP8Q_FPROP, 256, 256, 512, B, 512, C, B + 0x100000, 512, D, (void*)0x70000000,
                              FP8Q_BF16, 256, 1, NULL),
         FP8Q_ERR_UNSUPPORTED);                            /* accumulate needs FP32 output */
  EXPECT(fp8_gemm_blockscaled(FP8Q_WGRAD, 256, 256, 512, B, 512, C, B + 0x100000, 512, D, B + 4096,
                              FP8Q_F32, 256, 0, NULL),
         FP8Q_ERR_ALIAS);                                  /* C overlaps A */
  EXPECT(fp8_gemm_blockscaled_pow2(FP8Q_FPROP, 256, 256, 512, B, 512, C, B + 0x100000, 512, D,
                                   (void*)0x70000000, FP8Q_BF16, 256, 0, 4, NULL),
         FP8Q_ERR_ARG);
  EXPECT(fp8_requant_1x128_to_128x1(B, 256, 384, 384, C, FP8Q_SCALE_POW2, B + 256, 256, D, NULL),
         FP8Q_ERR_ALIAS);
  puts("fp8q C ABI: validation ok");
  return 0;
}

static int run(const char* in_path, const char* out_path) {
  FILE* f = fopen(in_path, "rb");
  if (!f) return 5;
  int64_t dims[3];
  if (fread(dims, sizeof(int64_t), 3, f) != 3) return 6;
  const int64_t M = dims[0], N = dims[1], K = dims[2];
  uint16_t* hx = malloc(sizeof(uint16_t) * M * K);
  uint16_t* hw = malloc(sizeof(uint16_t) * N * K);
  if (!hx || !hw) return 7;
  if (fread(hx, sizeof(uint16_t), M * K, f) != (size_t)(M * K) || fread(hw, sizeof(uint16_t), N * K, f) != (size_t)(N * K))
    return 8;
  fclose(f);

  void *x, *w, *y;
  uint8_t *qx, *qw;
  float *sx, *sw;
  const int64_t nsx = (K / 128) * M, nsw = (N / 128) * (K / 128);
  HIP_OK(hipMalloc(&x, 2 * M * K));
  HIP_OK(hipMalloc(&w, 2 * N * K));
  HIP_OK(hipMalloc(&y, 2 * M * N));
  HIP_OK(hipMalloc((void**)&qx, M * K));
  HIP_OK(hipMalloc((void**)&qw, N * K));
  HIP_OK(hipMalloc((void**)&sx, 4 * nsx));
  HIP_OK(hipMalloc((void**)&sw, 4 * nsw));
  HIP_OK(hipMemcpy(x, hx, 2 * M * K, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(w, hw, 2 * N * K, hipMemcpyHostToDevice));

  EXPECT(fp8_quant_tile(x, FP8Q_BF16, M, K, K, FP8Q_TILE_1x128, FP8Q_SCALE_MAXABS, qx, K, sx, NULL), FP8Q_OK);
  EXPECT(fp8_quant_block(w, FP8Q_BF16, N, K, K, FP8Q_SCALE_MAXABS, qw, K, sw, NULL, 0, NULL, NULL), FP8Q_OK);
  EXPECT(fp8_gemm_blockscaled(FP8Q_FPROP, M, N, K, qx, K, sx, qw, K, sw, y, FP8Q_BF16, N, 0, NULL), FP8Q_OK);
  HIP_OK(hipDeviceSynchronize());

  uint8_t* hq = malloc(M * K > N * K ? M * K : N * K);
  float* hs = malloc(4 * (nsx > nsw ? nsx : nsw));
  uint16_t* hy = malloc(2 * M * N);
  if (!hq || !hs || !hy) return 7;
  FILE* o = fopen(out_path, "wb");
  if (!o) return 9;
  HIP_OK(hipMemcpy(hq, qx, M * K, hipMemcpyDeviceToHost));
  fwrite(hq, 1, M * K, o);
  HIP_OK(hipMemcpy(hs, sx, 4 * nsx, hipMemcpyDeviceToHost));
  fwrite(hs, 4, nsx, o);
  HIP_OK(hipMemcpy(hq, qw, N * K, hipMemcpyDeviceToHost));
  fwrite(hq, 1, N * K, o);
  HIP_OK(hipMemcpy(hs, sw, 4 * nsw, hipMemcpyDeviceToHost));
  fwrite(hs, 4, nsw, o);
  HIP_OK(hipMemcpy(hy, y, 2 * M * N, hipMemcpyDeviceToHost));
  fwrite(hy, 2, M * N, o);
  fclose(o);
  hipFree(x); hipFree(w); hipFree(y); hipFree(qx); hipFree(qw); hipFree(sx); hipFree(sw);
  free(hx); free(hw); free(hq); free(hs); free(hy);
  puts("fp8q C ABI: quantize + Fprop ok");
  return 0;
}

int main(int argc, char** argv) {
  if (argc == 2 && strcmp(argv[1], "check") == 0) return check();
  if (argc == 4 && strcmp(argv[1], "run") == 0) return run(argv[2], argv[3]);
  fprintf(stderr, "usage: %s check | run IN OUT\n", argv[0]);
  return 64;
}
