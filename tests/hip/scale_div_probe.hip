// Test helper, not part of the library: runs the quantizers' scale divisions
// (fp8q_device.h: fl32(a / 448) and fl32(448 / a), the max-abs scale pair)
// over a contiguous range of float32 bit patterns, so that a GPU test can
// compare every result with IEEE division computed on the host.
#include "fp8q_device.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

__global__ void scale_div_probe_kernel(uint32_t first, int64_t n, float* __restrict__ s, float* __restrict__ inv) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x) {
    const float a = __uint_as_float(first + uint32_t(i));
    s[i] = fp8q::div_by_448(a);
    inv[i] = fp8q::div_448_by(a);
  }
}

// s[i] = fl32(a_i / 448), inv[i] = fl32(448 / a_i) for a_i = the float32 with
// bits first + i, 0 <= i < n (first + n - 1 must not wrap past 0xFFFFFFFF);
// s and inv are device buffers of n floats.  Returns 0, or 1 on a launch error.
extern "C" int fp8q_scale_div_probe(uint32_t first, int64_t n, float* s, float* inv, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(scale_div_probe_kernel, dim3(8192), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     first, n, s, inv);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
