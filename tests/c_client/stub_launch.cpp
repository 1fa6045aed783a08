// Host-only stand-ins for the HIP launchers behind the C ABI, so that the
// argument validation in abi.cpp can be built and run on a machine without a
// GPU (and under the host sanitizers).  Each stub only counts its calls: a
// request that passes validation reaches exactly one launcher.
#include "fp8q_launch.h"

extern "C" {
int fp8q_stub_launches = 0;
}

namespace fp8q {

static hipError_t hit() {
  ++fp8q_stub_launches;
  return hipSuccess;
}

hipError_t launch_quant_1x128(const void*, bool, int64_t, int64_t, int64_t, int, uint8_t*, int64_t, float*,
                              hipStream_t) { return hit(); }
hipError_t launch_quant_128x1(const void*, bool, int64_t, int64_t, int64_t, int, uint8_t*, int64_t, float*,
                              hipStream_t) { return hit(); }
hipError_t launch_quant_128x128(const void*, bool, int64_t, int64_t, int64_t, int, uint8_t*, int64_t, float*,
                                uint8_t*, int64_t, float*, hipStream_t) { return hit(); }
hipError_t launch_quant_dual(const void*, bool, int64_t, int64_t, int64_t, int, uint8_t*, int64_t, float*,
                             uint8_t*, int64_t, float*, hipStream_t) { return hit(); }
hipError_t launch_requant_128x1(const uint8_t*, int64_t, int64_t, int64_t, const float*, int, uint8_t*, int64_t,
                                float*, hipStream_t) { return hit(); }
hipError_t launch_gemm(int, int64_t, int64_t, int64_t, const uint8_t*, int64_t, const float*, const uint8_t*,
                       int64_t, const float*, void*, bool, int64_t, bool, hipStream_t) { return hit(); }
hipError_t launch_gemm_pow2(int, int64_t, int64_t, int64_t, const uint8_t*, int64_t, const float*,
                            const uint8_t*, int64_t, const float*, void*, bool, int64_t, bool, hipStream_t) {
  return hit();
}
hipError_t launch_gemm_pow2_one(int, int, int64_t, int64_t, int64_t, const uint8_t*, int64_t, const float*,
                                const uint8_t*, int64_t, const float*, void*, bool, int64_t, bool, hipStream_t) {
  return hit();
}
hipError_t launch_gemm_grouped(int32_t, int64_t, int64_t, int64_t, const int32_t*, const uint8_t*, int64_t,
                               const float*, const uint8_t*, const float*, void*, bool, int64_t, hipStream_t) {
  return hit();
}

}  // namespace fp8q
