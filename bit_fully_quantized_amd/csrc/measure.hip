// Measurement helper, not part of the path: the achievable dense f16 MFMA rate
// of the part, against which the products' rate is also reported.  Each wave
// runs four independent v_mfma_f32_32x32x16_f16 accumulation chains on register
// operands (no memory traffic in the loop), the instruction the products use.
#include "tj2_device.h"
#include "tj2_internal.h"

namespace tj2 {

namespace {

typedef float float16v_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_peak_kernel(int32_t iters, _Float16 x, float* __restrict__ out) {
  const half8_t a = {x, x, x, x, x, x, x, x};
  float16v_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int32_t i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c3, 0, 0, 0);
  }
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = ((c0[0] + c1[0]) + c2[0]) + c3[0];
}

}  // namespace

hipError_t launch_mfma_peak(int64_t workgroups, int32_t iters, float* out, hipStream_t s) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((uint32_t)workgroups), dim3(256), 0, s, iters, (_Float16)0.0625f, out);
  return hipGetLastError();
}

}  // namespace tj2
