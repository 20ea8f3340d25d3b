// libtj2_measure: measurement helpers that bench.py times beside the products.
// They are not part of the path and are built into a library of their own, so
// the product library libtj2 carries none of them (include/tj2_measure.h).
//
// tj2_mfma_peak_probe: the achievable dense f16 MFMA rate of the part.  Each
// wave runs four independent v_mfma_f32_32x32x16_f16 accumulation chains on
// register operands (no memory traffic in the loop), the instruction the
// products use.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tj2_measure.h"

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
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

extern "C" int32_t tj2_mfma_peak_probe(int64_t workgroups, int32_t iters, float* out, void* stream) {
  if (!out || workgroups < 1 || workgroups > ((int64_t)1 << 20) || iters < 1 || iters > (1 << 20)) return 1;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((uint32_t)workgroups), dim3(256), 0, (hipStream_t)stream, iters,
                     (_Float16)0.0625f, out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
