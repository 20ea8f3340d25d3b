// Conformance program for gfx950's stochastic-rounding conversions (test code).
//
// Input file: int64 n, float32 v[n], uint32 u[n] (16-bit draws).  For each i it
// converts v[i] with the 16-bit draw placed in the top half of the random
// operand, one element per instruction (the second slot of the packed FP4 form
// holds 0.0), and writes the E2M1 code and the E4M3FN code (uint8 each).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

typedef float float2_t __attribute__((ext_vector_type(2)));

#define CK(x)                                                                   \
  do {                                                                          \
    hipError_t e_ = (x);                                                        \
    if (e_ != hipSuccess) {                                                     \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(2);                                                                  \
    }                                                                           \
  } while (0)

__global__ void convert(const float* v, const unsigned* u, long n, unsigned char* fp4, unsigned char* fp8) {
  long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const unsigned r = u[i] << 16;
  float2_t x = {v[i], 0.0f};
  fp4[i] = (unsigned char)(__builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, x, r, 1.0f, 0) & 0xFu);
  fp8[i] = (unsigned char)(__builtin_amdgcn_cvt_scalef32_sr_fp8_f32(0u, v[i], r, 1.0f, 0) & 0xFFu);
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s input output\n", argv[0]);
    return 1;
  }
  FILE* f = fopen(argv[1], "rb");
  if (!f) return 1;
  long n = 0;
  if (fread(&n, 8, 1, f) != 1 || n <= 0 || n > (1L << 28)) return 1;
  std::vector<float> v(n);
  std::vector<unsigned> u(n);
  if (fread(v.data(), 4, n, f) != (size_t)n || fread(u.data(), 4, n, f) != (size_t)n) return 1;
  fclose(f);
  float* dv;
  unsigned* du;
  unsigned char *d4, *d8;
  CK(hipMalloc(&dv, n * 4));
  CK(hipMalloc(&du, n * 4));
  CK(hipMalloc(&d4, n));
  CK(hipMalloc(&d8, n));
  CK(hipMemcpy(dv, v.data(), n * 4, hipMemcpyHostToDevice));
  CK(hipMemcpy(du, u.data(), n * 4, hipMemcpyHostToDevice));
  convert<<<(unsigned)((n + 255) / 256), 256>>>(dv, du, n, d4, d8);
  CK(hipGetLastError());
  CK(hipDeviceSynchronize());
  std::vector<unsigned char> o4(n), o8(n);
  CK(hipMemcpy(o4.data(), d4, n, hipMemcpyDeviceToHost));
  CK(hipMemcpy(o8.data(), d8, n, hipMemcpyDeviceToHost));
  FILE* g = fopen(argv[2], "wb");
  if (!g) return 1;
  fwrite(o4.data(), 1, n, g);
  fwrite(o8.data(), 1, n, g);
  fclose(g);
  return 0;
}
