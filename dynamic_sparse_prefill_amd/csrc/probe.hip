// Attainable-peak probe: a loop of independent bf16 MFMAs at the occupancy of
// the attention kernel (8 waves per work-group, two per SIMD).  Its sustained
// rate over a launch of a few hundred ms is the ceiling that clock and power
// limits leave for any bf16 MFMA kernel on this GPU.
#include <hip/hip_runtime.h>

#include "crisp_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(512, 2) void mfma_loop_kernel(float* __restrict__ out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(threadIdx.x * 1e-3f + i);
    b[i] = (__bf16)(0.5f * i);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" int crisp_probe_mfma_bf16(float* out, int blocks, int iters, void* stream) {
  if (out == nullptr || blocks < 1 || blocks > 65536 || iters < 1 || iters > (1 << 26)) return -1;
  mfma_loop_kernel<<<blocks, 512, 0, (hipStream_t)stream>>>(out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
