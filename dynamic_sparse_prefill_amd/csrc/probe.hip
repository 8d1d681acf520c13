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

// The same loop with operands that change from one MFMA to the next: eight
// pre-loaded pairs of pseudo-random bf16 fragments (about unit scale, random
// signs and mantissas) taken in turn, as the operands of attention change from
// tile to tile.  Switching bits in the multipliers cost power that constant
// operands do not, so under a power limit this loop settles at a lower clock.
__device__ __forceinline__ float hash_unit(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352dU; x ^= x >> 15; x *= 0x846ca68bU; x ^= x >> 16;
  return (float)(int32_t)x * (1.f / 2147483648.f) * 2.f;   // uniform in [-2, 2)
}

__global__ __launch_bounds__(512, 2) void mfma_loop_data_kernel(float* __restrict__ out, int iters) {
  bf16x8 a[8], b[8];
  const uint32_t t = blockIdx.x * 512u + threadIdx.x;
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[s][i] = (__bf16)hash_unit(t * 128u + 16u * s + i);
      b[s][i] = (__bf16)hash_unit(t * 128u + 16u * s + 8u + i + 0x9e3779b9U);
    }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; it += 2) {
#pragma unroll
    for (int s = 0; s < 8; s += 4) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[s], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s + 1], b[s + 1], c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s + 2], b[s + 2], c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s + 3], b[s + 3], c3, 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" int crisp_probe_mfma_bf16_data(float* out, int blocks, int iters, void* stream) {
  if (out == nullptr || blocks < 1 || blocks > 65536 || iters < 2 || iters > (1 << 26) || (iters & 1)) return -1;
  mfma_loop_data_kernel<<<blocks, 512, 0, (hipStream_t)stream>>>(out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int crisp_probe_mfma_bf16(float* out, int blocks, int iters, void* stream) {
  if (out == nullptr || blocks < 1 || blocks > 65536 || iters < 1 || iters > (1 << 26)) return -1;
  mfma_loop_kernel<<<blocks, 512, 0, (hipStream_t)stream>>>(out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
