// Cross-lane reductions over lane pairs without an LDS round trip (gfx950
// v_permlane{16,32}_swap).  Both lanes of a pair get the same result, formed
// in the same order.
#pragma once
#include "common.h"

namespace crisp {

// lanes l and l ^ 32
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// lanes l and l ^ 16
__device__ __forceinline__ float row_pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace crisp
