// Small device helpers shared by the HIP translation units.
#pragma once

#include <hip/hip_runtime.h>

namespace pkv {

// The dispatcher sends workgroup b to XCD b % 8. Remap so that each XCD receives a contiguous
// range of work items (neighbouring items share blocks and cache lines in that XCD's L2).
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int q = n >> 3, r = n & 7;
  const int x = b & 7, k = b >> 3;
  return x * q + (x < r ? x : r) + k;
}

// Hardware base-2 exponential (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pkv
