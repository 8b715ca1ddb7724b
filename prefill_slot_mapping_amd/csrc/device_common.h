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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------------------

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) x = fmaxf(x, __shfl_xor(x, k));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) x += __shfl_xor(x, k);
  return x;
}

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// K/V rows are streamed once: nontemporal loads
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// value of lane ^ 1 (DPP quad permutation [1, 0, 3, 2])
__device__ __forceinline__ float dpp_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}

// max over a wave whose lanes hold values in equal pairs (lane 2k == lane 2k+1)
__device__ __forceinline__ float wave_max_pairs(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF,
                                                           false)));   // lane ^ 2
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF,
                                                           false)));   // half-row mirror
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF,
                                                           false)));   // row mirror
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

}  // namespace pkv
