// Wave-level lane exchanges and reductions used by the decode kernels (gfx950: DPP row
// permutes and the v_permlane16/32_swap instructions).
#pragma once

#include <hip/hip_runtime.h>

namespace pkv {

// lane ^ 2 within quads
static __device__ __forceinline__ float dpp_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
}
// lane i of a 16-lane row reads lane 7 - i of its 8-lane half (row_half_mirror)
static __device__ __forceinline__ float dpp_half_mirror(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
}
// lane i of a 16-lane row reads lane 15 - i (row_mirror)
static __device__ __forceinline__ float dpp_mirror(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
}
// lane i of a 16-lane row reads lane (i + n) % 16 (row_ror:n)
template <int N>
static __device__ __forceinline__ float dpp_ror(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xF, 0xF, false));
}

// op over the two 32-lane halves (every lane receives op(x[l], x[l ^ 32]))
template <typename Op>
static __device__ __forceinline__ float across32(float x, Op op) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// op over lanes l and l ^ 16 (every lane receives op(x[l], x[l ^ 16]))
template <typename Op>
static __device__ __forceinline__ float across16(float x, Op op) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// x through an empty register-to-register asm: a select between such values stays a select
// of registers (the optimizer would otherwise turn a select between array elements into a
// select between their addresses, which keeps the array in memory)
static __device__ __forceinline__ float opaque(float x) {
  asm("" : "+v"(x));
  return x;
}

struct MaxOp {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct AddOp {
  __device__ float operator()(float a, float b) const { return a + b; }
};

// max over the wave of values held in equal groups of SPL consecutive lanes (SPL = 2 or 4)
template <int SPL>
static __device__ __forceinline__ float max_over_groups(float x) {
  if constexpr (SPL == 2) x = fmaxf(x, dpp_xor2(x));
  x = fmaxf(x, dpp_half_mirror(x));
  x = fmaxf(x, dpp_mirror(x));
  x = across16(x, MaxOp());
  return across32(x, MaxOp());
}

// sum over the lanes l' of the wave with l' % SPL == l % SPL (SPL = 2 or 4); the order of the
// additions is fixed by the lane index alone
template <int SPL>
static __device__ __forceinline__ float sum_same_class(float x) {
  if constexpr (SPL == 2) x += dpp_xor2(x);
  x += dpp_ror<4>(x);
  x += dpp_ror<8>(x);
  x = across16(x, AddOp());
  return across32(x, AddOp());
}

// sum over lanes l, l ^ k for k = step, 2 step, ..., 32 (step a power of two >= 8)
template <int STEP>
static __device__ __forceinline__ float sum_key_groups(float x) {
  if constexpr (STEP <= 8) x += dpp_ror<8>(x);
  if constexpr (STEP <= 16) x = across16(x, AddOp());
  if constexpr (STEP <= 32) x = across32(x, AddOp());
  return x;
}

}  // namespace pkv
