// Split merge for gfx950 (MI355X).
//
// Source of the operation: "P3: native paged-KV continuous-batching sampler", section
// "Design > paged.py" (a fixed KV split per context length, no atomics): the partials of a
// row's splits are combined in a fixed order, so the result never depends on how the work was
// scheduled.
//
// For one (row, query head) with split partials (m_s, l_s, acc_s), s = 0 .. n-1, in the
// base-2 domain:  M = max_s m_s;  w_s = 2^(m_s - M);  out = (sum_s w_s acc_s) / (sum_s w_s l_s),
// both sums taken as float32 fused multiply-adds in ascending s.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "kernels.h"

namespace pkv {

// value of lane `src` (wave-uniform) as a scalar
__device__ __forceinline__ float lane_value(float x, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), src));
}

// splits s .. s + U - 1 of a chunk folded into num / den in ascending order: the U loads of
// this lane's columns first, then the fused multiply-adds (w_s, l_s held by lane s of the chunk)
template <int U, int C>
__device__ __forceinline__ void fold_splits(const float* accp, int64_t stride, int s, float wl,
                                            float ll, float (&num)[C], float& den) {
  float v[U][C];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int c = 0; c < C; ++c) v[u][c] = accp[(s + u) * stride + c];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float fw = lane_value(wl, s + u);
    den = fmaf(fw, lane_value(ll, s + u), den);
#pragma unroll
    for (int c = 0; c < C; ++c) num[c] = fmaf(fw, v[u][c], num[c]);
  }
}

// a row of U <= 8 splits: the accumulator loads, then m_s and l_s (lane s < U; the other
// lanes read split 0's and drop them), then the maximum, the weights and the ascending sums
template <int U, int C>
__device__ __forceinline__ void fold_row(const float* acc0, const float* pm, const float* pl,
                                         int64_t ps, int64_t stride, float (&num)[C],
                                         float& den) {
  float v[U][C];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int c = 0; c < C; ++c) v[u][c] = acc0[u * stride + c];
  const int lane = threadIdx.x & 63;
  const int64_t ix = lane < U ? lane * ps : 0;
  const float mraw = pm[ix], lraw = pl[ix];
  const float mv = lane < U ? mraw : -INFINITY;
  const float M = wave_max(fmaxf(-INFINITY, mv));
  const float wl = lane < U ? fast_exp2(mv - M) : 0.f;
  const float ll = lane < U ? lraw : 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float fw = lane_value(wl, u);
    den = fmaf(fw, lane_value(ll, u), den);
#pragma unroll
    for (int c = 0; c < C; ++c) num[c] = fmaf(fw, v[u][c], num[c]);
  }
}

// One wave per (row, query head); 4 waves per workgroup. Lane s holds split s's m and l
// (chunks of 64 splits), each lane owns D / 64 output columns.
template <int D>
__global__ void __launch_bounds__(256) merge_kernel(MergeArgs a) {
  constexpr int C = D / 64;  // columns per lane
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (w >= a.n_waves) return;
  const int item = w / a.hq;
  const int h = w - item * a.hq;
  const MergeItem it = a.items[item];
  const int n = it.n_splits;
  const int64_t p0 = static_cast<int64_t>(it.part) * a.hq + h;  // partial index of split 0
  const int64_t ps = a.hq;                                       // stride between splits

  float num[C], den = 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c) num[c] = 0.f;
  const float* acc0 = a.part_acc + p0 * D + lane * C;
  if (n <= 8) {
    // the usual row: every split's accumulator columns, m and l requested together, then the
    // same maximum, weights and ascending sums as below
    const float* pm = a.part_m + p0;
    const float* pl = a.part_l + p0;
    switch (n) {
      case 8: fold_row<8, C>(acc0, pm, pl, ps, ps * D, num, den); break;
      case 7: fold_row<7, C>(acc0, pm, pl, ps, ps * D, num, den); break;
      case 6: fold_row<6, C>(acc0, pm, pl, ps, ps * D, num, den); break;
      case 5: fold_row<5, C>(acc0, pm, pl, ps, ps * D, num, den); break;
      case 4: fold_row<4, C>(acc0, pm, pl, ps, ps * D, num, den); break;
      case 3: fold_row<3, C>(acc0, pm, pl, ps, ps * D, num, den); break;
      case 2: fold_row<2, C>(acc0, pm, pl, ps, ps * D, num, den); break;
      case 1: fold_row<1, C>(acc0, pm, pl, ps, ps * D, num, den); break;
      default: break;
    }
    float* o = a.out + (static_cast<int64_t>(it.row) * a.hq + h) * D + lane * C;
#pragma unroll
    for (int c = 0; c < C; ++c) o[c] = num[c] / den;
    return;
  }

  float M = -INFINITY;
  for (int s0 = 0; s0 < n; s0 += 64)
    if (s0 + lane < n) M = fmaxf(M, a.part_m[p0 + (s0 + lane) * ps]);
  M = wave_max(M);
  for (int s0 = 0; s0 < n; s0 += 64) {
    const int my = s0 + lane;
    float wl = 0.f, ll = 0.f;
    if (my < n) {
      wl = fast_exp2(a.part_m[p0 + my * ps] - M);
      ll = a.part_l[p0 + my * ps];
    }
    const int cnt = min(64, n - s0);
    const float* accp = a.part_acc + (p0 + s0 * ps) * D + lane * C;
    const int64_t stride = ps * D;
    // 8 splits' accumulator loads in flight at a time, the remaining 1-7 as one group of that
    // size (a row's few splits read together); the sums stay in ascending order
    int s = 0;
    for (; s + 8 <= cnt; s += 8) fold_splits<8, C>(accp, stride, s, wl, ll, num, den);
    switch (cnt - s) {
      case 7: fold_splits<7, C>(accp, stride, s, wl, ll, num, den); break;
      case 6: fold_splits<6, C>(accp, stride, s, wl, ll, num, den); break;
      case 5: fold_splits<5, C>(accp, stride, s, wl, ll, num, den); break;
      case 4: fold_splits<4, C>(accp, stride, s, wl, ll, num, den); break;
      case 3: fold_splits<3, C>(accp, stride, s, wl, ll, num, den); break;
      case 2: fold_splits<2, C>(accp, stride, s, wl, ll, num, den); break;
      case 1: fold_splits<1, C>(accp, stride, s, wl, ll, num, den); break;
      default: break;
    }
  }
  float* o = a.out + (static_cast<int64_t>(it.row) * a.hq + h) * D + lane * C;
#pragma unroll
  for (int c = 0; c < C; ++c) o[c] = num[c] / den;
}

hipError_t launch_merge(const MergeArgs& a, int64_t n_items, int head_dim, hipStream_t stream) {
  const int64_t waves = n_items * a.hq;
  if (waves == 0) return hipSuccess;
  if (waves > 0x7fffffffLL || waves != a.n_waves) return hipErrorInvalidValue;
  const uint32_t grid = static_cast<uint32_t>((waves + 3) / 4);
  if (head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, dim3(grid), dim3(256), 0, stream, a);
  else if (head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3(grid), dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
