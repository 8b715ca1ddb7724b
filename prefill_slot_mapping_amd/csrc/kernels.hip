// HIP kernels for gfx950 (MI355X): KV append, decode split pass, split merge.
//
// Sources of the operations:
//  - KV append: "P3: native paged-KV continuous-batching sampler", section "Design > paged.py"
//    (PagedKVCache: copy-free append, a write scatters into (block, offset) in place).
//  - Attention contract: same section, TritonPagedAttention (q, k/v cache blocks, block tables,
//    cu_seqlens_q, ctx_lens, slot mapping; a fixed KV split per context length, no atomics),
//    and "Finish RL Training Faster: Bitwise-Consistent ..." section 2 (kernel determinism,
//    batch independence).
//
// Numeric contract of the decode path (every choice below depends only on the row's own
// sequence, never on the batch): the keys of a row are cut into splits of kv_split tokens
// aligned at position 0; inside a split, 64-key tiles aligned at the split start go to wave
// (tile % 4) of the workgroup; each wave runs an online softmax over its tiles in ascending
// order, in the base-2 domain (scores are scaled by scale * log2 e and exponentiated with the
// hardware exp2); the four wave partials are merged in wave order, and the split partials in
// ascending split order by a second kernel. Accumulation is float32 throughout; bfloat16
// products are formed exactly by v_dot2_f32_bf16; probabilities stay float32 for P.V.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "kernels.h"

namespace pkv {

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

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// ---------------------------------------------------------------------------------------
// KV append: row t of k_new / v_new goes to slot slots[t]; a slot row is contiguous in the
// [num_blocks, block_size, Hkv, D] pool at byte offset slot * Hkv * D * elem_bytes.
// ---------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) write_kv_kernel(WriteArgs a) {
  const uint4* __restrict__ kn = static_cast<const uint4*>(a.k_new);
  const uint4* __restrict__ vn = static_cast<const uint4*>(a.v_new);
  uint4* __restrict__ kc = static_cast<uint4*>(a.k_cache);
  uint4* __restrict__ vc = static_cast<uint4*>(a.v_cache);
  const uint32_t chunks = static_cast<uint32_t>(a.chunks_per_row);
  const uint32_t total = static_cast<uint32_t>(a.n_rows) * chunks;
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < total; i += gridDim.x * 256u) {
    const uint32_t row = i / chunks;
    const uint32_t c = i - row * chunks;
    const int32_t s = a.slots[row];
    if (s < 0 || s >= a.n_slots) continue;
    const int64_t dst = static_cast<int64_t>(s) * chunks + c;
    kc[dst] = kn[i];
    vc[dst] = vn[i];
  }
}

hipError_t launch_write_kv(const WriteArgs& a, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(a.n_rows) * a.chunks_per_row;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(write_kv_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                     a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Decode split pass.
//
// Workgroup = 4 waves = one (query row, split, kv head) item; it serves the G query heads that
// read that kv head, so every K/V byte of the split is loaded from HBM once.
// Per 64-key tile a wave
//   1. loads K and V rows with 16-byte coalesced loads (LPT lanes cover one 256/512-byte head
//      row; the block table is read once per key, the slot broadcast by a lane shuffle),
//   2. stages K in LDS with an XOR swizzle on the 16-byte chunk index,
//   3. computes the G scores of one key per lane (no cross-lane reduction),
//   4. updates the per-head running max / sum and publishes p through LDS,
//   5. accumulates P.V in the split-D layout (each lane owns EPL columns of its key group).
// ---------------------------------------------------------------------------------------
template <int D, int G, bool BF>
__global__ void __launch_bounds__(256) decode_split_kernel(DecodeArgs a) {
  constexpr int E = BF ? 2 : 4;
  constexpr int ROWB = D * E;               // bytes of one head row
  constexpr int LPT = ROWB / 16;            // lanes per key row
  constexpr int TPI = 64 / LPT;             // keys per load instruction
  constexpr int NI = kDecodeTile / TPI;     // load instructions per tile
  constexpr int EPL = 16 / E;               // elements per lane chunk
  static_assert(LPT >= 1 && LPT <= 64 && (LPT & (LPT - 1)) == 0, "row must be 16..1024 bytes");

  __shared__ uint4 s_k[kDecodeWaves][kDecodeTile * LPT];
  __shared__ float s_p[kDecodeWaves][kDecodeTile * G];
  __shared__ uint4 s_q[G * LPT];
  __shared__ int s_bad;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int f = xcd_remap(blockIdx.x, gridDim.x);
  const int item_idx = f / a.hkv;
  const int g = f - item_idx * a.hkv;
  const DecodeItem it = a.items[item_idx];

  // the G query heads of this kv head are contiguous in q[row]
  const uint4* qsrc = reinterpret_cast<const uint4*>(
      static_cast<const char*>(a.q) + (static_cast<int64_t>(it.row) * a.hq +
                                       static_cast<int64_t>(g) * G) * ROWB);
  for (int c = tid; c < G * LPT; c += 256) s_q[c] = qsrc[c];
  if (tid == 0) s_bad = 0;
  __syncthreads();

  const int t0 = it.split * a.kv_split;
  const int t1 = min(it.n_keys, t0 + a.kv_split);
  const int32_t* bt = a.block_tables + static_cast<int64_t>(it.seq) * a.max_blocks;
  const uint4* __restrict__ kp = static_cast<const uint4*>(a.k_cache);
  const uint4* __restrict__ vp = static_cast<const uint4*>(a.v_cache);
  const int64_t slot_stride = static_cast<int64_t>(a.hkv) * LPT;  // uint4 per slot
  const int head_off = g * LPT;
  const int grp = lane / LPT;
  const int cl = lane & (LPT - 1);

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  bool bad = false;
  uint4* sk = s_k[wave];
  float* sp = s_p[wave];

  for (int ts = t0 + wave * kDecodeTile; ts < t1; ts += kDecodeWaves * kDecodeTile) {
    const int n = min(kDecodeTile, t1 - ts);
    // slot of this lane's key (key ts + lane)
    int slot_l = 0;
    int ok_l = 0;
    if (lane < n) {
      const int pos = ts + lane;
      const int j = pos / a.block_size;
      const int off = pos - j * a.block_size;
      const int b = bt[j];
      ok_l = static_cast<unsigned>(b) < static_cast<unsigned>(a.num_blocks);
      bad |= !ok_l;
      slot_l = ok_l ? b * a.block_size + off : 0;
    }
    uint4 kr[NI], vr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tok = i * TPI + grp;
      const int sl = __shfl(slot_l, tok);
      const int okk = __shfl(ok_l, tok);
      if (okk) {
        const int64_t off = static_cast<int64_t>(sl) * slot_stride + head_off + cl;
        kr[i] = kp[off];
        vr[i] = vp[off];
      } else {
        kr[i] = make_uint4(0u, 0u, 0u, 0u);
        vr[i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tok = i * TPI + grp;
      sk[tok * LPT + (cl ^ (tok & (LPT - 1)))] = kr[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // scores: lane = key
    float s[G];
    {
      float s0[G], s1[G];
#pragma unroll
      for (int h = 0; h < G; ++h) s0[h] = s1[h] = 0.f;
#pragma unroll
      for (int cc = 0; cc < LPT; ++cc) {
        const uint4 kc = sk[lane * LPT + (cc ^ (lane & (LPT - 1)))];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const uint4 qc = s_q[h * LPT + cc];
          if constexpr (BF) {
            s0[h] = dot2_bf16(qc.x, kc.x, s0[h]);
            s1[h] = dot2_bf16(qc.y, kc.y, s1[h]);
            s0[h] = dot2_bf16(qc.z, kc.z, s0[h]);
            s1[h] = dot2_bf16(qc.w, kc.w, s1[h]);
          } else {
            s0[h] = fmaf(__uint_as_float(qc.x), __uint_as_float(kc.x), s0[h]);
            s1[h] = fmaf(__uint_as_float(qc.y), __uint_as_float(kc.y), s1[h]);
            s0[h] = fmaf(__uint_as_float(qc.z), __uint_as_float(kc.z), s0[h]);
            s1[h] = fmaf(__uint_as_float(qc.w), __uint_as_float(kc.w), s1[h]);
          }
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = ok_l ? (s0[h] + s1[h]) * a.scale_log2e : -INFINITY;
    }

    // online softmax update (per head, wave-uniform max)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float tmax = wave_max(s[h]);
      const float mn = fmaxf(m[h], tmax);
      const float alpha = fast_exp2(m[h] - mn);
      const float p = fast_exp2(s[h] - mn);
      l[h] = l[h] * alpha + p;
      sp[lane * G + h] = p;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
      m[h] = mn;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // P.V, split-D layout: this lane owns columns cl*EPL .. cl*EPL+EPL-1 of keys i*TPI+grp
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tok = i * TPI + grp;
      float pp[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pp[h] = sp[tok * G + h];
      float vf[EPL];
      if constexpr (BF) {
        vf[0] = bf16_lo(vr[i].x); vf[1] = bf16_hi(vr[i].x);
        vf[2] = bf16_lo(vr[i].y); vf[3] = bf16_hi(vr[i].y);
        vf[4] = bf16_lo(vr[i].z); vf[5] = bf16_hi(vr[i].z);
        vf[6] = bf16_lo(vr[i].w); vf[7] = bf16_hi(vr[i].w);
      } else {
        vf[0] = __uint_as_float(vr[i].x); vf[1] = __uint_as_float(vr[i].y);
        vf[2] = __uint_as_float(vr[i].z); vf[3] = __uint_as_float(vr[i].w);
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pp[h], vf[e], acc[h][e]);
    }
    __builtin_amdgcn_wave_barrier();
  }

  // wave totals: l over keys (lanes), acc over the TPI key groups
#pragma unroll
  for (int h = 0; h < G; ++h) l[h] = wave_sum(l[h]);
#pragma unroll
  for (int k = LPT; k < 64; k <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], k);

  if (bad) s_bad = 1;
  __syncthreads();  // every wave is done with its K tiles: reuse s_k as merge scratch
  float* mg_acc = reinterpret_cast<float*>(&s_k[0][0]);      // [4][G][D]
  float* mg_m = mg_acc + kDecodeWaves * G * D;                // [4][G]
  float* mg_l = mg_m + kDecodeWaves * G;                      // [4][G]
  if (lane < LPT) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) mg_acc[(wave * G + h) * D + lane * EPL + e] = acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mg_m[wave * G + h] = m[h];
      mg_l[wave * G + h] = l[h];
    }
  }
  __syncthreads();
  const bool bad_row = s_bad != 0;
  for (int idx = tid; idx < G * D; idx += 256) {
    const int h = idx / D;
    const int d = idx - h * D;
    float M = mg_m[h];
#pragma unroll
    for (int w = 1; w < kDecodeWaves; ++w) M = fmaxf(M, mg_m[w * G + h]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float fw = fast_exp2(mg_m[w * G + h] - M);
      num = fmaf(fw, mg_acc[(w * G + h) * D + d], num);
      den = fmaf(fw, mg_l[w * G + h], den);
    }
    if (bad_row) num = den = __builtin_nanf("");
    const int hq = g * G + h;
    if (it.part < 0) {
      a.out[(static_cast<int64_t>(it.row) * a.hq + hq) * D + d] = num / den;
    } else {
      const int64_t p = static_cast<int64_t>(it.part + it.split) * a.hq + hq;
      a.part_acc[p * D + d] = num;
      if (d == 0) {
        a.part_m[p] = M;
        a.part_l[p] = den;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Split merge: out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s, ascending s.
// One workgroup of D threads per (row, query head).
// ---------------------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(D) merge_kernel(MergeArgs a) {
  const int b = blockIdx.x;
  const int item = b / a.hq;
  const int h = b - item * a.hq;
  const int d = threadIdx.x;
  const MergeItem it = a.items[item];
  float M = -INFINITY;
  for (int s = 0; s < it.n_splits; ++s)
    M = fmaxf(M, a.part_m[static_cast<int64_t>(it.part + s) * a.hq + h]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < it.n_splits; ++s) {
    const int64_t p = static_cast<int64_t>(it.part + s) * a.hq + h;
    const float fw = fast_exp2(a.part_m[p] - M);
    num = fmaf(fw, a.part_acc[p * D + d], num);
    den = fmaf(fw, a.part_l[p], den);
  }
  a.out[(static_cast<int64_t>(it.row) * a.hq + h) * D + d] = num / den;
}

// ---------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------
bool decode_supported(int head_dim, int group) {
  return (head_dim == 64 || head_dim == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

template <int D, bool BF>
static hipError_t launch_decode_d(const DecodeArgs& a, uint32_t grid, int group,
                                  hipStream_t stream) {
  switch (group) {
    case 1: hipLaunchKernelGGL((decode_split_kernel<D, 1, BF>), dim3(grid), dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<D, 2, BF>), dim3(grid), dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_split_kernel<D, 4, BF>), dim3(grid), dim3(256), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((decode_split_kernel<D, 8, BF>), dim3(grid), dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int64_t n_items, int head_dim, int group,
                         bool bf16, hipStream_t stream) {
  const int64_t grid64 = n_items * a.hkv;
  if (grid64 == 0) return hipSuccess;
  if (grid64 > 0x7fffffffLL) return hipErrorInvalidValue;
  const uint32_t grid = static_cast<uint32_t>(grid64);
  if (head_dim == 64)
    return bf16 ? launch_decode_d<64, true>(a, grid, group, stream)
                : launch_decode_d<64, false>(a, grid, group, stream);
  if (head_dim == 128)
    return bf16 ? launch_decode_d<128, true>(a, grid, group, stream)
                : launch_decode_d<128, false>(a, grid, group, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const MergeArgs& a, int64_t n_items, int head_dim, hipStream_t stream) {
  const int64_t grid64 = n_items * a.hq;
  if (grid64 == 0) return hipSuccess;
  if (grid64 > 0x7fffffffLL) return hipErrorInvalidValue;
  const uint32_t grid = static_cast<uint32_t>(grid64);
  if (head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, dim3(grid), dim3(64), 0, stream, a);
  else if (head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3(grid), dim3(128), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
