// Decode split pass for gfx950 (MI355X).
//
// Sources of the operation: "P3: native paged-KV continuous-batching sampler", section
// "Design > paged.py", TritonPagedAttention (q, k/v cache blocks, block tables, cu_seqlens_q,
// ctx_lens; a fixed KV split per context length, no atomics), and "Finish RL Training Faster:
// Bitwise-Consistent ..." section 2 (kernel determinism, batch independence).
//
// Numeric contract (every choice depends only on the row's own sequence, never on the batch):
// the keys of a row are cut into splits of kv_split tokens aligned at position 0; inside a
// split, 32-key half tiles aligned at the split start go to wave (half tile % 4); each wave
// runs an online softmax over its half tiles in ascending order in the base-2 domain (scores
// scaled by scale * log2 e, hardware exp2); the four wave partials are merged in wave order and
// the split partials in ascending split order (merge kernel). Accumulation is float32
// throughout; bfloat16 products are formed exactly by v_dot2_f32_bf16; probabilities stay
// float32 for P.V.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "kernels.h"

namespace pkv {

// ---------------------------------------------------------------------------------------
// Decode split pass.
//
// Workgroup = 4 waves = one (query row, split, kv head) item; it serves the G query heads that
// read that kv head, so every K/V byte of the split is loaded from HBM once.
// Prologue: the split's slots (one block-table read per key) and the G query rows go to LDS.
// The split is cut into 32-key half tiles aligned at the split start; half tile j belongs to
// wave j % 4. Each wave double-buffers its half tiles in registers: the loads of the next
// half tile are in flight while the current one is computed. Per half tile a wave
//   1. has loaded K and V rows with coalesced 16-byte nontemporal loads (LPT lanes cover one
//      head row; keys past the split end re-read the last key, whose p is 0),
//   2. stages K in LDS (XOR swizzle on 16-byte chunks) and computes the scores with two lanes
//      per key (each covers half of D; one DPP exchange completes the dot product),
//   3. updates the per-head running max (wave-uniform) and publishes p through LDS,
//   4. accumulates P.V in the split-D layout (each lane owns EPL columns of its key group).
// ---------------------------------------------------------------------------------------
template <int D, int G, bool BF>
__global__ void __launch_bounds__(256) decode_split_kernel(DecodeArgs a) {
  // G = query heads served by one work item: all heads of a kv head when the group has at
  // most 4 of them, else 4 consecutive heads (two items of a larger group share a kv head and
  // read its K/V through the same XCD's L2)
  constexpr int E = BF ? 2 : 4;
  constexpr int ROWB = D * E;               // bytes of one head row
  constexpr int LPT = ROWB / 16;            // lanes per key row
  constexpr int TPI = 64 / LPT;             // keys per load instruction
  constexpr int HT = kDecodeTile / 2;       // keys per half tile
  constexpr int NI = HT / TPI;              // load instructions per half tile and tensor
  constexpr int EPL = 16 / E;               // elements per lane chunk
  constexpr int CPH = LPT / 2;              // chunks per lane in the score stage
  static_assert(LPT >= 2 && LPT <= 32 && (LPT & (LPT - 1)) == 0 && HT % TPI == 0, "shape");

  __shared__ uint4 s_k[kDecodeWaves][HT * LPT];
  __shared__ float s_p[kDecodeWaves][HT * G];
  __shared__ uint4 s_q[G * LPT];
  __shared__ int s_slot[kMaxDecodeSplit];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int f = xcd_remap(blockIdx.x, gridDim.x);
  const int subs = a.hq / G;                 // work items per (row, split)
  const int item_idx = f / subs;
  const int hq0 = (f - item_idx * subs) * G; // first query head of this work item
  const int g = hq0 / a.group;               // the kv head those heads read
  const DecodeItem it = a.items[item_idx];

  const int t0 = it.split * a.kv_split;
  const int t1 = min(it.n_keys, t0 + a.kv_split);
  const int32_t* bt = a.block_tables + static_cast<int64_t>(it.seq) * a.max_blocks;
  bool bad = false;

  // an out-of-pool block id marks the item bad and is replaced by slot 0, so no load ever
  // leaves the pool
  for (int k = tid; k < t1 - t0; k += 256) {
    const int pos = t0 + k;
    int j, off;
    if (a.bs_log2 >= 0) {
      j = pos >> a.bs_log2;
      off = pos & (a.block_size - 1);
    } else {
      j = pos / a.block_size;
      off = pos - j * a.block_size;
    }
    const int b = bt[j];
    const bool ok = static_cast<unsigned>(b) < static_cast<unsigned>(a.num_blocks);
    bad |= !ok;
    s_slot[k] = ok ? b * a.block_size + off : 0;
  }
  const uint4* qsrc = reinterpret_cast<const uint4*>(
      static_cast<const char*>(a.q) + (static_cast<int64_t>(it.row) * a.hq + hq0) * ROWB);
  for (int c = tid; c < G * LPT; c += 256) s_q[c] = qsrc[c];
  __syncthreads();

  const uint4* __restrict__ kp = static_cast<const uint4*>(a.k_cache);
  const uint4* __restrict__ vp = static_cast<const uint4*>(a.v_cache);
  const int64_t slot_stride = static_cast<int64_t>(a.hkv) * LPT;  // uint4 per slot
  const int head_off = g * LPT;
  const int grp = lane / LPT;               // P.V stage / loads: key group of this lane
  const int cl = lane & (LPT - 1);          // P.V stage / loads: chunk of this lane
  const int kk = lane >> 1;                 // score stage: key of this lane
  const int hf = lane & 1;                  // score stage: half of D of this lane
  uint4* sk = s_k[wave];
  float* sp = s_p[wave];

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  auto load = [&](uint4 (&kr)[NI], uint4 (&vr)[NI], int hs) {
    const int n = min(HT, t1 - hs);
    const int* slots = s_slot + (hs - t0);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tok = min(i * TPI + grp, n - 1);
      const int64_t off = static_cast<int64_t>(slots[tok]) * slot_stride + head_off + cl;
      kr[i] = load_nt(kp + off);
      vr[i] = load_nt(vp + off);
    }
  };

  auto compute = [&](const uint4 (&kr)[NI], const uint4 (&vr)[NI], int hs) {
    const int n = min(HT, t1 - hs);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tok = i * TPI + grp;
      sk[tok * LPT + (cl ^ (tok & (LPT - 1)))] = kr[i];
    }
    // scores: lanes 2k and 2k+1 hold halves of key k's dot products
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = 0.f;
#pragma unroll
    for (int u = 0; u < CPH; ++u) {
      const int c = hf * CPH + u;
      const uint4 kc = sk[kk * LPT + (c ^ (kk & (LPT - 1)))];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint4 qc = s_q[h * LPT + c];
        if constexpr (BF) {
          float t = dot2_bf16(qc.x, kc.x, 0.f);
          t = dot2_bf16(qc.y, kc.y, t);
          t = dot2_bf16(qc.z, kc.z, t);
          t = dot2_bf16(qc.w, kc.w, t);
          s[h] += t;
        } else {
          float t = __uint_as_float(qc.x) * __uint_as_float(kc.x);
          t = fmaf(__uint_as_float(qc.y), __uint_as_float(kc.y), t);
          t = fmaf(__uint_as_float(qc.z), __uint_as_float(kc.z), t);
          t = fmaf(__uint_as_float(qc.w), __uint_as_float(kc.w), t);
          s[h] += t;
        }
      }
    }
    const bool valid = kk < n;
    bool moved = false;
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s[h] += dpp_xor1(s[h]);
      s[h] = valid ? s[h] * a.scale_log2e : -INFINITY;
      const float mn = fmaxf(m[h], wave_max_pairs(s[h]));
      alpha[h] = fast_exp2(m[h] - mn);
      moved |= alpha[h] != 1.f;
      m[h] = mn;
    }
    // p of (key kk, head h) is formed by the lane of that key with hf == h % 2
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if ((h & 1) == hf) {
        const float p = fast_exp2(s[h] - m[h]);
        l[h] = l[h] * alpha[h] + p;
        sp[kk * G + h] = p;
      }
    }
    // rescale only when some head's max moved (multiplying by exactly 1 changes nothing)
    if (__any(moved)) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha[h];
    }
    // P.V, split-D layout: this lane owns columns cl*EPL .. +EPL of keys i*TPI + grp
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
  };

  // this wave's half tiles: hs = t0 + HT * (wave + 4 j), j = 0, 1, ...
  constexpr int kStep = kDecodeWaves * HT;
  uint4 ka[NI], va[NI], kb[NI], vb[NI];
  int hs = t0 + wave * HT;
  if (hs < t1) load(ka, va, hs);
  while (hs < t1) {
    const int hs1 = hs + kStep;
    if (hs1 < t1) load(kb, vb, hs1);
    compute(ka, va, hs);
    if (hs1 >= t1) break;
    const int hs2 = hs1 + kStep;
    if (hs2 < t1) load(ka, va, hs2);
    compute(kb, vb, hs1);
    hs = hs2;
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

  const bool bad_row = __syncthreads_or(bad) != 0;  // also: every wave is done with s_k
  float* mg_acc = reinterpret_cast<float*>(&s_k[0][0]);      // [4][G][D]
  float* mg_m = mg_acc + kDecodeWaves * G * D;                // [4][G]
  float* mg_l = mg_m + kDecodeWaves * G;                      // [4][G]
  static_assert(sizeof(s_k) >= sizeof(float) * kDecodeWaves * G * (D + 2), "merge scratch");
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
    const int hq = hq0 + h;
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
// launcher
// ---------------------------------------------------------------------------------------
bool decode_supported(int head_dim, int group) {
  return (head_dim == 64 || head_dim == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

// query heads per decode work item
static int decode_heads_per_item(int group) { return group < 4 ? group : 4; }

template <int D, bool BF>
static hipError_t launch_decode_d(const DecodeArgs& a, uint32_t grid, int gi,
                                  hipStream_t stream) {
  switch (gi) {
    case 1: hipLaunchKernelGGL((decode_split_kernel<D, 1, BF>), dim3(grid), dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<D, 2, BF>), dim3(grid), dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_split_kernel<D, 4, BF>), dim3(grid), dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int64_t n_items, int head_dim, int group,
                         bool bf16, hipStream_t stream) {
  const int gi = decode_heads_per_item(group);
  const int64_t grid64 = n_items * (a.hq / gi);
  if (grid64 == 0) return hipSuccess;
  if (grid64 > 0x7fffffffLL || a.group != group) return hipErrorInvalidValue;
  const uint32_t grid = static_cast<uint32_t>(grid64);
  if (head_dim == 64)
    return bf16 ? launch_decode_d<64, true>(a, grid, gi, stream)
                : launch_decode_d<64, false>(a, grid, gi, stream);
  if (head_dim == 128)
    return bf16 ? launch_decode_d<128, true>(a, grid, gi, stream)
                : launch_decode_d<128, false>(a, grid, gi, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
