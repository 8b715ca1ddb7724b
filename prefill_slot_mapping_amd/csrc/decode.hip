// Decode split pass for gfx950 (MI355X): the dispatch of every pool type, and the vector kernel
// of float32 pools. bf16 and E4M3 pools run on the MFMA kernel of decode_mfma.hip.
//
// Sources of the operation: "P3: native paged-KV continuous-batching sampler", section
// "Design > paged.py", TritonPagedAttention (q, k/v cache blocks, block tables, cu_seqlens_q,
// ctx_lens; a fixed KV split per context length, no atomics), and "Finish RL Training Faster:
// Bitwise-Consistent ..." section 2 (kernel determinism, batch independence).
//
// Numeric contract of the float32 kernel (every choice depends only on the row's own sequence
// and the kernel instance, which is fixed by head_dim and group size, never by the batch): the
// keys of a row are cut into splits of kv_split tokens aligned at position 0; inside a split,
// tiles of 32 keys aligned at the split start go to wave (tile % 4); each wave runs an online
// softmax over its tiles in ascending order in the base-2 domain (scores scaled by
// scale * log2 e, hardware exp2) whose per-head reference moves to the tile maximum only when
// a score exceeds it by more than 8 (groups below 8; groups of 8 keep the running maximum);
// the four wave partials are merged in wave order and the split partials in ascending split
// order (merge kernel). Products and sums are float32 FMAs over the head dimension in
// ascending 16-byte chunks, one part of the dimension per lane of a key's lane pair, the two
// parts then added; probabilities stay float32 for P.V.
//
// This file is compiled with -fno-honor-nans (lets maxima fuse with their lane permutes): no
// floating-point operation here sees a NaN; a row whose block table is bad is written as a NaN
// bit pattern through an integer select.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "kernels.h"
#include "lane_ops.h"

namespace pkv {

// ---------------------------------------------------------------------------------------
// Decode split pass over float32 pools.
//
// Workgroup = 4 waves = one (query row, split, kv head) item serving all G query heads of
// that kv head, so every K/V byte of the split is loaded from HBM once; one wave per SIMD.
// Prologue: the split's slots (one block-table read per key; keys past the split end repeat
// the last key, whose probability is forced to 0) and the G query rows go to LDS. The slots
// are stored transposed per tile so that a lane's slots are contiguous.
// The split is cut into HT-key tiles aligned at the split start; tile j belongs to wave j % 4.
// Each wave double-buffers its tiles in registers: the loads of the next tile are in flight
// while the current one is computed. Per tile a wave
//   1. has loaded K and V rows with coalesced 16-byte nontemporal loads (LPT lanes cover one
//      head row),
//   2. stages K in LDS (XOR swizzle on 16-byte chunks) and computes the scores with SPL =
//      64 / HT lanes per key (each covers D / SPL; a DPP exchange completes the dot product),
//   3. updates the per-head reference (wave-uniform) and publishes p through LDS (lane
//      h % SPL of each key's group forms p for head h),
//   4. accumulates P.V in the split-D layout (each lane owns EPL columns of its key group).
// ---------------------------------------------------------------------------------------
template <int D, int G, int HT, int W>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(W, W)))
decode_f32_kernel(DecodeArgs a) {
  constexpr int ROWB = D * 4;               // bytes of one head row
  constexpr int LPT = ROWB / 16;            // lanes per key row
  constexpr int TPI = 64 / LPT;             // keys per load instruction (key groups)
  constexpr int NI = HT / TPI;              // load instructions per tile and tensor
  constexpr int EPL = 4;                    // elements per lane chunk
  constexpr int SPL = 64 / HT;              // score stage: lanes per key (2 or 4)
  constexpr int CPH = LPT / SPL;            // score stage: chunks per lane
  constexpr int GO = G >= SPL ? G / SPL : 1;  // heads whose p a lane forms
  constexpr float kRescaleLog2 = 8.f;       // lazy rescale threshold (log2 units)
  // groups of 8 keep the running maximum (the lazy reference's extra live registers would
  // not fit)
  constexpr bool kLazy = G < 8;
  static_assert(LPT >= 8 && LPT <= 32 && (LPT & (LPT - 1)) == 0 && HT % TPI == 0, "shape");
  static_assert(HT == 16 || HT == 32, "tile");
  static_assert(NI % 2 == 0, "slot reads are 8- or 16-byte vectors");

  // K tiles of the four waves; reused as the wave-merge scratch at the end
  constexpr int kTileU4 = kDecodeWaves * HT * LPT;
  constexpr int kMergeU4 = (kDecodeWaves * G * (D + 2) * 4 + 15) / 16;
  __shared__ uint4 s_k[kTileU4 > kMergeU4 ? kTileU4 : kMergeU4];
  __shared__ __align__(16) float s_p[kDecodeWaves][HT * G];
  __shared__ uint4 s_q[G * LPT];
  __shared__ __align__(16) uint32_t s_slot[kMaxDecodeSplit];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  // Items in grid order: the host lists them longest first and the hardware deals consecutive
  // workgroups to the 8 XCDs in turn, so every XCD gets its share of full and short splits
  // (contiguous per-XCD ranges of that list would leave the XCD holding the short ones idle).
  const int f = blockIdx.x;
  const int item_idx = f / a.hkv;
  const int g = f - item_idx * a.hkv;        // the kv head of this work item
  const int hq0 = g * G;                     // its first query head
  const DecodeItem it = a.items[item_idx];

  const int t0 = it.split * a.kv_split;
  const int t1 = min(it.n_keys, t0 + a.kv_split);
  const int nk = t1 - t0;                    // >= 1
  const int nk_pad = (nk + HT - 1) / HT * HT;
  const int32_t* bt = a.block_tables + static_cast<int64_t>(it.seq) * a.max_blocks;
  bool bad = false;

  // an out-of-pool block id marks the item bad and is replaced by slot 0, so no load ever
  // leaves the pool
  for (int k = tid; k < nk_pad; k += 256) {
    const int pos = t0 + min(k, nk - 1);
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
    const int w = k % HT;
    s_slot[(k - w) + (w % TPI) * NI + w / TPI] = ok ? static_cast<uint32_t>(b * a.block_size + off) : 0u;
  }
  {
    const uint4* qsrc = reinterpret_cast<const uint4*>(
        static_cast<const char*>(a.q) + (static_cast<int64_t>(it.row) * a.hq + hq0) * ROWB);
    for (int c = tid; c < G * LPT; c += 256) s_q[c] = qsrc[c];
  }
  __syncthreads();

  const int grp = lane / LPT;               // P.V stage / loads: key group of this lane
  const int cl = lane & (LPT - 1);          // P.V stage / loads: chunk of this lane
  const int kk = lane / SPL;                // score stage: key of this lane
  const int hf = lane % SPL;                // score stage: part of D of this lane
  const uint32_t slot_bytes = static_cast<uint32_t>(a.hkv) * ROWB;  // < 2^32 for any head count
  const char* kbase = static_cast<const char*>(a.k_cache) + g * ROWB + cl * 16;
  const char* vbase = static_cast<const char*>(a.v_cache) + g * ROWB + cl * 16;
  uint4* sk = s_k + wave * HT * LPT;
  float* sp = s_p[wave];

  float m[G], lo[GO], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < GO; ++j) lo[j] = 0.f;

  auto load = [&](uint4 (&kr)[NI], uint4 (&vr)[NI], int hs) {
    const uint32_t* sl = s_slot + (hs - t0) + grp * NI;
    constexpr int SV = NI % 4 == 0 ? 4 : 2;
#pragma unroll
    for (int i4 = 0; i4 < NI; i4 += SV) {
      uint32_t ss[4];
      if constexpr (SV == 4) {
        const uint4 s4 = *reinterpret_cast<const uint4*>(sl + i4);
        ss[0] = s4.x; ss[1] = s4.y; ss[2] = s4.z; ss[3] = s4.w;
      } else {
        const uint2 s2 = *reinterpret_cast<const uint2*>(sl + i4);
        ss[0] = s2.x; ss[1] = s2.y;
      }
#pragma unroll
      for (int u = 0; u < SV; ++u) {
        const uint64_t off = static_cast<uint64_t>(ss[u]) * slot_bytes;
        kr[i4 + u] = load_nt(reinterpret_cast<const uint4*>(kbase + off));
        vr[i4 + u] = load_nt(reinterpret_cast<const uint4*>(vbase + off));
      }
    }
  };

  // scores, softmax and P.V of the tile staged in sk (K) and vr (V)
  auto compute = [&](const uint4 (&kr)[NI], const uint4 (&vr)[NI], int hs) {
    // the lanes exchange K and p through LDS (each lane reads values other lanes wrote)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tok = i * TPI + grp;
      sk[tok * LPT + (cl ^ (tok & (LPT - 1)))] = kr[i];
    }
    asm volatile("" ::: "memory");
    const int n = min(HT, t1 - hs);
    // scores: lanes SPL k .. SPL k + SPL - 1 hold parts of key k's dot products
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
        s[h] = fmaf(__uint_as_float(qc.x), __uint_as_float(kc.x), s[h]);
        s[h] = fmaf(__uint_as_float(qc.y), __uint_as_float(kc.y), s[h]);
        s[h] = fmaf(__uint_as_float(qc.z), __uint_as_float(kc.z), s[h]);
        s[h] = fmaf(__uint_as_float(qc.w), __uint_as_float(kc.w), s[h]);
      }
    }
    const bool valid = kk < n;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s[h] += dpp_xor1(s[h]);
      if constexpr (SPL == 4) s[h] += dpp_xor2(s[h]);
      s[h] = valid ? s[h] * a.scale_log2e : -INFINITY;
    }
    if constexpr (kLazy) {
      // A head's reference m moves only when one of its scores rises more than kRescaleLog2
      // above it (then to the tile maximum): p = exp2(s - m) stays below 2^kRescaleLog2, and
      // tiles that do not move it skip the wave maxima and the accumulator rescale.
      bool over = false;
#pragma unroll
      for (int h = 0; h < G; ++h) over |= s[h] > m[h] + kRescaleLog2;
      if (__any(over)) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float mt = max_over_groups<SPL>(s[h]);
          const float mn = mt > m[h] + kRescaleLog2 ? mt : m[h];
          const float al = fast_exp2(m[h] - mn);  // exactly 1 for a head that keeps m
          m[h] = mn;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] *= al;
          const int j = G >= SPL ? h / SPL : 0;
          lo[j] = hf == (G >= SPL ? h % SPL : h) ? lo[j] * al : lo[j];
        }
      }
    } else {
      // m is the running maximum; the accumulators are rescaled when some head's maximum
      // moved (multiplying by exactly 1 changes nothing)
      bool moved = false;
      float alpha[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(m[h], max_over_groups<SPL>(s[h]));
        alpha[h] = fast_exp2(m[h] - mn);
        moved |= alpha[h] != 1.f;
        m[h] = mn;
      }
#pragma unroll
      for (int j = 0; j < GO; ++j) {
        float av = alpha[G >= SPL ? j * SPL : 0];
#pragma unroll
        for (int q = 1; q < (G >= SPL ? SPL : G); ++q)
          av = hf == q ? opaque(alpha[j * SPL + q]) : av;
        lo[j] *= av;
      }
      if (__any(moved)) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha[h];
      }
    }
    // p of (key kk, head h) is formed by the lane of that key with hf == h % SPL (heads
    // below SPL: by the lanes hf < G, the others idle)
#pragma unroll
    for (int j = 0; j < GO; ++j) {
      float sv = s[G >= SPL ? j * SPL : 0], mv = m[G >= SPL ? j * SPL : 0];
#pragma unroll
      for (int q = 1; q < (G >= SPL ? SPL : G); ++q) {
        sv = hf == q ? opaque(s[j * SPL + q]) : sv;
        mv = hf == q ? opaque(m[j * SPL + q]) : mv;
      }
      const float p = fast_exp2(sv - mv);
      lo[j] += p;
      if (G >= SPL || hf < G) sp[kk * G + j * SPL + hf] = p;
    }
    // P.V, split-D layout: this lane owns columns cl*EPL .. +EPL of keys i*TPI + grp
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tok = i * TPI + grp;
      float pp[G];
      if constexpr (G >= 4) {
#pragma unroll
        for (int h4 = 0; h4 < G; h4 += 4) {
          const float4 t = *reinterpret_cast<const float4*>(sp + tok * G + h4);
          pp[h4] = t.x; pp[h4 + 1] = t.y; pp[h4 + 2] = t.z; pp[h4 + 3] = t.w;
        }
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) pp[h] = sp[tok * G + h];
      }
      const float vf[EPL] = {__uint_as_float(vr[i].x), __uint_as_float(vr[i].y),
                             __uint_as_float(vr[i].z), __uint_as_float(vr[i].w)};
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pp[h], vf[e], acc[h][e]);
    }
  };

  // this wave's tiles: hs = t0 + HT * (wave + 4 j), j = 0, 1, ...
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

  const bool bad_row = __syncthreads_or(bad) != 0;  // also: every wave is done with s_k
  float* mg_acc = reinterpret_cast<float*>(s_k);             // [4][G][D]
  float* mg_m = mg_acc + kDecodeWaves * G * D;                // [4][G]
  float* mg_l = mg_m + kDecodeWaves * G;                      // [4][G]
  // wave totals: l over the lanes that formed it, acc over the TPI key groups
#pragma unroll
  for (int j = 0; j < GO; ++j) lo[j] = sum_same_class<SPL>(lo[j]);
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = sum_key_groups<LPT>(acc[h][e]);
  if (lane < LPT) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) mg_acc[(wave * G + h) * D + lane * EPL + e] = acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) mg_m[wave * G + h] = m[h];
  }
  if (lane < (G >= SPL ? SPL : G)) {
#pragma unroll
    for (int j = 0; j < GO; ++j) mg_l[wave * G + j * SPL + lane] = lo[j];
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
    const uint32_t nan_bits = 0x7fc00000u;
    const int hq = hq0 + h;
    if (it.part < 0) {
      const float o = num / den;
      a.out[(static_cast<int64_t>(it.row) * a.hq + hq) * D + d] =
          __uint_as_float(bad_row ? nan_bits : __float_as_uint(o));
    } else {
      const int64_t p = static_cast<int64_t>(it.part + it.split) * a.hq + hq;
      a.part_acc[p * D + d] = __uint_as_float(bad_row ? nan_bits : __float_as_uint(num));
      if (d == 0) {
        a.part_m[p] = M;
        a.part_l[p] = __uint_as_float(bad_row ? nan_bits : __float_as_uint(den));
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------
bool decode_supported(int head_dim, int group) {
  return (head_dim == 64 || head_dim == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

// float32 pools: 32-key tiles at one wave per SIMD (a row is twice the bytes of bf16).
template <int D>
static hipError_t launch_f32_d(const DecodeArgs& a, uint32_t grid, int group,
                               hipStream_t stream) {
  switch (group) {
    case 1: hipLaunchKernelGGL((decode_f32_kernel<D, 1, 32, 1>), dim3(grid), dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_f32_kernel<D, 2, 32, 1>), dim3(grid), dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_f32_kernel<D, 4, 32, 1>), dim3(grid), dim3(256), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((decode_f32_kernel<D, 8, 32, 1>), dim3(grid), dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Group items (bf16 and E4M3 pools): the MFMA kernel with the rows of an item in its columns.
bool decode_groups_supported(int head_dim, int group) {
  return decode_mfma_supported(head_dim, group);
}
int decode_group_rows(int group) { return decode_mfma_group_rows(group); }

hipError_t launch_decode_groups(const DecodeArgs& a, int64_t n_groups, int head_dim, int group,
                                bool fp8, hipStream_t stream) {
  const int64_t grid64 = n_groups * a.hkv;
  if (grid64 == 0) return hipSuccess;
  if (grid64 > 0x7fffffffLL || a.group != group || !decode_groups_supported(head_dim, group))
    return hipErrorInvalidValue;
  return launch_decode_mfma(a, static_cast<uint32_t>(grid64), head_dim, group, fp8, true, stream);
}

hipError_t launch_decode(const DecodeArgs& a, int64_t n_items, int head_dim, int group,
                         bool bf16, hipStream_t stream) {
  const int64_t grid64 = n_items * a.hkv;
  if (grid64 == 0) return hipSuccess;
  if (grid64 > 0x7fffffffLL || a.group != group || !decode_supported(head_dim, group))
    return hipErrorInvalidValue;
  const uint32_t grid = static_cast<uint32_t>(grid64);
  if (bf16) return launch_decode_mfma(a, grid, head_dim, group, false, false, stream);
  return head_dim == 64 ? launch_f32_d<64>(a, grid, group, stream)
                        : launch_f32_d<128>(a, grid, group, stream);
}

bool decode_fp8_supported(int head_dim, int group) { return decode_mfma_supported(head_dim, group); }

hipError_t launch_decode_fp8(const DecodeArgs& a, int64_t n_items, int head_dim, int group,
                             hipStream_t stream) {
  const int64_t grid64 = n_items * a.hkv;
  if (grid64 == 0) return hipSuccess;
  if (grid64 > 0x7fffffffLL || a.group != group || !decode_fp8_supported(head_dim, group))
    return hipErrorInvalidValue;
  return launch_decode_mfma(a, static_cast<uint32_t>(grid64), head_dim, group, true, false, stream);
}

}  // namespace pkv
