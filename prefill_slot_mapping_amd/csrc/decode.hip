// Decode split pass for gfx950 (MI355X).
//
// Sources of the operation: "P3: native paged-KV continuous-batching sampler", section
// "Design > paged.py", TritonPagedAttention (q, k/v cache blocks, block tables, cu_seqlens_q,
// ctx_lens; a fixed KV split per context length, no atomics), and "Finish RL Training Faster:
// Bitwise-Consistent ..." section 2 (kernel determinism, batch independence).
//
// Numeric contract (every choice depends only on the row's own sequence and the kernel
// instance, which is fixed by head_dim, group size and element type, never by the batch):
// the keys of a row are cut into splits of kv_split tokens aligned at position 0; inside a
// split, tiles of HT keys (16 or 32, per instance) aligned at the split start go to wave
// (tile % 4); each wave runs an online softmax over its tiles in ascending order in the base-2
// domain (scores scaled by scale * log2 e, hardware exp2) whose per-head reference moves to
// the tile maximum only when a score exceeds it by more than 8; the four wave partials are
// merged in wave order and the split partials in ascending split order (merge kernel). Accumulation
// is float32 throughout; bfloat16 products are formed exactly by v_dot2_f32_bf16 and summed
// over the head dimension in ascending 16-byte chunks, one part of the dimension per lane of a
// key's lane group, the parts then added in a fixed butterfly; probabilities stay float32 for
// P.V. bf16 groups of 8 run on the MFMA kernel of decode_mfma.hip instead, whose contract is
// fixed per instance in the same way.
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
// Decode split pass.
//
// Workgroup = 4 waves = one (query row, split, kv head) item serving all G query heads of
// that kv head, so every K/V byte of the split is loaded from HBM once. W waves of this kernel
// share a SIMD (register budget 512 / W per lane).
// Prologue: the split's slots (one block-table read per key; keys past the split end repeat
// the last key, whose probability is forced to 0) and the G query rows go to LDS. The slots
// are stored transposed per half tile so that a lane's slots are contiguous.
// The split is cut into HT-key tiles aligned at the split start; tile j belongs to wave j % 4.
// Each wave double-buffers its tiles in registers: the loads of the next tile are in flight
// while the current one is computed. Per tile a wave
//   1. has loaded K and V rows with coalesced 16-byte nontemporal loads (LPT lanes cover one
//      head row),
//   2. stages K in LDS (XOR swizzle on 16-byte chunks) and computes the scores with SPL =
//      64 / HT lanes per key (each covers D / SPL; DPP exchanges complete the dot product),
//   3. updates the per-head running max (wave-uniform) and publishes p through LDS (lane
//      h % SPL of each key's group forms p for head h),
//   4. accumulates P.V in the split-D layout (each lane owns EPL columns of its key group).
// ---------------------------------------------------------------------------------------
// R > 1: a group item (DecodeGroupItem) of up to R rows whose split reads the same physical
// blocks. The split's K and V tiles are loaded once; each row keeps its own running state
// (reference, sums, accumulators) and its own wave merge, and runs exactly the operations of
// the R = 1 kernel on every tile in the same order, so its bits do not depend on the rows it
// was grouped with. The slots come from the first row's table; a row whose table names other
// blocks over the split (the host planned from tables that differ from the device's) is
// written as NaN instead of reading the first row's keys.
template <int D, int G, bool BF, int HT, int W, int R = 1>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(W, W)))
decode_split_kernel(DecodeArgs a) {
  constexpr int E = BF ? 2 : 4;
  constexpr int ROWB = D * E;               // bytes of one head row
  constexpr int LPT = ROWB / 16;            // lanes per key row
  constexpr int TPI = 64 / LPT;             // keys per load instruction (key groups)
  constexpr int NI = HT / TPI;              // load instructions per tile and tensor
  constexpr int EPL = 16 / E;               // elements per lane chunk
  constexpr int SPL = 64 / HT;              // score stage: lanes per key (2 or 4)
  constexpr int CPH = LPT / SPL;            // score stage: chunks per lane
  constexpr int GO = G >= SPL ? G / SPL : 1;  // heads whose p a lane forms
  constexpr float kRescaleLog2 = 8.f;       // lazy rescale threshold (log2 units)
  // groups of 8 keep the running maximum (the lazy reference's extra live registers would
  // spill at two waves per SIMD)
  constexpr bool kLazy = G < 8;
  static_assert(LPT >= 8 && LPT <= 32 && (LPT & (LPT - 1)) == 0 && HT % TPI == 0, "shape");
  static_assert(HT == 16 || HT == 32, "tile");
  static_assert(NI % 2 == 0, "slot reads are 8- or 16-byte vectors");
  static_assert(R >= 1 && R <= kGroupRows, "rows per item");

  // K tiles of the four waves; reused as the wave-merge scratch at the end
  constexpr int kTileU4 = kDecodeWaves * HT * LPT;
  constexpr int kMergeU4 = (kDecodeWaves * G * (D + 2) * 4 + 15) / 16;
  __shared__ uint4 s_k[kTileU4 > kMergeU4 ? kTileU4 : kMergeU4];
  __shared__ __align__(16) float s_p[kDecodeWaves][HT * G];
  __shared__ uint4 s_q[R][G * LPT];
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
  int split, n_keys, n_rows;
  int row[R], seq[R], part[R];
  if constexpr (R == 1) {
    const DecodeItem it = a.items[item_idx];
    split = it.split;
    n_keys = it.n_keys;
    n_rows = 1;
    row[0] = it.row;
    seq[0] = it.seq;
    part[0] = it.part;
  } else {
    const DecodeGroupItem it = a.groups[item_idx];
    split = it.split;
    n_keys = it.n_keys;
    n_rows = it.n_rows;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      row[r] = it.row[r];
      seq[r] = it.seq[r];
      part[r] = it.part[r];
    }
  }

  const int t0 = split * a.kv_split;
  const int t1 = min(n_keys, t0 + a.kv_split);
  const int nk = t1 - t0;                    // >= 1
  const int nk_pad = (nk + HT - 1) / HT * HT;
  const int32_t* bt = a.block_tables + static_cast<int64_t>(seq[0]) * a.max_blocks;
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
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r >= n_rows) break;
    const uint4* qsrc = reinterpret_cast<const uint4*>(
        static_cast<const char*>(a.q) + (static_cast<int64_t>(row[r]) * a.hq + hq0) * ROWB);
    for (int c = tid; c < G * LPT; c += 256) s_q[r][c] = qsrc[c];
  }
  // rows after the first must name the same blocks over the split
  bool row_bad[R];
  row_bad[0] = false;
  if constexpr (R > 1) {
    const int j0 = a.bs_log2 >= 0 ? t0 >> a.bs_log2 : t0 / a.block_size;
    const int j1 = a.bs_log2 >= 0 ? (t1 - 1) >> a.bs_log2 : (t1 - 1) / a.block_size;
#pragma unroll
    for (int r = 1; r < R; ++r) {
      bool mis = false;
      if (r < n_rows) {
        const int32_t* btr = a.block_tables + static_cast<int64_t>(seq[r]) * a.max_blocks;
        for (int j = j0 + tid; j <= j1; j += 256) mis |= btr[j] != bt[j];
      }
      row_bad[r] = __syncthreads_or(mis) != 0;
    }
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

  float m[R][G], lo[R][GO], acc[R][G][EPL];
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[r][h] = -INFINITY;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[r][h][e] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < GO; ++j) lo[r][j] = 0.f;
  }

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

  // one row's scores, softmax and P.V on the tile staged in sk (K) and vr (V)
  auto row_tile = [&](const uint4 (&vr)[NI], int hs, int r) {
    // The lanes exchange p through sp (each lane reads values other lanes wrote). The compiler
    // barrier makes every row reload them: without it a lane that writes no p for a head (group
    // sizes below SPL) could be handed the previous row's values it read from the same slots.
    asm volatile("" ::: "memory");
    const int n = min(HT, t1 - hs);
    const uint4* sq = s_q[r];
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
        const uint4 qc = sq[h * LPT + c];
        if constexpr (BF) {
          s[h] = dot2_bf16(qc.x, kc.x, s[h]);
          s[h] = dot2_bf16(qc.y, kc.y, s[h]);
          s[h] = dot2_bf16(qc.z, kc.z, s[h]);
          s[h] = dot2_bf16(qc.w, kc.w, s[h]);
        } else {
          s[h] = fmaf(__uint_as_float(qc.x), __uint_as_float(kc.x), s[h]);
          s[h] = fmaf(__uint_as_float(qc.y), __uint_as_float(kc.y), s[h]);
          s[h] = fmaf(__uint_as_float(qc.z), __uint_as_float(kc.z), s[h]);
          s[h] = fmaf(__uint_as_float(qc.w), __uint_as_float(kc.w), s[h]);
        }
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
      for (int h = 0; h < G; ++h) over |= s[h] > m[r][h] + kRescaleLog2;
      if (__any(over)) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float mt = max_over_groups<SPL>(s[h]);
          const float mn = mt > m[r][h] + kRescaleLog2 ? mt : m[r][h];
          const float al = fast_exp2(m[r][h] - mn);  // exactly 1 for a head that keeps m
          m[r][h] = mn;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[r][h][e] *= al;
          const int j = G >= SPL ? h / SPL : 0;
          lo[r][j] = hf == (G >= SPL ? h % SPL : h) ? lo[r][j] * al : lo[r][j];
        }
      }
    } else {
      // m is the running maximum; the accumulators are rescaled when some head's maximum
      // moved (multiplying by exactly 1 changes nothing)
      bool moved = false;
      float alpha[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(m[r][h], max_over_groups<SPL>(s[h]));
        alpha[h] = fast_exp2(m[r][h] - mn);
        moved |= alpha[h] != 1.f;
        m[r][h] = mn;
      }
#pragma unroll
      for (int j = 0; j < GO; ++j) {
        float av = alpha[G >= SPL ? j * SPL : 0];
#pragma unroll
        for (int q = 1; q < (G >= SPL ? SPL : G); ++q)
          av = hf == q ? opaque(alpha[j * SPL + q]) : av;
        lo[r][j] *= av;
      }
      if (__any(moved)) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[r][h][e] *= alpha[h];
      }
    }
    // p of (key kk, head h) is formed by the lane of that key with hf == h % SPL (heads
    // below SPL: by the lanes hf < G, the others idle)
#pragma unroll
    for (int j = 0; j < GO; ++j) {
      float sv = s[G >= SPL ? j * SPL : 0], mv = m[r][G >= SPL ? j * SPL : 0];
#pragma unroll
      for (int q = 1; q < (G >= SPL ? SPL : G); ++q) {
        sv = hf == q ? opaque(s[j * SPL + q]) : sv;
        mv = hf == q ? opaque(m[r][j * SPL + q]) : mv;
      }
      const float p = fast_exp2(sv - mv);
      lo[r][j] += p;
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
        for (int e = 0; e < EPL; ++e) acc[r][h][e] = fmaf(pp[h], vf[e], acc[r][h][e]);
    }
  };

  auto compute = [&](const uint4 (&kr)[NI], const uint4 (&vr)[NI], int hs) {
    // q chunks are re-read from LDS in every tile: holding them in registers across the loop
    // would cost more registers than the K/V buffers
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tok = i * TPI + grp;
      sk[tok * LPT + (cl ^ (tok & (LPT - 1)))] = kr[i];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r >= n_rows) break;
      row_tile(vr, hs, r);
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

  const bool bad_blk = __syncthreads_or(bad) != 0;  // also: every wave is done with s_k
  float* mg_acc = reinterpret_cast<float*>(s_k);             // [4][G][D]
  float* mg_m = mg_acc + kDecodeWaves * G * D;                // [4][G]
  float* mg_l = mg_m + kDecodeWaves * G;                      // [4][G]
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r >= n_rows) break;
    if (r > 0) __syncthreads();   // the previous row's merge has read the scratch
    // wave totals: l over the lanes that formed it, acc over the TPI key groups
#pragma unroll
    for (int j = 0; j < GO; ++j) lo[r][j] = sum_same_class<SPL>(lo[r][j]);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[r][h][e] = sum_key_groups<LPT>(acc[r][h][e]);
    if (lane < LPT) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) mg_acc[(wave * G + h) * D + lane * EPL + e] = acc[r][h][e];
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) mg_m[wave * G + h] = m[r][h];
    }
    if (lane < (G >= SPL ? SPL : G)) {
#pragma unroll
      for (int j = 0; j < GO; ++j) mg_l[wave * G + j * SPL + lane] = lo[r][j];
    }
    __syncthreads();
    const bool bad_row = bad_blk || row_bad[r];
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
      if (part[r] < 0) {
        const float o = num / den;
        a.out[(static_cast<int64_t>(row[r]) * a.hq + hq) * D + d] =
            __uint_as_float(bad_row ? nan_bits : __float_as_uint(o));
      } else {
        const int64_t p = static_cast<int64_t>(part[r] + split) * a.hq + hq;
        a.part_acc[p * D + d] = __uint_as_float(bad_row ? nan_bits : __float_as_uint(num));
        if (d == 0) {
          a.part_m[p] = M;
          a.part_l[p] = __uint_as_float(bad_row ? nan_bits : __float_as_uint(den));
        }
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

// Keys per tile and waves per SIMD of each decode_split_kernel instance (measured on the
// batched, long-context and prefix-shared decode steps): bf16 groups of 4 run 16-key tiles at
// three waves per SIMD (160 registers at head_dim 128); other bf16 instances run 32-key tiles
// at two waves; float32 (twice the bytes per row) one wave. bf16 groups of 8 run on the MFMA
// kernel (decode_mfma.hip): on the long-context step 245 us per decode pass against 256 us for
// the paired-wave kernel this file held before (one wave of a pair loading K, the other V,
// each computing 4 of the 8 heads), and 161 against 221 us for this kernel at head_dim 64.
template <int D, bool BF, int G>
constexpr int tile_keys() {
  return (BF && D == 128 && G >= 4) ? 16 : (BF && D == 64 && G == 4) ? 16 : 32;
}
template <int D, bool BF, int G>
constexpr int waves_per_simd() {
  return !BF ? 1 : (G == 4 ? 3 : 2);
}
template <int D, bool BF, int G>
static hipError_t launch_one(const DecodeArgs& a, uint32_t grid, hipStream_t stream) {
  if constexpr (BF && G == 8) {
    return launch_decode_mfma(a, grid, D, G, false, stream);
  } else {
    hipLaunchKernelGGL((decode_split_kernel<D, G, BF, tile_keys<D, BF, G>(), waves_per_simd<D, BF, G>()>),
                       dim3(grid), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
}
template <int D, bool BF>
static hipError_t launch_decode_d(const DecodeArgs& a, uint32_t grid, int group,
                                  hipStream_t stream) {
  switch (group) {
    case 1: return launch_one<D, BF, 1>(a, grid, stream);
    case 2: return launch_one<D, BF, 2>(a, grid, stream);
    case 4: return launch_one<D, BF, 4>(a, grid, stream);
    case 8: return launch_one<D, BF, 8>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

// Group items: bf16 groups up to 4, the single-row kernel with the state of kGroupR rows at
// kGroupW waves per SIMD (measured on the prefix-shared step: 2 rows at two waves per SIMD
// 151 us per decode pass beside the per-row launch; 4 rows at one wave 183 us; wider row
// sets spill at two waves).
constexpr int kGroupR = 2;
constexpr int kGroupW = 2;
bool decode_groups_supported(int head_dim, int group) {
  return (head_dim == 64 || head_dim == 128) && (group == 1 || group == 2 || group == 4);
}
int decode_group_rows() { return kGroupR; }

template <int D, int G>
static void launch_group_one(const DecodeArgs& a, uint32_t grid, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_kernel<D, G, true, tile_keys<D, true, G>(), kGroupW, kGroupR>),
                     dim3(grid), dim3(256), 0, stream, a);
}

hipError_t launch_decode_groups(const DecodeArgs& a, int64_t n_groups, int head_dim, int group,
                                hipStream_t stream) {
  const int64_t grid64 = n_groups * a.hkv;
  if (grid64 == 0) return hipSuccess;
  if (grid64 > 0x7fffffffLL || a.group != group || !decode_groups_supported(head_dim, group))
    return hipErrorInvalidValue;
  const uint32_t grid = static_cast<uint32_t>(grid64);
  switch (group * 1000 + head_dim) {
    case 1064: launch_group_one<64, 1>(a, grid, stream); break;
    case 2064: launch_group_one<64, 2>(a, grid, stream); break;
    case 4064: launch_group_one<64, 4>(a, grid, stream); break;
    case 1128: launch_group_one<128, 1>(a, grid, stream); break;
    case 2128: launch_group_one<128, 2>(a, grid, stream); break;
    case 4128: launch_group_one<128, 4>(a, grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int64_t n_items, int head_dim, int group,
                         bool bf16, hipStream_t stream) {
  const int64_t grid64 = n_items * a.hkv;
  if (grid64 == 0) return hipSuccess;
  if (grid64 > 0x7fffffffLL || a.group != group) return hipErrorInvalidValue;
  const uint32_t grid = static_cast<uint32_t>(grid64);
  if (head_dim == 64)
    return bf16 ? launch_decode_d<64, true>(a, grid, group, stream)
                : launch_decode_d<64, false>(a, grid, group, stream);
  if (head_dim == 128)
    return bf16 ? launch_decode_d<128, true>(a, grid, group, stream)
                : launch_decode_d<128, false>(a, grid, group, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
