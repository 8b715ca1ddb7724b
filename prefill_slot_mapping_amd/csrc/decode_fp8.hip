// Decode split pass over FP8 (OCP E4M3) pools for gfx950 (MI355X).
//
// Sources of the operation: "P3: native paged-KV continuous-batching sampler", section
// "Design > paged.py", TritonPagedAttention (a fixed KV split per context length, no atomics),
// and "Finish RL Training Faster: Bitwise-Consistent ..." section 2 (batch independence), with
// the KV cache stored as E4M3 codes and per-tensor scales (the consistency page's FP8 KV at
// about 57 % of the BF16 bytes).
//
// Numeric contract: the split, tile, wave and merge order of decode_split_kernel (tiles of HT
// keys aligned at the split start go to wave tile % 4; lazy per-head reference; wave partials
// merged in wave order, split partials in ascending split order). q is bfloat16. A K code is
// widened exactly to bfloat16 (every E4M3 value is a bfloat16 value) and multiplied by q with
// v_dot2_f32_bf16 (exact products, float32 sums over ascending 16-element chunks); the K
// scale is folded into the score scale. A V code is widened exactly to float32 for P.V and
// the V scale multiplies the accumulated numerator once, before the merge.
//
// Built with -fno-honor-nans like decode.hip: no floating-point operation sees a NaN; a row
// whose block table is bad is written as a NaN bit pattern through an integer select.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "kernels.h"
#include "lane_ops.h"

namespace pkv {

namespace {

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two E4M3 codes (bytes 0-1, or 2-3 with hi) of w -> a bfloat16 pair, exactly
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, bool hi) {
  return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                                         : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}

// two E4M3 codes -> two float32 values, exactly
__device__ __forceinline__ f32x2_t e4m3x2_to_f32x2(uint32_t w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_pk_f32_fp8(w, true) : __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
}

__device__ __forceinline__ uint2 load_nt8(const uint2* p) {
  typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(t.x, t.y);
}

}  // namespace

// ---------------------------------------------------------------------------------------
// Workgroup = 4 waves = one (query row, split, kv head) item serving the G query heads of the
// kv head. K rows (D bytes) are loaded 16 bytes per lane (LPTK lanes per row) and staged in
// LDS for the score stage (SPL lanes per key); V rows are loaded 8 bytes per lane (LPTV lanes
// per row), so that P.V keeps 8 accumulators per head per lane. A tile carries half the bytes
// of a bfloat16 tile, so each wave keeps NBUF - 1 tiles in flight in a register ring while it
// computes one (a tile's registers are few: 16 per 16 keys at head_dim 128).
// ---------------------------------------------------------------------------------------
template <int D, int G, int HT, int W, int NBUF>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(W, W)))
decode_fp8_kernel(DecodeArgs a) {
  constexpr int QROWB = D * 2;                // bytes of one bfloat16 q row
  constexpr int KROWB = D;                    // bytes of one E4M3 head row
  constexpr int LPTK = KROWB / 16;            // K load lanes per row
  constexpr int TPIK = 64 / LPTK;             // keys per K load instruction
  constexpr int NIK = HT / TPIK;              // K load instructions per tile
  constexpr int LPTV = KROWB / 8;             // V load lanes per row
  constexpr int TPIV = 64 / LPTV;             // keys per V load instruction (key groups)
  constexpr int NIV = HT / TPIV;              // V load instructions per tile
  constexpr int EPL = 8;                      // V elements per lane
  constexpr int SPL = 64 / HT;                // score stage: lanes per key
  constexpr int CPH = LPTK / SPL;             // score stage: K chunks per lane
  constexpr int GO = G >= SPL ? G / SPL : 1;  // heads whose p a lane forms
  constexpr float kRescaleLog2 = 8.f;
  static_assert(NIK >= 1 && NIV >= 1 && CPH >= 1 && HT % TPIK == 0 && HT % TPIV == 0, "shape");
  static_assert(HT == 16 || HT == 32, "tile");

  constexpr int kTileU4 = kDecodeWaves * HT * LPTK;
  constexpr int kMergeU4 = (kDecodeWaves * G * (D + 2) * 4 + 15) / 16;
  __shared__ uint4 s_k[kTileU4 > kMergeU4 ? kTileU4 : kMergeU4];
  __shared__ __align__(16) float s_p[kDecodeWaves][HT * G];
  __shared__ uint4 s_q[G * (QROWB / 16)];
  __shared__ uint32_t s_slot[kMaxDecodeSplit];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  // Items in grid order: the host lists them longest first and the hardware deals consecutive
  // workgroups to the 8 XCDs in turn, so every XCD gets its share of full and short splits.
  // (The heads of one item read disjoint cache lines, so keeping them on one XCD buys nothing.)
  const int f = blockIdx.x;
  const int item_idx = f / a.hkv;
  const int g = f - item_idx * a.hkv;
  const int hq0 = g * G;
  const DecodeItem it = a.items[item_idx];

  const int t0 = it.split * a.kv_split;
  const int t1 = min(it.n_keys, t0 + a.kv_split);
  const int nk = t1 - t0;
  const int nk_pad = (nk + HT - 1) / HT * HT;
  const int32_t* bt = a.block_tables + static_cast<int64_t>(it.seq) * a.max_blocks;
  bool bad = false;
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
    s_slot[k] = ok ? static_cast<uint32_t>(b * a.block_size + off) : 0u;
  }
  const uint4* qsrc = reinterpret_cast<const uint4*>(
      static_cast<const char*>(a.q) + (static_cast<int64_t>(it.row) * a.hq + hq0) * QROWB);
  for (int c = tid; c < G * (QROWB / 16); c += 256) s_q[c] = qsrc[c];
  __syncthreads();

  const int grpk = lane / LPTK, clk = lane & (LPTK - 1);
  const int grpv = lane / LPTV, clv = lane & (LPTV - 1);
  const int kk = lane / SPL, hf = lane % SPL;
  const uint32_t slot_bytes = static_cast<uint32_t>(a.hkv) * KROWB;
  const char* kbase = static_cast<const char*>(a.k_cache) + g * KROWB + clk * 16;
  const char* vbase = static_cast<const char*>(a.v_cache) + g * KROWB + clv * 8;
  uint4* sk = s_k + wave * HT * LPTK;
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

  auto load = [&](uint4 (&kr)[NIK], uint2 (&vr)[NIV], int hs) {
    const uint32_t* sl = s_slot + (hs - t0);
#pragma unroll
    for (int i = 0; i < NIK; ++i)
      kr[i] = load_nt(reinterpret_cast<const uint4*>(
          kbase + static_cast<uint64_t>(sl[i * TPIK + grpk]) * slot_bytes));
#pragma unroll
    for (int i = 0; i < NIV; ++i)
      vr[i] = load_nt8(reinterpret_cast<const uint2*>(
          vbase + static_cast<uint64_t>(sl[i * TPIV + grpv]) * slot_bytes));
  };

  auto compute = [&](const uint4 (&kr)[NIK], const uint2 (&vr)[NIV], int hs) {
    asm volatile("" ::: "memory");
    const int n = min(HT, t1 - hs);
#pragma unroll
    for (int i = 0; i < NIK; ++i) {
      const int tok = i * TPIK + grpk;
      sk[tok * LPTK + (clk ^ (tok & (LPTK - 1)))] = kr[i];
    }
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = 0.f;
#pragma unroll
    for (int u = 0; u < CPH; ++u) {
      const int c = hf * CPH + u;              // K chunk: elements 16 c .. 16 c + 15
      const uint4 kc = sk[kk * LPTK + (c ^ (kk & (LPTK - 1)))];
      const uint32_t kw[4] = {kc.x, kc.y, kc.z, kc.w};
      uint32_t kb[8];
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) {
        kb[2 * w2] = e4m3x2_to_bf16x2(kw[w2], false);
        kb[2 * w2 + 1] = e4m3x2_to_bf16x2(kw[w2], true);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint4 q0 = s_q[h * (QROWB / 16) + 2 * c];
        const uint4 q1 = s_q[h * (QROWB / 16) + 2 * c + 1];
        s[h] = dot2_bf16(q0.x, kb[0], s[h]);
        s[h] = dot2_bf16(q0.y, kb[1], s[h]);
        s[h] = dot2_bf16(q0.z, kb[2], s[h]);
        s[h] = dot2_bf16(q0.w, kb[3], s[h]);
        s[h] = dot2_bf16(q1.x, kb[4], s[h]);
        s[h] = dot2_bf16(q1.y, kb[5], s[h]);
        s[h] = dot2_bf16(q1.z, kb[6], s[h]);
        s[h] = dot2_bf16(q1.w, kb[7], s[h]);
      }
    }
    const bool valid = kk < n;
    bool over = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s[h] += dpp_xor1(s[h]);
      if constexpr (SPL == 4) s[h] += dpp_xor2(s[h]);
      s[h] = valid ? s[h] * a.scale_log2e : -INFINITY;
      over |= s[h] > m[h] + kRescaleLog2;
    }
    if (__any(over)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mt = max_over_groups<SPL>(s[h]);
        const float mn = mt > m[h] + kRescaleLog2 ? mt : m[h];
        const float al = fast_exp2(m[h] - mn);
        m[h] = mn;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= al;
        const int j = G >= SPL ? h / SPL : 0;
        lo[j] = hf == (G >= SPL ? h % SPL : h) ? lo[j] * al : lo[j];
      }
    }
#pragma unroll
    for (int j = 0; j < GO; ++j) {
      float sv = s[G >= SPL ? j * SPL : 0], mv = m[G >= SPL ? j * SPL : 0];
#pragma unroll
      for (int r = 1; r < (G >= SPL ? SPL : G); ++r) {
        sv = hf == r ? opaque(s[j * SPL + r]) : sv;
        mv = hf == r ? opaque(m[j * SPL + r]) : mv;
      }
      const float p = fast_exp2(sv - mv);
      lo[j] += p;
      if (G >= SPL || hf < G) sp[kk * G + j * SPL + hf] = p;
    }
#pragma unroll
    for (int i = 0; i < NIV; ++i) {
      const int tok = i * TPIV + grpv;
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
      const f32x2_t v0 = e4m3x2_to_f32x2(vr[i].x, false), v1 = e4m3x2_to_f32x2(vr[i].x, true);
      const f32x2_t v2 = e4m3x2_to_f32x2(vr[i].y, false), v3 = e4m3x2_to_f32x2(vr[i].y, true);
      const float vf[EPL] = {v0.x, v0.y, v1.x, v1.y, v2.x, v2.y, v3.x, v3.y};
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pp[h], vf[e], acc[h][e]);
    }
  };

  // tiles hs, hs + kStep, ... of this wave, ascending; tile i lives in ring buffer i % NBUF
  constexpr int kStep = kDecodeWaves * HT;
  uint4 kbuf[NBUF][NIK];
  uint2 vbuf[NBUF][NIV];
  int hs = t0 + wave * HT;
#pragma unroll
  for (int b = 0; b < NBUF - 1; ++b)
    if (hs + b * kStep < t1) load(kbuf[b], vbuf[b], hs + b * kStep);
  for (bool more = hs < t1; more;) {
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      const int cur = hs + b * kStep;
      if (more && cur < t1) {
        const int nxt = cur + (NBUF - 1) * kStep;
        if (nxt < t1) load(kbuf[(b + NBUF - 1) % NBUF], vbuf[(b + NBUF - 1) % NBUF], nxt);
        compute(kbuf[b], vbuf[b], cur);
      } else {
        more = false;
      }
    }
    hs += NBUF * kStep;
    more = more && hs < t1;
  }

#pragma unroll
  for (int j = 0; j < GO; ++j) lo[j] = sum_same_class<SPL>(lo[j]);
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = sum_key_groups<LPTV>(acc[h][e]);

  const bool bad_row = __syncthreads_or(bad) != 0;
  float* mg_acc = reinterpret_cast<float*>(s_k);             // [4][G][D]
  float* mg_m = mg_acc + kDecodeWaves * G * D;                // [4][G]
  float* mg_l = mg_m + kDecodeWaves * G;                      // [4][G]
  if (lane < LPTV) {
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
    num *= a.v_scale;
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

bool decode_fp8_supported(int head_dim, int group) {
  return (head_dim == 64 || head_dim == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

// Instances (keys per tile, waves-per-SIMD register budget, ring depth), measured on the
// batched 64-sequence step (groups of 4) and 32-sequence steps with groups of 1 and 2.
template <int D>
static hipError_t launch_fp8_d(const DecodeArgs& a, uint32_t grid, int group,
                               hipStream_t stream) {
  switch (group) {
    case 1: hipLaunchKernelGGL((decode_fp8_kernel<D, 1, 32, 3, 2>), dim3(grid), dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_fp8_kernel<D, 2, 32, 3, 2>), dim3(grid), dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_fp8_kernel<D, 4, 16, 4, 3>), dim3(grid), dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_fp8(const DecodeArgs& a, int64_t n_items, int head_dim, int group,
                             hipStream_t stream) {
  const int64_t grid64 = n_items * a.hkv;
  if (grid64 == 0) return hipSuccess;
  if (grid64 > 0x7fffffffLL || a.group != group) return hipErrorInvalidValue;
  const uint32_t grid = static_cast<uint32_t>(grid64);
  // groups of 8: the MFMA kernel (measured on the long-context E4M3 step: 143 us per decode
  // pass against 278 us for this kernel with 16-key tiles at two waves per SIMD)
  if (decode_mfma_supported(head_dim, group))
    return launch_decode_mfma(a, grid, head_dim, group, true, stream);
  if (head_dim == 64) return launch_fp8_d<64>(a, grid, group, stream);
  if (head_dim == 128) return launch_fp8_d<128>(a, grid, group, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
