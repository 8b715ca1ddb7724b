// Prefill-chunk attention on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Source of the operation: "P3: native paged-KV continuous-batching sampler", section
// "Design > paged.py" (TorchPagedAttention: each query row attends over exactly its own keys;
// a prefill chunk sees the prior context and its own earlier rows) and the mutant list of
// section "Evidence" (prefill causal mask off by one). The rows of a segment are the last
// q_len positions of its context; key j is visible to the row at position pos iff j <= pos.
//
// Work item: (prefill tile = up to 128 / G consecutive query rows of one segment, kv head g).
// The G query heads that read kv head g are packed with the rows into 128 "M-rows"
// (M-row = query row * G + head), 32 per wave. For each 64-key tile, aligned at absolute
// position 0 and visited in ascending order up to the tile holding the item's last row:
//   S^T[key][mrow] = K Q^T     16 MFMAs (2 key blocks x D/16 k-steps; K from LDS, Q in VGPRs)
//   masked online softmax per M-row in the base-2 domain (float32), one row per lane pair
//   O^T[d][mrow] += V^T P^T    P split into bf16 hi + lo parts (two MFMAs, ~16-bit P)
// K and V tiles are staged row-major in LDS with an XOR swizzle on 16-byte chunks; the V^T
// operand is read with ds_read_b64_tr_b16 (the hardware transpose read), so no transposed
// store is needed. Keys past the item's last row are not loaded (zero-filled, so 0 * V = 0);
// a tile that none of a wave's rows can see is skipped by that wave, which is bitwise the same
// as processing it (max unchanged, alpha = 1, p = 0). Hence a row's bits depend only on its
// own query, position and sequence K/V, never on how its segment was chunked or batched.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "kernels.h"

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// 16-byte chunk swizzle of a K/V row in LDS. For D = 128 (16 chunks): consecutive rows get
// distinct chunk offsets for the S^T operand reads (16 rows, one chunk each), and four rows
// starting at a multiple of four get distinct aligned chunk pairs for the transpose reads.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
  constexpr int H = CPR / 2;
  return ((row % H) << 1) | ((row / H) & 1);
}

template <int D, int G>
__global__ void __launch_bounds__(256) prefill_kernel(PrefillArgs a) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per head row
  constexpr int KS = D / 16;                 // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;                 // 32-wide d blocks of O^T
  constexpr int NLD = kPrefillKeyTile * CPR / 256;  // chunks per thread per tensor per tile
  static_assert(NLD >= 1, "tile must cover the workgroup");

  __shared__ uint4 s_k[kPrefillKeyTile * CPR];
  __shared__ uint4 s_v[kPrefillKeyTile * CPR];
  __shared__ int s_slot[2][kPrefillKeyTile];
  __shared__ int s_bad;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h32 = lane >> 5;
  const int f = xcd_remap(blockIdx.x, gridDim.x);
  const int g = f / a.n_items;
  const int item_idx = f - g * a.n_items;
  const PrefillItem it = a.items[item_idx];

  // this lane's M-row
  const int mr = wave * 32 + l32;
  const int qrow = mr / G;
  const int head = mr - qrow * G;
  const bool real = qrow < it.n_rows;
  const int pos = real ? it.pos0 + qrow : -1;
  const int wave_rows_lo = wave * 32 / G;
  const int wave_rows_hi = min(it.n_rows, (wave + 1) * 32 / G);
  const int wave_last_pos = wave_rows_hi > wave_rows_lo ? it.pos0 + wave_rows_hi - 1 : -1;

  // Q fragments (B operand of S^T = K Q^T): Q[mrow][16 ks + 8 h32 .. + 8]
  bf16x8_t qf[KS];
  {
    const uint4* qsrc = reinterpret_cast<const uint4*>(
        static_cast<const char*>(a.q) +
        ((static_cast<int64_t>(it.row0) + (real ? qrow : 0)) * a.hq +
         static_cast<int64_t>(g) * G + head) * (D * 2));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 v = real ? qsrc[2 * ks + h32] : make_uint4(0u, 0u, 0u, 0u);
      qf[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  const int key_limit = it.pos0 + it.n_rows;           // keys >= key_limit: no row needs them
  const int n_tiles = (key_limit + kPrefillKeyTile - 1) / kPrefillKeyTile;
  const int32_t* bt = a.block_tables + static_cast<int64_t>(it.seq) * a.max_blocks;
  const uint4* __restrict__ kp = static_cast<const uint4*>(a.k_cache);
  const uint4* __restrict__ vp = static_cast<const uint4*>(a.v_cache);
  const int64_t slot_stride = static_cast<int64_t>(a.hkv) * CPR;    // uint4 per slot
  const int head_off = g * CPR;
  bool bad = false;

  // slot of key (tile kt, key t) for t < 64, or -1 when not needed / not valid
  auto tile_slots = [&](int kt, int buf) {
    if (tid < kPrefillKeyTile) {
      const int kabs = kt * kPrefillKeyTile + tid;
      int slot = -1;
      if (kabs < key_limit) {
        int j, off;
        if (a.bs_log2 >= 0) {
          j = kabs >> a.bs_log2;
          off = kabs & (a.block_size - 1);
        } else {
          j = kabs / a.block_size;
          off = kabs - j * a.block_size;
        }
        const int b = bt[j];
        if (static_cast<unsigned>(b) < static_cast<unsigned>(a.num_blocks)) {
          slot = b * a.block_size + off;
        } else {
          bad = true;
        }
      }
      s_slot[buf][tid] = slot;
    }
  };

  uint4 kreg[NLD], vreg[NLD];
  auto load_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int ci = tid + 256 * i;
      const int key = ci / CPR;
      const int c = ci - key * CPR;
      const int slot = s_slot[buf][key];
      if (slot >= 0) {
        const int64_t off = static_cast<int64_t>(slot) * slot_stride + head_off + c;
        kreg[i] = kp[off];
        vreg[i] = vp[off];
      } else {
        kreg[i] = make_uint4(0u, 0u, 0u, 0u);
        vreg[i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };

  f32x16_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float sl2 = a.scale_log2e;

  if (tid == 0) s_bad = 0;
  tile_slots(0, 0);
  __syncthreads();
  load_tile(0);

  for (int kt = 0; kt < n_tiles; ++kt) {
    const int buf = kt & 1;
    __syncthreads();  // every wave is done with the previous tile's LDS
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int ci = tid + 256 * i;
      const int key = ci / CPR;
      const int c = ci - key * CPR;
      const int p = key * CPR + (c ^ swz<CPR>(key));
      s_k[p] = kreg[i];
      s_v[p] = vreg[i];
    }
    if (kt + 1 < n_tiles) tile_slots(kt + 1, buf ^ 1);
    __syncthreads();
    if (kt + 1 < n_tiles) load_tile(buf ^ 1);   // in flight while this tile is computed

    if (kt * kPrefillKeyTile > wave_last_pos) continue;  // no row of this wave sees this tile

    // ---- S^T = K Q^T: two 32-key blocks ----
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      const int row = kb * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 kv = s_k[row * CPR + ((2 * ks + h32) ^ swz<CPR>(row))];
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kv), qf[ks],
                                                        s[kb], 0, 0, 0);
      }
    }

    // ---- masked online softmax for this lane's M-row (keys split with lane ^ 32) ----
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kt * kPrefillKeyTile + kb * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3);
        const float v = key <= pos ? s[kb][r] * sl2 : -INFINITY;
        s[kb][r] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const bool live = m_new != -INFINITY;
    const float alpha = live ? fast_exp2(m_run - m_new) : 1.f;
    m_run = m_new;
    // Rescale only when some row's max moved: multiplying by exactly 1 is a no-op, so skipping
    // it when every alpha is 1 leaves every row's bits unchanged.
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    }

    // ---- O^T += V^T P^T per 16-key k-step (kb, m); the A operand (V^T) comes from two
    //      transpose reads, the B operand (P^T) is this lane's own probabilities ----
    const int grp16 = lane >> 4;          // 16-lane group: d half (grp16 & 1), key half (>> 1)
    const int i16 = lane & 15;
    const int rsub = i16 >> 2;            // row this lane addresses inside a 4-row read
    const int csub = 4 * (i16 & 3);       // element column offset inside the 16-wide d strip
    __attribute__((address_space(3))) char* vbase =
        (__attribute__((address_space(3))) char*)(s_v);
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        bf16x8_t phi, plo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p = live ? fast_exp2(s[kb][8 * m + j] - m_new) : 0.f;
          psum += p;
          const __bf16 ph = static_cast<__bf16>(p);
          phi[j] = ph;
          plo[j] = static_cast<__bf16>(p - static_cast<float>(ph));
        }
        const int r0 = kb * 32 + 16 * m + 4 * (grp16 >> 1) + rsub;   // slots 0..3
        const int r1 = r0 + 8;                                        // slots 4..7
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int dcol = 32 * db + 16 * (grp16 & 1) + csub;
          const int cchunk = dcol >> 3;
          const int cin = dcol & 7;
          lds_s16x4_t* p0 =
              (lds_s16x4_t*)(vbase + (r0 * CPR + (cchunk ^ swz<CPR>(r0))) * 16 + cin * 2);
          lds_s16x4_t* p1 =
              (lds_s16x4_t*)(vbase + (r1 * CPR + (cchunk ^ swz<CPR>(r1))) * 16 + cin * 2);
          const s16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p0);
          const s16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p1);
          const s16x4_t tt[2] = {t0, t1};
          const bf16x8_t va = __builtin_bit_cast(bf16x8_t, tt);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, phi, acc[db], 0, 0, 0);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, plo, acc[db], 0, 0, 0);
        }
      }
    l_run = l_run * alpha + psum;
  }

  if (bad) s_bad = 1;
  __syncthreads();
  const bool bad_item = s_bad != 0;
  if (!real) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  float* dst = a.out + ((static_cast<int64_t>(it.row0) + qrow) * a.hq +
                        static_cast<int64_t>(g) * G + head) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      float4 o;
      o.x = acc[db][4 * rq + 0] / l_tot;
      o.y = acc[db][4 * rq + 1] / l_tot;
      o.z = acc[db][4 * rq + 2] / l_tot;
      o.w = acc[db][4 * rq + 3] / l_tot;
      if (bad_item) o = make_float4(__builtin_nanf(""), __builtin_nanf(""),
                                    __builtin_nanf(""), __builtin_nanf(""));
      *reinterpret_cast<float4*>(dst + 32 * db + 8 * rq + 4 * h32) = o;
    }
}

bool prefill_supported(int head_dim, int group, bool bf16) {
  return bf16 && (head_dim == 64 || head_dim == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

template <int D>
static hipError_t launch_prefill_d(const PrefillArgs& a, uint32_t grid, int group,
                                   hipStream_t stream) {
  switch (group) {
    case 1: hipLaunchKernelGGL((prefill_kernel<D, 1>), dim3(grid), dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<D, 2>), dim3(grid), dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<D, 4>), dim3(grid), dim3(256), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<D, 8>), dim3(grid), dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, int64_t n_items, int head_dim, int group,
                          hipStream_t stream) {
  const int64_t grid64 = n_items * a.hkv;
  if (grid64 == 0) return hipSuccess;
  if (grid64 > 0x7fffffffLL || n_items != a.n_items) return hipErrorInvalidValue;
  const uint32_t grid = static_cast<uint32_t>(grid64);
  if (head_dim == 64) return launch_prefill_d<64>(a, grid, group, stream);
  if (head_dim == 128) return launch_prefill_d<128>(a, grid, group, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
