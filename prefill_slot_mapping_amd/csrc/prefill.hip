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
//   O^T[d][mrow] += V^T P^T    P split into bf16 hi + lo parts (two MFMAs, ~16-bit P): hi is
//                              p with its low 16 bits cleared, lo the exact remainder rounded
// K and V tiles are staged row-major in LDS with an XOR swizzle on 16-byte chunks; the V^T
// operand is read with ds_read_b64_tr_b16 (the hardware transpose read), so no transposed
// store is needed. Keys past the item's last row are not loaded (zero-filled, so 0 * V = 0);
// a tile that none of a wave's rows can see is skipped by that wave, which is bitwise the same
// as processing it (max unchanged, alpha = 1, p = 0). Hence a row's bits depend only on its
// own query, position and sequence K/V, never on how its segment was chunked or batched.
//
// E4M3 pools (the F8 instances; "Finish RL Training Faster: Bitwise-Consistent ...", section
// 4.2, FP8 KV storage with one read path): a tile's codes (half the bytes) are copied global ->
// LDS into a double-buffered staging area, then every wave widens its share of them exactly
// to bfloat16 into the one bf16 tile buffer the MFMA operand reads use (every E4M3 value is a
// bfloat16 value). The K scale is folded into the score scale by the host; the V scale
// multiplies each output once. Everything else, and so the numeric contract, is as above.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "lane_ops.h"

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef unsigned u32x4v_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4v_t lds_u32x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;

// x through an empty register-to-register asm: values derived from it inside a loop are
// recomputed there instead of being held as loop invariants
__device__ __forceinline__ uint32_t opaque_u32(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// 16-byte chunk swizzle of a K/V row in LDS. For D = 128 (16 chunks): consecutive rows get
// distinct chunk offsets for the S^T operand reads (16 rows, one chunk each), and four rows
// starting at a multiple of four get distinct aligned chunk pairs for the transpose reads.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
  constexpr int H = CPR / 2;
  return ((row % H) << 1) | ((row / H) & 1);
}

// 16 bytes per lane from global memory straight into LDS at lds_base + lane * 16 (M0 holds the
// wave-uniform LDS byte address). Issued through inline assembly so that the compiler does not
// track these LDS writes (it would otherwise wait for every outstanding tile load before each
// LDS read that might alias); completion is awaited explicitly in tile_barrier().
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds_base) : "memory", "m0");
}

// As dma16, from the wave-uniform base address sbase plus this lane's 32-bit byte offset voff.
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_base) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p))));
}

// Every tile DMA and LDS access of this wave has completed, then the workgroup meets.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16 E4M3 codes -> 16 bfloat16 values (two 16-byte chunks), exactly
__device__ __forceinline__ void e4m3x16_to_bf16(uint4 c, uint4& lo, uint4& hi) {
  auto pk = [](uint32_t w, bool h) {
    return __builtin_bit_cast(uint32_t, h ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                                          : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  };
  lo = make_uint4(pk(c.x, false), pk(c.x, true), pk(c.y, false), pk(c.y, true));
  hi = make_uint4(pk(c.z, false), pk(c.z, true), pk(c.w, false), pk(c.w, true));
}

// The LDS writes of this wave have completed, then the workgroup meets (tile DMAs in flight
// stay in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D, int G, bool F8>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_kernel(PrefillArgs a) {
  constexpr int CPR = D / 8;                 // 16-byte bf16 chunks per head row
  constexpr int KS = D / 16;                 // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;                 // 32-wide d blocks of O^T
  constexpr int TC = kPrefillKeyTile * CPR;  // chunks per tile and tensor
  constexpr int NJ = TC / 256;               // DMA instructions per wave per tensor per tile
  constexpr int CPC = D / 16;                // 16-byte code chunks per E4M3 head row
  constexpr int TCC = kPrefillKeyTile * CPC; // code chunks per tile and tensor
  constexpr int NJC = TCC / 256;             // code DMA instructions per wave per tensor
  static_assert(NJ >= 1 && TC % 256 == 0, "tile must cover the workgroup");
  static_assert(!F8 || (NJC >= 1 && TCC % 256 == 0), "code tile must cover the workgroup");

  // [buffer][tensor: 0 = K, 1 = V][chunk]: tile kt lives in buffer kt % 2 (bf16 pools), or in
  // the one buffer after its codes are widened (E4M3 pools: codes of tile kt in s_code[kt % 2])
  constexpr int NBK = F8 ? 1 : 2;
  __shared__ uint4 s_kv[NBK][2][TC];
  __shared__ uint4 s_code[F8 ? 2 : 1][2][F8 ? TCC : 1];
  // a window of the sequence's block-table entries (validated), starting at entry win0
  __shared__ int s_blk[kPrefillBlockWindow];
  __shared__ int s_bad;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  // padding M-rows (past the item's rows) behave like the last row with a zero query: finite
  // values, never written
  const int pos = real ? it.pos0 + qrow : it.pos0 + it.n_rows - 1;
  const int wave_rows_lo = wave * 32 / G;
  const int wave_rows_hi = min(it.n_rows, (wave + 1) * 32 / G);
  const int wave_last_pos = wave_rows_hi > wave_rows_lo ? it.pos0 + wave_rows_hi - 1 : -1;
  const int wave_first_pos = it.pos0 + wave_rows_lo;   // every real row of the wave sees keys <= this
  constexpr float kRescaleSlack = 8.f;

  // Q fragments (B operand of S^T = K Q^T): Q[mrow][16 ks + 8 h32 .. + 8]
  bf16x8_t qf[KS];
  {
    const uint4* qsrc = reinterpret_cast<const uint4*>(
        static_cast<const char*>(a.q) +
        ((static_cast<int64_t>(it.row0) + (real ? qrow : 0)) * a.hq +
         static_cast<int64_t>(g) * G + head) * (D * 2));
    const uint32_t sign = a.negate_q ? 0x80008000u : 0u;   // scale < 0: fold its sign into q
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = real ? qsrc[2 * ks + h32] : make_uint4(0u, 0u, 0u, 0u);
      v.x ^= sign;
      v.y ^= sign;
      v.z ^= sign;
      v.w ^= sign;
      qf[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  const int key_limit = it.pos0 + it.n_rows;           // keys >= key_limit: no row needs them
  // this item's keys: [kv0, kv_end), tiles kt0 .. n_tiles - 1 (a split is a whole number of tiles)
  const int kv0 = a.tile_split > 0 ? it.split * a.tile_split : 0;
  const int kv_end = a.tile_split > 0
      ? static_cast<int>(min(static_cast<int64_t>(kv0) + a.tile_split, static_cast<int64_t>(key_limit)))
      : key_limit;
  const int kt0 = kv0 / kPrefillKeyTile;
  const int n_tiles = (kv_end + kPrefillKeyTile - 1) / kPrefillKeyTile;
  const int32_t* bt = a.block_tables + static_cast<int64_t>(it.seq) * a.max_blocks;
  const uint4* __restrict__ kp = static_cast<const uint4*>(a.k_cache);
  const uint4* __restrict__ vp = static_cast<const uint4*>(a.v_cache);
  const uint32_t slot_stride = static_cast<uint32_t>(a.hkv * CPR);  // uint4 per slot
  const int head_off = g * CPR;
  bool bad = false;

  auto entry_of = [&](int key) { return a.bs_log2 >= 0 ? key >> a.bs_log2 : key / a.block_size; };
  const int n_entries = entry_of(key_limit - 1) + 1;
  int win0 = entry_of(kv0);

  // Block-table entries win0 .. win0 + window - 1 into s_blk. An out-of-pool block id marks the
  // item bad and is replaced by block 0, so no load ever leaves the pool.
  auto load_window = [&]() {
    const int n = min(kPrefillBlockWindow, n_entries - win0);
    for (int i = tid; i < n; i += 256) {
      const int b = bt[win0 + i];
      const bool ok = static_cast<unsigned>(b) < static_cast<unsigned>(a.num_blocks);
      bad |= !ok;
      s_blk[i] = ok ? b : 0;
    }
  };

  // K and V of tile kt into LDS buffer buf. Chunk position P holds chunk (P % CPR) ^ swz(row)
  // of key row P / CPR, so the swizzled layout comes from the source addresses. Keys no row
  // needs re-read the item's last key (finite data whose p is exactly 0).
  // E4M3 codes of tile kt into staging buffer buf, row-major (code chunk P = chunk P % CPC of
  // key row P / CPC); keys no row needs re-read the item's last key.
  const uint32_t stride_c = static_cast<uint32_t>(a.hkv * CPC);  // code chunks per slot
  uint32_t lane_off_c[F8 ? NJC : 1];
  if constexpr (F8) {
    static_assert(NJC * 64 / CPC == 16, "a wave copies 16 keys of a tile");
#pragma unroll
    for (int j = 0; j < NJC; ++j)
      lane_off_c[j] = (static_cast<uint32_t>((j * 64 + lane) / CPC) * stride_c + g * CPC +
                       lane % CPC) * 16u;
  }
  auto dma_codes = [&](int kt, int buf) {
    const uint4* __restrict__ kc = static_cast<const uint4*>(a.k_cache);
    const uint4* __restrict__ vc = static_cast<const uint4*>(a.v_cache);
    const int key0 = kt * kPrefillKeyTile + wave * 16;
    if (a.bs_log2 >= 4 && key0 + 15 <= key_limit - 1) {   // as in dma_tile
      const int e = key0 >> a.bs_log2;
      const int blk = __builtin_amdgcn_readfirstlane(s_blk[e - win0]);
      const uint32_t slot0 = static_cast<uint32_t>(blk) * a.block_size + (key0 - (e << a.bs_log2));
      const uint64_t base = static_cast<uint64_t>(slot0) * stride_c;
#pragma unroll
      for (int j = 0; j < NJC; ++j) {
        const int cb = (wave * NJC + j) * 64;
        dma16_s(kc + base, lane_off_c[j], lds_addr(&s_code[buf][0][cb]));
        dma16_s(vc + base, lane_off_c[j], lds_addr(&s_code[buf][1][cb]));
      }
      return;
    }
    uint64_t off[NJC];
#pragma unroll
    for (int j = 0; j < NJC; ++j) {
      const int P = (wave * NJC + j) * 64 + lane;
      const int row = P / CPC;
      const int key = min(kt * kPrefillKeyTile + row, key_limit - 1);
      const int e = entry_of(key);
      const int in_blk = key - e * a.block_size;
      const uint32_t slot = static_cast<uint32_t>(s_blk[e - win0] * a.block_size + in_blk);
      off[j] = static_cast<uint64_t>(slot) * stride_c + g * CPC + (P % CPC);
    }
#pragma unroll
    for (int j = 0; j < NJC; ++j) {
      const int base = (wave * NJC + j) * 64;
      dma16(kc + off[j], lds_addr(&s_code[buf][0][base]));
      dma16(vc + off[j], lds_addr(&s_code[buf][1][base]));
    }
  };

  // codes of staging buffer buf -> bfloat16 in the swizzled layout of s_kv[0], all waves
  auto widen = [&](int buf) {
#pragma unroll
    for (int j = 0; j < NJC; ++j) {
      const int P = (wave * NJC + j) * 64 + lane;
      const int row = P / CPC;
      const int c = P % CPC;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        uint4 lo, hi;
        e4m3x16_to_bf16(s_code[buf][t][P], lo, hi);
        s_kv[0][t][row * CPR + ((2 * c) ^ swz<CPR>(row))] = lo;
        s_kv[0][t][row * CPR + ((2 * c + 1) ^ swz<CPR>(row))] = hi;
      }
    }
  };

  // Each wave copies 16 consecutive keys of a tile (NJ * 64 / CPR rows). With blocks of at
  // least 16 keys (a power of two) those keys are consecutive slots of one block: one
  // block-table lookup per tile, a wave-uniform base address and per-lane offsets fixed for the
  // whole item (chunk position P of the wave's rows, swizzled as below).
  static_assert(NJ * 64 / CPR == 16, "a wave copies 16 keys of a tile");
  uint32_t lane_off[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int r = (j * 64 + lane) / CPR;          // key row within the wave's 16
    const int row = wave * 16 + r;
    lane_off[j] = (static_cast<uint32_t>(r) * slot_stride + head_off +
                   ((lane % CPR) ^ swz<CPR>(row))) * 16u;
  }
  const bool one_block_rows = a.bs_log2 >= 4;
  auto dma_tile = [&](int kt, int buf) {
    const int key0 = kt * kPrefillKeyTile + wave * 16;
    if (one_block_rows && key0 + 15 <= key_limit - 1) {
      const int e = key0 >> a.bs_log2;
      const int blk = __builtin_amdgcn_readfirstlane(s_blk[e - win0]);
      const uint32_t slot0 = static_cast<uint32_t>(blk) * a.block_size + (key0 - (e << a.bs_log2));
      const uint64_t base = static_cast<uint64_t>(slot0) * slot_stride;
      const uint4* kb = kp + base;
      const uint4* vb = vp + base;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int cb = (wave * NJ + j) * 64;
        dma16_s(kb, lane_off[j], lds_addr(&s_kv[buf][0][cb]));
        dma16_s(vb, lane_off[j], lds_addr(&s_kv[buf][1][cb]));
      }
      return;
    }
    uint64_t off[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int P = (wave * NJ + j) * 64 + lane;
      const int row = P / CPR;
      const int key = min(kt * kPrefillKeyTile + row, key_limit - 1);
      const int e = entry_of(key);
      const int in_blk = key - e * a.block_size;
      const uint32_t slot = static_cast<uint32_t>(s_blk[e - win0] * a.block_size + in_blk);
      off[j] = static_cast<uint64_t>(slot) * slot_stride + head_off + ((P % CPR) ^ swz<CPR>(row));
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int base = (wave * NJ + j) * 64;
      dma16(kp + off[j], lds_addr(&s_kv[buf][0][base]));
      dma16(vp + off[j], lds_addr(&s_kv[buf][1][base]));
    }
  };

  f32x16_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m_ref = -INFINITY;
  float l_run = 0.f;
  const float sl2 = a.scale_log2e;   // |scale| * log2(e)

  // Fixed parts of this lane's LDS operand addresses (tile rows are swizzled by swz).
  // S^T operand: key row l32 (+ 32 kb), chunk (2 ks + h32) ^ swz(l32) (swz(l32 + 32 kb) is
  // swz(l32)), at byte k_base + ((32 ks) ^ k_x0).
  const uint32_t k_sw = swz<CPR>(l32);
  const uint32_t k_base = static_cast<uint32_t>(l32 * CPR * 16) + 16u * (h32 ^ (k_sw & 1u));
  const uint32_t k_x0 = 16u * (k_sw & ~1u);
  // V^T operand of k-step q, d block db: this lane reads 4 elements at column
  // 32 db + 16 (grp16 & 1) + csub of key row 16 q + r (slots 0..3, r = 4 (grp16 >> 1) + rsub)
  // and of key row 16 q + r + 8 (slots 4..7); the chunk of row 16 q + r is swizzled by swz(r).
  // The byte offset is 16 q CPR 16 + v_base + ((64 db) ^ v_y).
  const int grp16 = lane >> 4;          // 16-lane group: d half (grp16 & 1), key half (>> 1)
  const int i16 = lane & 15;
  const int rsub = i16 >> 2;            // row this lane addresses inside a 4-row read
  const int csub = 4 * (i16 & 3);       // element column offset inside the 16-wide d strip
  const uint32_t vr0 = 4 * (grp16 >> 1) + rsub;
  const uint32_t vc0 = 2 * (grp16 & 1) + (csub >> 3);   // chunk of the strip in d block 0
  const uint32_t v_sw0 = swz<CPR>(vr0), v_sw1 = swz<CPR>(vr0 + 8);
  const uint32_t v_base0 = vr0 * CPR * 16 + 16u * (vc0 ^ (v_sw0 & 3u)) + 2u * (csub & 7);
  const uint32_t v_base1 = (vr0 + 8) * CPR * 16 + 16u * (vc0 ^ (v_sw1 & 3u)) + 2u * (csub & 7);
  const uint32_t v_y0_ = 16u * (v_sw0 & ~3u), v_y1_ = 16u * (v_sw1 & ~3u);

  if (tid == 0) s_bad = 0;
  load_window();
  __syncthreads();
  if constexpr (F8) dma_codes(kt0, 0);
  else dma_tile(kt0, 0);

  // Tiles kt0 .. kd - 1 cross no row of this wave (each of its rows sees every key of them)
  // and take the unmasked form; tiles kd .. n_tiles - 1 take the masked form (on a tile that
  // crosses none of the wave's rows the mask keeps every key of a used row, so masking there
  // changes no value). Padding M-rows compute finite values that are never written. Each form
  // has a loop of its own (register allocation of one form does not burden the other); both
  // meet the same workgroup barriers per tile.
  const int kd = min(max((wave_first_pos + 1) / kPrefillKeyTile, kt0), n_tiles);
  auto tile_step = [&](int kt, auto masked_tag) {
    const int par = (kt - kt0) & 1;   // tile kt in buffer par (E4M3: its codes)
    const int buf = F8 ? 0 : par;
    // tile kt has landed in LDS; every wave is done with tile kt - 1 and with the block window
    tile_barrier();
    if (kt + 1 < n_tiles) {
      const int last_key = min((kt + 2) * kPrefillKeyTile, kv_end) - 1;
      if (entry_of(last_key) >= win0 + kPrefillBlockWindow) {   // uniform: slide the window
        win0 = entry_of((kt + 1) * kPrefillKeyTile);
        load_window();
        tile_barrier();
      }
      // in flight while this tile is computed
      if constexpr (F8) dma_codes(kt + 1, par ^ 1);
      else dma_tile(kt + 1, buf ^ 1);
    }
    if constexpr (F8) {
      // every wave widens its share of tile kt (its codes landed before the barrier above; the
      // bf16 buffer is free: every wave has finished tile kt - 1), then the workgroup meets
      widen(par);
      lds_barrier();
    }

    if (kt * kPrefillKeyTile > wave_last_pos) return;  // no row of this wave sees this tile
    // LDS byte addresses of the operand reads, derived once per tile from this lane's fixed
    // parts (kept opaque so that the compiler recomputes them here instead of holding every
    // derived address in a register across the loop)
    const uint32_t k_x = opaque_u32(k_x0);
    const uint32_t v_y0 = opaque_u32(v_y0_);
    const uint32_t v_y1 = opaque_u32(v_y1_);
    // (LDS pointers, so that the k-step's and block's constant parts become instruction offsets)
    lds_char_t* const k_ptr = (lds_char_t*)(s_kv[buf][0]) + k_base;
    lds_char_t* const v_ptr = (lds_char_t*)(s_kv[buf][1]);

    // ---- S^T = K Q^T: two 32-key blocks; every K fragment of the tile is read before the
    //      MFMAs so that the LDS latency is paid once ----
    f32x16_t s[2];
    u32x4v_t kf[2][KS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[kb][ks] =
            *(const lds_u32x4_t*)(k_ptr + ((32u * ks) ^ k_x) + kb * 32 * CPR * 16);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[kb][ks]),
                                                        qf[ks], s[kb], 0, 0, 0);
    }

    // ---- online softmax for this lane's M-row (keys split with lane ^ 32), base 2 ----
    // Exponents are taken against a reference m_ref that trails the running max by less than
    // kRescaleSlack (p <= 2^slack); O and l are rescaled only when the max rises past it. Each
    // form is straight-line code, so the exponentials of one key group can be scheduled beside
    // the MFMAs of the previous one.
    const int tile_key0 = kt * kPrefillKeyTile;
    // V^T operand of k-step q (key rows 16 q .. 16 q + 15), all d blocks
    auto read_v = [&](int q, bf16x8_t (&vf)[DB]) {
      const uint32_t qoff = 16u * q * CPR * 16;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        lds_char_t* const a0 = v_ptr + (v_base0 + ((64u * db) ^ v_y0)) + qoff;
        lds_char_t* const a1 = v_ptr + (v_base1 + ((64u * db) ^ v_y1)) + qoff;
        const s16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)a0);
        const s16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)a1);
        const s16x4_t tt[2] = {t0, t1};
        vf[db] = __builtin_bit_cast(bf16x8_t, tt);
      }
    };
    auto softmax_pv = [&](auto masked_tag) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      // the first k-step's V^T reads are in flight during the max
      bf16x8_t vf[DB];
      read_v(0, vf);
      __builtin_amdgcn_sched_barrier(0);
      // key of score register r of block kb for this lane
      auto key_of = [&](int kb, int r) {
        return tile_key0 + kb * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3);
      };
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          tmax = fmaxf(tmax, (!MASKED || key_of(kb, r) <= pos) ? s[kb][r] : -INFINITY);
      tmax = across32(tmax, MaxOp());
      // scale >= 0 keeps the order of scores; fmaxf drops the NaN of -inf * 0
      const float m_cand = fmaxf(m_ref, tmax * sl2);
      const bool need = m_cand > m_ref + kRescaleSlack;
      if (__any(need)) {
        // a multiply by exactly 1 (rows that keep their reference) changes nothing
        const float alpha = need ? fast_exp2(m_ref - m_cand) : 1.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
        l_run *= alpha;
        m_ref = need ? m_cand : m_ref;
      }
      const float neg_m = -m_ref;

      // ---- O^T += V^T P^T per 16-key k-step q = (kb, m); the A operand (V^T) comes from two
      //      transpose reads, the B operand (P^T) is this lane's own probabilities ----
      float psum = 0.f;
      // P = hi + lo for k-step q: hi = p with its low 16 bits cleared (a bfloat16 value), lo =
      // the exact float32 remainder rounded to bfloat16, so hi + lo carries about 16 bits of p
      auto make_p = [&](int q, bf16x8_t& phi, bf16x8_t& plo) {
        const int kb = q >> 1, m = q & 1;
        uint32_t phw[4], plw[4];
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          float p0 = fast_exp2(fmaf(s[kb][8 * m + j], sl2, neg_m));
          float p1 = fast_exp2(fmaf(s[kb][8 * m + j + 1], sl2, neg_m));
          if constexpr (MASKED) {
            const int key = key_of(kb, 8 * m + j);
            p0 = key <= pos ? p0 : 0.f;
            p1 = key + 1 <= pos ? p1 : 0.f;
          }
          psum += p0;
          psum += p1;
          const uint32_t b0 = __float_as_uint(p0), b1 = __float_as_uint(p1);
          phw[j / 2] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
          const float l0 = p0 - __uint_as_float(b0 & 0xffff0000u);
          const float l1 = p1 - __uint_as_float(b1 & 0xffff0000u);
          typedef float f32x2_t __attribute__((ext_vector_type(2)));
          plw[j / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{l0, l1}, bf16x2_t));
        }
        phi = __builtin_bit_cast(bf16x8_t, phw);
        plo = __builtin_bit_cast(bf16x8_t, plw);
      };
      bf16x8_t phi, plo;
      make_p(0, phi, plo);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // the next k-step's V^T reads are in flight during this one's MFMAs
        bf16x8_t vn[DB];
        if (q + 1 < 4) read_v(q + 1, vn);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db], phi, acc[db], 0, 0, 0);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db], plo, acc[db], 0, 0, 0);
        }
        if (q + 1 < 4) {
          make_p(q + 1, phi, plo);
#pragma unroll
          for (int db = 0; db < DB; ++db) vf[db] = vn[db];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      l_run += psum;
    };
    softmax_pv(masked_tag);
  };
  for (int kt = kt0; kt < kd; ++kt) tile_step(kt, std::false_type{});
  for (int kt = kd; kt < n_tiles; ++kt) tile_step(kt, std::true_type{});

  if (bad) s_bad = 1;
  __syncthreads();
  const bool bad_item = s_bad != 0;
  if (!real) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float vs = a.v_scale;
  if (a.tile_split > 0 && !(it.split == 0 && pos < a.tile_split)) {
    // a row whose keys reach past split 0: the partial (m, l, V-scaled acc) of this split, or
    // nothing when the row ends before the split
    if (pos < kv0) return;
    const int64_t pidx = (static_cast<int64_t>(it.part) + static_cast<int64_t>(qrow) * it.pstride +
                          it.split) * a.hq + static_cast<int64_t>(g) * G + head;
    if (h32 == 0) {
      a.part_m[pidx] = m_ref;
      a.part_l[pidx] = bad_item ? __builtin_nanf("") : l_tot;
    }
    float* pd = a.part_acc + pidx * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        float4 o;
        o.x = F8 ? acc[db][4 * rq + 0] * vs : acc[db][4 * rq + 0];
        o.y = F8 ? acc[db][4 * rq + 1] * vs : acc[db][4 * rq + 1];
        o.z = F8 ? acc[db][4 * rq + 2] * vs : acc[db][4 * rq + 2];
        o.w = F8 ? acc[db][4 * rq + 3] * vs : acc[db][4 * rq + 3];
        if (bad_item) o = make_float4(__builtin_nanf(""), __builtin_nanf(""),
                                      __builtin_nanf(""), __builtin_nanf(""));
        *reinterpret_cast<float4*>(pd + 32 * db + 8 * rq + 4 * h32) = o;
      }
    return;
  }
  float* dst = a.out + ((static_cast<int64_t>(it.row0) + qrow) * a.hq +
                        static_cast<int64_t>(g) * G + head) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      float4 o;
      if constexpr (F8) {
        o.x = acc[db][4 * rq + 0] * vs / l_tot;
        o.y = acc[db][4 * rq + 1] * vs / l_tot;
        o.z = acc[db][4 * rq + 2] * vs / l_tot;
        o.w = acc[db][4 * rq + 3] * vs / l_tot;
      } else {
        o.x = acc[db][4 * rq + 0] / l_tot;
        o.y = acc[db][4 * rq + 1] / l_tot;
        o.z = acc[db][4 * rq + 2] / l_tot;
        o.w = acc[db][4 * rq + 3] / l_tot;
      }
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
static hipError_t launch_prefill_d(const PrefillArgs& a, uint32_t grid, int group, bool fp8,
                                   uint32_t lds_pad, hipStream_t stream) {
  if (fp8) {
    switch (group) {   // E4M3 pools: the groups the E4M3 decode pass serves
      case 1: hipLaunchKernelGGL((prefill_kernel<D, 1, true>), dim3(grid), dim3(256), lds_pad, stream, a); break;
      case 2: hipLaunchKernelGGL((prefill_kernel<D, 2, true>), dim3(grid), dim3(256), lds_pad, stream, a); break;
      case 4: hipLaunchKernelGGL((prefill_kernel<D, 4, true>), dim3(grid), dim3(256), lds_pad, stream, a); break;
      case 8: hipLaunchKernelGGL((prefill_kernel<D, 8, true>), dim3(grid), dim3(256), lds_pad, stream, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (group) {
    case 1: hipLaunchKernelGGL((prefill_kernel<D, 1, false>), dim3(grid), dim3(256), lds_pad, stream, a); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<D, 2, false>), dim3(grid), dim3(256), lds_pad, stream, a); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<D, 4, false>), dim3(grid), dim3(256), lds_pad, stream, a); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<D, 8, false>), dim3(grid), dim3(256), lds_pad, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, int64_t n_items, int head_dim, int group,
                          bool fp8, hipStream_t stream, uint32_t lds_pad) {
  const int64_t grid64 = n_items * a.hkv;
  if (grid64 == 0) return hipSuccess;
  if (grid64 > 0x7fffffffLL || n_items != a.n_items) return hipErrorInvalidValue;
  const uint32_t grid = static_cast<uint32_t>(grid64);
  if (head_dim == 64) return launch_prefill_d<64>(a, grid, group, fp8, lds_pad, stream);
  if (head_dim == 128) return launch_prefill_d<128>(a, grid, group, fp8, lds_pad, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
