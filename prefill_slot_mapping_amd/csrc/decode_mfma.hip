// Decode split pass on bf16 MFMA (v_mfma_f32_16x16x32_bf16) for gfx950 (MI355X), for groups of
// 8 query heads per kv head, over bf16 pools and over E4M3 pools. There the vector kernels'
// per-key arithmetic (G x head_dim multiply-adds for the scores and as many for P.V, plus the
// code widening of E4M3) and their per-lane head layouts bound them below the HBM rate.
//
// Sources of the operation: "P3: native paged-KV continuous-batching sampler", section
// "Design > paged.py", TritonPagedAttention (a fixed KV split per context length, no atomics),
// "Finish RL Training Faster: Bitwise-Consistent ..." section 2 (batch independence) and section
// 4.2 (FP8 KV storage with per-tensor scales, one read path).
//
// Work item: (query row, split, kv head), as for the other decode kernels (same lists, same
// partial slots, same split merge). Four waves; tile i of the split (32 keys aligned at the split
// start) goes to wave i % 4, which visits its tiles in ascending order. A tile's K and V rows are
// loaded whole, 16 bytes a lane (each load instruction reads complete rows: 8 keys of E4M3 codes
// at head_dim 128, 4 keys of bf16); reading 64-byte pieces of 16 rows per instruction straight
// into the operand layout was 15 % slower. Per tile and wave:
//   S^T[key][head] = K Q^T   two 16-key blocks x D/32 MFMAs. K rows go to the wave's LDS tile
//                            (16-byte chunks XOR-swizzled per row, so the 16 rows of an operand
//                            read fall on distinct banks) and come back as the A operand: lane l
//                            takes key l % 16, k-step st the 8 values at d = 64 (st / 2) +
//                            16 (l / 16) + 8 (st % 2) + e (E4M3 codes widened exactly to bf16) -
//                            a fixed order of the dot product's terms, the same for q and K. The
//                            G query heads are the B operand's columns (columns past G are
//                            zero). An E4M3 K scale is folded into the score scale by the host.
//   softmax, base 2          lane l holds head l % 16 at keys 4 (l / 16) + r of each block; the
//                            lazy reference of the other decode kernels (rescale only when a
//                            score passes it by 8), p = 2^(s scale_log2e - m), l summed per lane.
//   O^T[d][head] += V^T P^T  D/16 MFMAs per P part; P = hi + lo (hi: p with its low 16 bits
//                            cleared, a bf16 value; lo: the float32 remainder rounded to bf16),
//                            about 16 bits of p. V rows replace K in the wave's LDS tile once the
//                            scores are read (16-byte chunks XOR-swizzled per row) and come back
//                            transposed, each lane one d column over its 8 keys: one
//                            ds_read_b64_tr_b8 per 16-wide d block for E4M3 codes (widened
//                            exactly to bf16 in registers), two ds_read_b64_tr_b16 for bf16.
// Keys past the split's context are masked (-inf scores; their V rows zeroed before the LDS
// write, so no pool value past the context enters a sum). The wave partials are merged in wave
// order exactly as in the vector decode kernels, an E4M3 V scale applied once to the merged
// numerator. Every operation depends only on the row's query, its own keys and the split, never
// on other rows of the batch.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "kernels.h"
#include "lane_ops.h"

namespace pkv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;

constexpr int kMfmaTileKeys = 32;

// E4M3 V tile: 16-byte chunk swizzle of row r (CPR chunks a row). The transposed read of a d
// block takes 8 rows {4q .. 4q + 3, 16 + 4q .. 16 + 4q + 3} (q = lane quarter), both halves of
// their chunk; rows of one parity share a bank half, so their chunks must differ - over the
// rows of two neighbouring quarters too (for D = 128: bits 1, 4 and 2 of r; for D = 64, whose
// rows cover a quarter of the banks: bits 2 and 4).
template <int CPR>
__device__ __forceinline__ int vswz8(int r) {
  if constexpr (CPR == 8) return ((r >> 1) & 1) | (((r >> 4) & 1) << 1) | (((r >> 2) & 1) << 2);
  else return ((r >> 2) & 1) | (((r >> 4) & 1) << 1);
}

// bf16 V tile: chunk swizzle of row r (CPR chunks a row). The transposed read of d block db
// takes chunks 2 db and 2 db + 1 of rows 4q .. 4q + 3 in lane quarter q; over the 8 rows of two
// neighbouring quarters the chunk pairs must land on distinct banks (XOR with an even value keeps
// a pair's chunks apart, the low bit separates the two row octets).
template <int CPR>
__device__ __forceinline__ int vswz16(int r) {
  if constexpr (CPR == 16) return ((r & 7) << 1) | ((r >> 3) & 1);
  else return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
}

// K tile (either element type): chunk swizzle of row r, so that the 16 rows an A-operand read
// takes (one chunk position each) fall on distinct banks: rows sharing a 256-byte bank span
// (256 / row bytes of them) get distinct chunk positions.
template <int CPR>
__device__ __forceinline__ int kswz(int r) {
  constexpr int kRowsPerSpan = CPR >= 16 ? 1 : 16 / CPR;
  return (r / kRowsPerSpan) & (CPR - 1);
}

// 16 bytes at base + off (base the same in every lane), nontemporal, as a global-memory load
// with a scalar base and a 32-bit lane offset
__device__ __forceinline__ uint4 load_nt_global(const char* base, uint32_t off) {
  asm("" : "+v"(off));   // a 32-bit value here, so the offset is not widened ahead of time
  typedef unsigned u4v __attribute__((ext_vector_type(4)));
  const __attribute__((address_space(1))) u4v* p =
      reinterpret_cast<const __attribute__((address_space(1))) u4v*>(
          (const __attribute__((address_space(1))) char*)(base) + off);
  const u4v t = __builtin_nontemporal_load(p);
  return make_uint4(t.x, t.y, t.z, t.w);
}

// a pointer that is the same in every lane, as such (scalar registers)
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t x = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x >> 32));
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// two E4M3 codes (bytes 0-1, or 2-3 with hi) of w -> a bfloat16 pair, exactly
__device__ __forceinline__ uint32_t e4m3x2_bf16x2(uint32_t w, bool hi) {
  return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                                         : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}

// eight E4M3 codes (w0 bytes 0-3, w1 bytes 0-3) -> eight bfloat16 values, exactly
__device__ __forceinline__ uint4 e4m3x8_bf16x8(uint32_t w0, uint32_t w1) {
  return make_uint4(e4m3x2_bf16x2(w0, false), e4m3x2_bf16x2(w0, true),
                    e4m3x2_bf16x2(w1, false), e4m3x2_bf16x2(w1, true));
}

}  // namespace

template <int D, int G, int W, bool FP8, int R>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(W, W)))
decode_mfma_kernel(DecodeArgs a) {
  constexpr int TK = kMfmaTileKeys;
  constexpr int RB = FP8 ? D : 2 * D;     // bytes of a pool row (one key, one kv head)
  constexpr int KS = D / 32;              // k-steps of S^T per 16-key block
  constexpr int CPRV = RB / 16;           // 16-byte chunks of a pool row
  constexpr int RPI = 64 / CPRV;          // rows per K / V load instruction
  constexpr int VU4 = TK / RPI;           // K / V load instructions per tile
  constexpr int DB = D / 16;              // 16-wide d blocks of O^T
  constexpr float kRescaleLog2 = 8.f;
  constexpr int NC = R * G;               // MFMA columns in use: (row r, head h) at r G + h
  static_assert(NC >= 1 && NC <= 16 && R <= kGroupRows && VU4 >= 1 && TK % RPI == 0, "shape");

  constexpr int kTileBytes = kDecodeWaves * TK * RB;
  constexpr int MD = D + 4;                // merge row stride (floats): columns on distinct banks
  constexpr int kMergeBytes = kDecodeWaves * NC * (MD + 2) * 4;
  __shared__ __align__(16) char s_kv[kTileBytes > kMergeBytes ? kTileBytes : kMergeBytes];
  __shared__ uint32_t s_slot[kMaxDecodeSplit];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int quarter = lane >> 4;   // S^T / O^T rows 4 quarter .. + 3; K d range; P keys
  const int col = lane & 15;       // S^T / O^T column: query head col of the group (< G)
  // Items in grid order: the host lists them longest first and the hardware deals consecutive
  // workgroups to the 8 XCDs in turn, so every XCD gets its share of full and short splits.
  const int f = blockIdx.x;
  const int item_idx = f / a.hkv;
  const int g = f - item_idx * a.hkv;
  const int hq0 = g * G;
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
  const int nk = t1 - t0;
  const int nk_pad = (nk + TK - 1) / TK * TK;
  const int32_t* bt = a.block_tables + static_cast<int64_t>(seq[0]) * a.max_blocks;
  // slot of each key of the split (keys past the context: the last key's slot); an out-of-pool
  // block id marks the item bad and reads slot 0
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
  // group items: rows after the first must name the same blocks over the split (else they are
  // written as NaN rather than computed from the first row's keys)
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

  // B operand of S^T: column col = (row col / G, head col % G) takes that q row's 8 d of k-step
  // st in this lane's quarter; columns past the item's rows are zero
  bf16x8_t qf[KS];
  {
    const int cr = col / G;
    int qrow = row[0];
#pragma unroll
    for (int r = 1; r < R; ++r) qrow = cr == r ? row[r] : qrow;
    const bool hv = col < NC && cr < n_rows;
    const uint4* qs = reinterpret_cast<const uint4*>(
        static_cast<const char*>(a.q) +
        (static_cast<int64_t>(hv ? qrow : row[0]) * a.hq + hq0 + (hv ? col % G : 0)) * (D * 2));
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const int d0 = 64 * (st / 2) + 16 * quarter + 8 * (st % 2);
      qf[st] = __builtin_bit_cast(bf16x8_t, hv ? qs[d0 / 8] : make_uint4(0u, 0u, 0u, 0u));
    }
  }
  __syncthreads();

  const uint64_t slot_bytes = static_cast<uint64_t>(a.hkv) * RB;
  const int vrow = lane / CPRV;     // row of a K / V load instruction
  const int vchunk = lane % CPRV;   // 16-byte chunk of that row
  const char* kbase = static_cast<const char*>(a.k_cache) + g * RB + vchunk * 16;
  const char* vbase = static_cast<const char*>(a.v_cache) + g * RB + vchunk * 16;
  // this lane's byte offset from the slot of the first key its instruction row covers
  const uint32_t lane_off = static_cast<uint32_t>(vrow * slot_bytes) + vchunk * 16;
  const char* kbase_u = static_cast<const char*>(a.k_cache) + g * RB;   // the same in every lane
  const char* vbase_u = static_cast<const char*>(a.v_cache) + g * RB;
  // blocks of 16 keys or more (a power of two): the 16 keys of a tile half are consecutive
  // slots of one block (tiles start at multiples of 32 keys); the lane's 32-bit offset from
  // its instruction's first row (under 16 rows) needs slots of at most 64 MiB
  const bool halves_in_block = a.bs_log2 >= 4 && slot_bytes <= (uint64_t{1} << 26);
  const int last16 = (nk - 1) & ~15;

  // the wave's LDS tile: K codes / values of the tile, then (once the scores are taken) its V
  char* skv = s_kv + wave * TK * RB;
  lds_char_t* skv_lds = (lds_char_t*)(skv);
  // transposed-read address of this lane. E4M3: row 4 quarter + k (k = col >> 1 < 4) or
  // 16 + 4 quarter + k - 4, the half col & 1 of chunk db. bf16: rows 4 quarter + (col >> 2) and
  // 16 + that, 8 bytes at 4 (col & 3) values into d block db (chunk 2 db + ((col & 3) >> 1)).
  const int k8 = col >> 1;
  const int tr_row = FP8 ? (k8 < 4 ? 4 * quarter + k8 : 16 + 4 * quarter + k8 - 4)
                         : 4 * quarter + (col >> 2);
  const int tr_off = tr_row * RB + 8 * (col & 1);
  const int tr_sw = FP8 ? vswz8<CPRV>(tr_row) : vswz16<CPRV>(tr_row);
  const int tr_h = (col & 3) >> 1;

  float m_ref = -INFINITY;
  float l_run = 0.f;
  f32x4_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const float sl2 = a.scale_log2e;

  // slots of the first keys of the tile's two halves (blocks of 16 keys or more)
  auto half_bases = [&](int ts, uint32_t& base0, uint32_t& base1) {
    base0 = __builtin_amdgcn_readfirstlane(s_slot[ts]);
    base1 = __builtin_amdgcn_readfirstlane(s_slot[min(ts + 16, last16)]);
  };
  // K and V rows of tile ts: the slots first (one uniform branch per tile, the LDS reads of
  // the general path issued together), then the loads; lane (vrow, vchunk) of instruction u
  // takes chunk vchunk of key u RPI + vrow of both tensors
  auto load_kv = [&](uint4 (&kr)[VU4], uint4 (&vr)[VU4], int ts) {
    if (halves_in_block) {
      // instruction u covers rows u RPI .. u RPI + RPI - 1, all in one half (RPI divides 16):
      // the slot of its first row is the same in every lane, the lane adds its row and chunk
      uint32_t base0, base1;
      half_bases(ts, base0, base1);
#pragma unroll
      for (int u = 0; u < VU4; ++u) {
        const int r0 = u * RPI;
        const uint64_t row0 = static_cast<uint64_t>((r0 < 16 ? base0 : base1) + (r0 & 15)) *
                              slot_bytes;
        // (the row's address kept uniform, so that the load takes it as its scalar base)
        const char* kp = uniform_ptr(kbase_u + row0);
        const char* vp = uniform_ptr(vbase_u + row0);
        kr[u] = load_nt_global(kp, lane_off);
        vr[u] = load_nt_global(vp, lane_off);
      }
      return;
    }
    uint32_t sl[VU4];
    {
#pragma unroll
      for (int u = 0; u < VU4; ++u) sl[u] = s_slot[ts + u * RPI + vrow];
    }
#pragma unroll
    for (int u = 0; u < VU4; ++u) {
      kr[u] = load_nt(reinterpret_cast<const uint4*>(kbase + sl[u] * slot_bytes));
      vr[u] = load_nt(reinterpret_cast<const uint4*>(vbase + sl[u] * slot_bytes));
    }
  };

  // Tile ts from buffers kr / vr, which are refilled with tile nxt (when refill) once consumed
  // (after the K and V tiles' LDS writes), so that tile stays in flight through the score
  // MFMAs, softmax and P.V of this one.
  auto compute = [&](uint4 (&kr)[VU4], uint4 (&vr)[VU4], int ts, bool refill, int nxt) {
    asm volatile("" ::: "memory");
    const int n = nk - ts;   // keys of this tile inside the context (>= 1)
    // ---- K rows into the wave's LDS tile (keys past the context are masked below) ----
#pragma unroll
    for (int u = 0; u < VU4; ++u) {
      const int r = u * RPI + vrow;
      *reinterpret_cast<uint4*>(skv + r * RB + ((vchunk ^ kswz<CPRV>(r)) * 16)) = kr[u];
    }

    // ---- S^T = K Q^T, the two 16-key blocks interleaved ----
    f32x4_t s[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int st = 0; st < KS; ++st)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key = 16 * kb + col;
        uint4 kf;
        if constexpr (FP8) {
          const int c = 4 * (st / 2) + quarter;
          const uint2 w2 = *reinterpret_cast<const uint2*>(
              skv + key * RB + ((c ^ kswz<CPRV>(key)) * 16) + 8 * (st & 1));
          kf = e4m3x8_bf16x8(w2.x, w2.y);
        } else {
          const int c = 8 * (st / 2) + 2 * quarter + (st & 1);
          kf = *reinterpret_cast<const uint4*>(skv + key * RB + ((c ^ kswz<CPRV>(key)) * 16));
        }
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf), qf[st],
                                                        s[kb], 0, 0, 0);
      }

    // ---- V rows into the same tile once the scores are read (rows past the context: zero) ----
#pragma unroll
    for (int u = 0; u < VU4; ++u) {
      const int r = u * RPI + vrow;
      uint4 v = vr[u];
      if (n < TK && r >= n) v = make_uint4(0u, 0u, 0u, 0u);
      const int sw = FP8 ? vswz8<CPRV>(r) : vswz16<CPRV>(r);
      *reinterpret_cast<uint4*>(skv + r * RB + ((vchunk ^ sw) * 16)) = v;
    }
    if (refill) load_kv(kr, vr, nxt);

    // ---- lazy online softmax (base 2) for head col over this lane's 8 keys ----
    float t[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) t[kb][r] = s[kb][r] * sl2;
    if (n < TK) {   // the split's last tile: keys past the context get -inf
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * kb + 4 * quarter + r >= n) t[kb][r] = -INFINITY;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, t[kb][r]);
    tmax = across16(tmax, MaxOp());
    tmax = across32(tmax, MaxOp());
    const float m_cand = fmaxf(m_ref, tmax);
    const bool need = m_cand > m_ref + kRescaleLog2;
    if (__any(need)) {
      // a multiply by exactly 1 (heads that keep their reference) changes nothing
      const float al = need ? fast_exp2(m_ref - m_cand) : 1.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[db][r] *= al;
      l_run *= al;
      m_ref = need ? m_cand : m_ref;
    }
    uint32_t phw[4], plw[4];
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const float p0 = fast_exp2(t[kb][r] - m_ref);
        const float p1 = fast_exp2(t[kb][r + 1] - m_ref);
        ps += p0;
        ps += p1;
        const uint32_t b0 = __float_as_uint(p0), b1 = __float_as_uint(p1);
        phw[2 * kb + r / 2] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
        const float l0 = p0 - __uint_as_float(b0 & 0xffff0000u);
        const float l1 = p1 - __uint_as_float(b1 & 0xffff0000u);
        plw[2 * kb + r / 2] =
            __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{l0, l1}, bf16x2_t));
      }
    l_run += ps;
    const bf16x8_t phi = __builtin_bit_cast(bf16x8_t, phw);
    const bf16x8_t plo = __builtin_bit_cast(bf16x8_t, plw);

    // ---- O^T += V^T P^T: V^T from transposed reads per d block (keys 4 quarter + 0..3,
    //      16 + 4 quarter + 0..3 at d = 16 db + col): one of E4M3 codes, two of bf16 ----
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      bf16x8_t va;
      if constexpr (FP8) {
        const i32x2_t c8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (lds_i32x2_t*)(skv_lds + tr_off + ((db ^ tr_sw) * 16)));
        va = __builtin_bit_cast(
            bf16x8_t, e4m3x8_bf16x8(static_cast<uint32_t>(c8.x), static_cast<uint32_t>(c8.y)));
      } else {
        const int off = tr_off + (((2 * db + tr_h) ^ tr_sw) * 16);
        const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(skv_lds + off));
        const i16x4_t v1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(skv_lds + off + 16 * RB));
        va = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi, acc[db], 0, 0, 0);
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo, acc[db], 0, 0, 0);
    }
  };

  // Tiles j = 0 .. n_tiles - 1 of this wave (keys wave TK + j kStep ..), ascending, through one
  // register buffer: tile j + 1 is loaded as soon as tile j's registers are consumed, inside
  // the loop unconditionally, so the compiler's wait before each tile covers just that tile (a
  // load under a condition between a load and its use makes it wait for every load). Measured
  // on the long-context E4M3 step: two or three buffers at two waves per SIMD, or one buffer at
  // four (with spills), were slower than one buffer at three.
  constexpr int kStep = kDecodeWaves * TK;
  const int n_tiles = nk > wave * TK ? (nk - wave * TK + kStep - 1) / kStep : 0;
  uint4 kbuf[VU4];
  uint4 vbuf[VU4];
  if (n_tiles > 0) {
    load_kv(kbuf, vbuf, wave * TK);
    for (int j = 0; j + 1 < n_tiles; ++j)
      compute(kbuf, vbuf, wave * TK + j * kStep, true, wave * TK + (j + 1) * kStep);
    compute(kbuf, vbuf, wave * TK + (n_tiles - 1) * kStep, false, 0);
  }

  // l over the four key quarters of head col (the same sum in every lane of the head)
  l_run = across16(l_run, AddOp());
  l_run = across32(l_run, AddOp());

  const bool bad_row = __syncthreads_or(bad) != 0;   // also: every wave is done with s_kv
  float* mg_acc = reinterpret_cast<float*>(s_kv);          // [4][NC][MD]
  float* mg_m = mg_acc + kDecodeWaves * NC * MD;           // [4][NC]
  float* mg_l = mg_m + kDecodeWaves * NC;                  // [4][NC]
  if (col < NC) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
      *reinterpret_cast<f32x4_t*>(mg_acc + (wave * NC + col) * MD + 16 * db + 4 * quarter) = acc[db];
    if (quarter == 0) {
      mg_m[wave * NC + col] = m_ref;
      mg_l[wave * NC + col] = l_run;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < NC * D; idx += 256) {
    const int c = idx / D;
    const int d = idx - c * D;
    const int cr = c / G;
    if (cr >= n_rows) continue;
    int orow = row[0], opart = part[0];
    bool obad = row_bad[0];
#pragma unroll
    for (int r = 1; r < R; ++r) {
      orow = cr == r ? row[r] : orow;
      opart = cr == r ? part[r] : opart;
      obad = cr == r ? row_bad[r] : obad;
    }
    obad = obad || bad_row;
    float M = mg_m[c];
#pragma unroll
    for (int w = 1; w < kDecodeWaves; ++w) M = fmaxf(M, mg_m[w * NC + c]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float fw = fast_exp2(mg_m[w * NC + c] - M);
      num = fmaf(fw, mg_acc[(w * NC + c) * MD + d], num);
      den = fmaf(fw, mg_l[w * NC + c], den);
    }
    if constexpr (FP8) num *= a.v_scale;
    const uint32_t nan_bits = 0x7fc00000u;
    const int hq = hq0 + c - cr * G;
    if (opart < 0) {
      const float o = num / den;
      a.out[(static_cast<int64_t>(orow) * a.hq + hq) * D + d] =
          __uint_as_float(obad ? nan_bits : __float_as_uint(o));
    } else {
      const int64_t p = static_cast<int64_t>(opart + split) * a.hq + hq;
      a.part_acc[p * D + d] = __uint_as_float(obad ? nan_bits : __float_as_uint(num));
      if (d == 0) {
        a.part_m[p] = M;
        a.part_l[p] = __uint_as_float(obad ? nan_bits : __float_as_uint(den));
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------------------
bool decode_mfma_supported(int head_dim, int group) {
  return (head_dim == 64 || head_dim == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

// Rows of a group item: as many as fill the 16 MFMA columns, at most kGroupRows.
int decode_mfma_group_rows(int group) {
  return group >= 1 && group <= 16 ? (16 / group < kGroupRows ? 16 / group : kGroupRows) : 1;
}

namespace {

// Waves per SIMD (measured on the long-context and batched decode steps): three, except bf16
// at head_dim 128 (226 registers: two; at three it spills and takes 1.4 times as long).
template <int D, bool FP8>
constexpr int mfma_waves() {
  return (!FP8 && D == 128) ? 2 : 3;
}

template <int D, int G, bool FP8>
void launch_g(const DecodeArgs& a, uint32_t grid, bool groups, hipStream_t stream) {
  constexpr int W = mfma_waves<D, FP8>();
  constexpr int RG = 16 / G < kGroupRows ? 16 / G : kGroupRows;
  if (groups)
    hipLaunchKernelGGL((decode_mfma_kernel<D, G, W, FP8, RG>), dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<D, G, W, FP8, 1>), dim3(grid), dim3(256), 0, stream, a);
}

template <int D, bool FP8>
hipError_t launch_d(const DecodeArgs& a, uint32_t grid, int group, bool groups,
                    hipStream_t stream) {
  switch (group) {
    case 1: launch_g<D, 1, FP8>(a, grid, groups, stream); break;
    case 2: launch_g<D, 2, FP8>(a, grid, groups, stream); break;
    case 4: launch_g<D, 4, FP8>(a, grid, groups, stream); break;
    case 8: launch_g<D, 8, FP8>(a, grid, groups, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, uint32_t grid, int head_dim, int group,
                              bool fp8, bool groups, hipStream_t stream) {
  if (!decode_mfma_supported(head_dim, group)) return hipErrorInvalidValue;
  if (head_dim == 64)
    return fp8 ? launch_d<64, true>(a, grid, group, groups, stream)
               : launch_d<64, false>(a, grid, group, groups, stream);
  return fp8 ? launch_d<128, true>(a, grid, group, groups, stream)
             : launch_d<128, false>(a, grid, group, groups, stream);
}

}  // namespace pkv
