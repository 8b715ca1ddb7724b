// Internal launch interface of the HIP kernels (write_kv.hip, decode.hip, merge.hip,
// prefill.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.h"

namespace pkv {

struct WriteArgs {
  const void* k_new;
  const void* v_new;
  const int32_t* slots;
  int32_t n_rows;
  int32_t chunks_per_row;  // num_kv_heads * head_dim * elem_bytes / 16
  int64_t n_slots;         // num_blocks * block_size
  void* k_cache;
  void* v_cache;
};

// Work lists staged in pinned host memory, copied to the workspace by the first blocks of a
// fused append launch (src is the device mapping of the staging buffer).
struct StageArgs {
  const uint4* src;
  uint4* dst;
  int32_t n_u4;         // 16-byte chunks to copy
  int32_t copy_blocks;  // blocks [0, copy_blocks) copy; the others append
};

struct CopyArgs {
  void* k_cache;
  void* v_cache;
  const int32_t* pairs;       // [2 * n_pairs] (src, dst) block ids, validated on the host
  int32_t n_pairs;
  int32_t chunks_per_block;   // block_size * num_kv_heads * head_dim * elem_bytes / 16
};

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int32_t max_blocks;
  int32_t block_size;
  int32_t bs_log2;  // log2(block_size) when it is a power of two, else -1
  int32_t num_blocks;
  int32_t hq;
  int32_t hkv;
  int32_t group;      // hq / hkv
  int32_t kv_split;
  float scale_log2e;  // softmax scale times log2(e): scores live in the base-2 domain
                      // (E4M3 pools: times the K scale as well)
  float v_scale;      // E4M3 pools: the V scale (1 otherwise)
  const DecodeItem* items;
  const DecodeGroupItem* groups;  // group items (launch_decode_groups only)
  float* out;
  float* part_m;
  float* part_l;
  float* part_acc;
};

struct WriteFp8Args {
  const void* k_new;       // bfloat16 [n_rows, Hkv, D]
  const void* v_new;
  const int32_t* slots;
  int32_t n_rows;
  int32_t chunks_per_row;  // num_kv_heads * head_dim / 16 (16-byte chunks of a pool row)
  int64_t n_slots;
  float k_inv_scale;       // float32(1 / k_scale)
  float v_inv_scale;
  void* k_cache;           // E4M3 codes [NB, BS, Hkv, D]
  void* v_cache;
};

struct MergeArgs {
  const MergeItem* items;
  int32_t hq;
  int32_t n_waves;  // merge items x hq
  const float* part_m;
  const float* part_l;
  const float* part_acc;
  float* out;
};

struct PrefillArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int32_t max_blocks;
  int32_t block_size;
  int32_t bs_log2;  // log2(block_size) when it is a power of two, else -1
  int32_t num_blocks;
  int32_t hq;
  int32_t hkv;
  int32_t n_items;
  float scale_log2e;  // |scale| * log2(e) (E4M3 pools: times the K scale as well)
  int32_t negate_q;   // scale < 0: the kernel flips the sign of q instead
  float v_scale;      // E4M3 pools: the V scale (1 otherwise)
  const PrefillItem* items;
  float* out;
  int32_t tile_split;  // > 0: each item covers one KV split of this many keys (see PrefillItem)
  float* part_m;       // split partials, laid out as those of DecodeArgs
  float* part_l;
  float* part_acc;
};

// Each launcher enqueues one kernel on `stream` and returns hipSuccess or the launch error.
hipError_t launch_write_kv(const WriteArgs& a, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream);
hipError_t launch_write_kv_fp8(const WriteFp8Args& a, hipStream_t stream);
// The copy of st and the append of a in one launch; a.slots may point into st.src's memory.
hipError_t launch_stage_write_kv(const StageArgs& st, const WriteArgs& a, hipStream_t stream);
hipError_t launch_stage_write_kv_fp8(const StageArgs& st, const WriteFp8Args& a,
                                     hipStream_t stream);
hipError_t launch_decode_fp8(const DecodeArgs& a, int64_t n_items, int head_dim, int group,
                             hipStream_t stream);
// decode_mfma.hip: the decode split pass on MFMA, bf16 or E4M3 pools (grid = items x hkv).
// groups: a.groups holds group items of up to decode_mfma_group_rows(group) rows; otherwise
// a.items holds per-row items.
bool decode_mfma_supported(int head_dim, int group);
int decode_mfma_group_rows(int group);
hipError_t launch_decode_mfma(const DecodeArgs& a, uint32_t grid, int head_dim, int group,
                              bool fp8, bool groups, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int64_t n_items, int head_dim, int group,
                         bool bf16, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, int64_t n_items, int head_dim, hipStream_t stream);
// The group items a.groups[0 .. n_groups): each row computed exactly as by launch_decode
// (bf16 pools) or launch_decode_fp8 (fp8: E4M3 pools).
hipError_t launch_decode_groups(const DecodeArgs& a, int64_t n_groups, int head_dim, int group,
                                bool fp8, hipStream_t stream);
// lds_pad: dynamic LDS bytes the kernel does not use, reserved so that fewer workgroups share a
// compute unit (room for other kernels' workgroups beside them)
hipError_t launch_prefill(const PrefillArgs& a, int64_t n_items, int head_dim, int group,
                          bool fp8, hipStream_t stream, uint32_t lds_pad = 0);

// Whether a (head_dim, group, dtype) combination has a built decode / prefill kernel.
bool decode_supported(int head_dim, int group);
// Whether a (head_dim, group) combination of bf16 or E4M3 pools has a group-item decode
// kernel, and how many rows its group items hold at most.
bool decode_groups_supported(int head_dim, int group);
int decode_group_rows(int group);
bool decode_fp8_supported(int head_dim, int group);
bool prefill_supported(int head_dim, int group, bool bf16);

}  // namespace pkv
