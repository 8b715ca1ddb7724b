// Work-list records and workspace layout shared by the host planner and the HIP kernels.
#pragma once

#include <cstddef>
#include <cstdint>

namespace pkv {

// Granularity of kv_split: a multiple of every decode tile (16 or 32 keys) times the waves.
constexpr int kDecodeTile = 64;
// Waves per decode workgroup; tile i of a split is handled by wave i % kDecodeWaves.
constexpr int kDecodeWaves = 4;
// Largest kv_split the decode kernel stages slots for (one int per key of a split in LDS).
constexpr int kMaxDecodeSplit = 2048;
// Keys per prefill KV tile (tiles are aligned at absolute position 0).
constexpr int kPrefillKeyTile = 64;
// Query "M-rows" (query row x head pairs) per prefill workgroup: 4 waves x 32.
constexpr int kPrefillMRows = 128;
// Block-table entries a prefill workgroup holds in LDS at a time.
constexpr int kPrefillBlockWindow = 512;

// One decode work item: split `split` of query row `row` (sequence `seq`), covering keys
// [split * kv_split, min(n_keys, (split + 1) * kv_split)). The kernel grid runs each item once
// per group of (at most 4) query heads.
// part < 0: the row has one split and the kernel writes the final output; otherwise the
// item writes partial slot (part + split) for its heads.
struct DecodeItem {
  int32_t row;
  int32_t seq;
  int32_t n_keys;
  int32_t split;
  int32_t part;
  int32_t pad0, pad1, pad2;
};

// Rows per group item at most.
constexpr int kGroupRows = 4;

// One decode split read once for several rows: split `split` of rows row[0 .. n_rows) (of
// sequences seq[]), whose block tables hold the same physical blocks over the split's keys
// [split * kv_split, (split + 1) * kv_split) and whose contexts cover the whole split (n_keys,
// the smallest of theirs, is at least (split + 1) * kv_split). Each row's arithmetic is that of
// its single-row item; row r writes its output (part[r] < 0) or partial slot part[r] + split.
struct DecodeGroupItem {
  int32_t split;
  int32_t n_rows;
  int32_t n_keys;
  int32_t pad;
  int32_t row[kGroupRows];
  int32_t seq[kGroupRows];
  int32_t part[kGroupRows];
};

// Split merge of one query row: partial slots part .. part + n_splits - 1, in ascending order.
struct MergeItem {
  int32_t row;
  int32_t n_splits;
  int32_t part;
  int32_t pad;
};

// One prefill tile: rows row0 .. row0 + n_rows - 1 of sequence seq, at positions
// pos0 .. pos0 + n_rows - 1. The kernel grid runs items x Hkv. Without a tile split the item
// covers keys [0, pos0 + n_rows); with one (PrefillArgs::tile_split = S > 0) it covers keys
// [split * S, (split + 1) * S) of those, and a row at position pos whose keys reach past split
// 0 (pos >= S) writes partial slot part + (row - row0) * pstride + split instead of its output.
struct PrefillItem {
  int32_t seq;
  int32_t row0;
  int32_t n_rows;
  int32_t pos0;
  int32_t split;
  int32_t part;
  int32_t pstride;
  int32_t pad;
};

// Byte offsets of each region inside the caller's workspace (all 256-byte aligned).
struct WorkspaceLayout {
  size_t decode_off = 0, group_off = 0, merge_off = 0, prefill_off = 0, slots_off = 0,
         part_m_off = 0, part_l_off = 0, part_acc_off = 0, total = 0;
  int64_t n_decode = 0, n_group = 0, n_merge = 0, n_prefill = 0, n_part = 0;
  size_t list_bytes = 0;  // lists (+ fused-append slots): the part copied from the host
};

}  // namespace pkv
