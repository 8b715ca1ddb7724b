// Host work planner of a ragged attention step: routing of each segment to the decode split
// pass or the prefill tile pass, the work lists of both, and the workspace layout.
//
// Follows the kernel contract of "P3: native paged-KV continuous-batching sampler", section
// "Design > paged.py" (TritonPagedAttention): a flat ragged step described by cu_seqlens_q and
// ctx_lens, a fixed KV split per context length, no atomics. Routing and every item depend only
// on the row's own segment, never on the rest of the step. Pure host C++ (no HIP), so that it
// can be built and exercised on its own.
#pragma once

#include <cstddef>
#include <cstdint>
#include <utility>
#include <vector>

#include "plan.h"

namespace pkv {

struct SharedSplits;

struct StepShape {
  const int32_t* ctx;
  const int32_t* cu;
  int32_t B;
  int32_t kv_split;
  bool prefill_on_mfma;  // segments with q_len > 1 use the prefill kernel
  bool all_mfma;         // phase-consistent mode: every segment (decode rows too) uses it
  int32_t prefill_rows_per_item;
  int32_t tile_split;    // > 0 (phase-consistent mode: kv_split): tile items cover one KV split
  // Shared reads (optional): with a host copy of the block tables and group_rows > 1, a decode
  // split that covers the same physical blocks in several rows (whole splits only) is listed
  // once per group of up to group_rows of those rows instead of once per row.
  const int32_t* bt_host = nullptr;   // [B, bt_stride] host int32, or null
  int32_t bt_stride = 0;
  int32_t block_size = 0;
  int32_t group_rows = 0;
  int32_t hkv = 1;   // kv heads (the group launch runs each item once per kv head)
  const SharedSplits* shared = nullptr;   // find_shared_splits of this shape, when taken
};

// The decode splits read once for several rows: group items, and the (row, split) pairs they
// take from the per-row items (sorted).
struct SharedSplits {
  std::vector<DecodeGroupItem> groups;
  std::vector<std::pair<int32_t, int32_t>> taken;   // (row, split), ascending
  bool contains(int32_t row, int32_t split) const;
};

// Groups the whole decode splits of s that cover the same physical blocks in several rows
// (none without host tables or with group_rows < 2). Rows sharing a split are cut into groups
// of up to group_rows in step order; a last group of one row stays a per-row item. The result
// depends only on which rows share blocks; each row's arithmetic is the same in either kind of
// item.
SharedSplits find_shared_splits(const StepShape& s);

// Workspace regions are aligned to this many bytes.
constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Whether segment b (q_len ql >= 1) runs on the prefill tile kernel.
bool on_tiles(const StepShape& s, int32_t ql);

// Counts and layout only (no lists). n_write_rows > 0 reserves the slot array of a fused KV
// append after the work lists (copied from the host with them).
WorkspaceLayout layout_for(const StepShape& s, int32_t hq, int32_t head_dim,
                           int32_t n_write_rows = 0);

// Writes the work lists of layout L (decode items, decode group items, merge items, prefill
// items) into host memory laid out as the workspace (offsets of L). Items are listed longest
// first.
void build_lists(const StepShape& s, const WorkspaceLayout& L, char* host);

// Validates a step's host metadata: cu[0] == 0, cu non-decreasing, cu[B] == T,
// 0 <= q_len <= ctx_len (<= max_keys when max_keys >= 0). PKV_OK or PKV_ERR_INVALID.
int32_t check_step(const int32_t* ctx, const int32_t* cu, int32_t B, int32_t T,
                   int64_t max_keys);

}  // namespace pkv
