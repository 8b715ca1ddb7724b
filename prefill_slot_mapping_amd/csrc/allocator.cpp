// Host block allocator and slot mapping.
//
// "P3: native paged-KV continuous-batching sampler", section "Design > paged.py":
// BlockAllocator is a LIFO free list plus refcounts; freeing at refcount 0 is an error (a
// double free would hand one block to two sequences); check_consistent proves free +
// referenced == total with no duplicates; slots() refuses a write into a block with
// refcount > 1. "Optional paged KV cache (vLLM-style) — v1 design", section "Design":
// exhaustion is a typed error, never a silent truncation. Multi-id calls are all-or-nothing.
#include <algorithm>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "common.h"

struct pkv_alloc {
  int32_t num_blocks = 0;
  std::vector<int32_t> stack;     // free list; top = back()
  std::vector<int32_t> refcount;  // one per block
};

namespace pkv {

static thread_local std::string g_last_error;

int32_t fail(int32_t status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int32_t ok() {
  g_last_error.clear();
  return PKV_OK;
}

}  // namespace pkv

using pkv::fail;
using pkv::ok;

extern "C" const char* pkv_last_error(void) { return pkv::g_last_error.c_str(); }

extern "C" const char* pkv_version(void) { return "pkv 0.1.0 gfx950"; }

extern "C" int32_t pkv_alloc_create(int32_t num_blocks, pkv_alloc** out) {
  if (out == nullptr) return fail(PKV_ERR_INVALID, "pkv_alloc_create: out is NULL");
  *out = nullptr;
  if (num_blocks < 0) return fail(PKV_ERR_INVALID, "pkv_alloc_create: num_blocks < 0");
  pkv_alloc* a = new (std::nothrow) pkv_alloc();
  if (a == nullptr) return fail(PKV_ERR_INVALID, "pkv_alloc_create: out of host memory");
  a->num_blocks = num_blocks;
  a->stack.resize(num_blocks);
  for (int32_t i = 0; i < num_blocks; ++i) a->stack[i] = num_blocks - 1 - i;  // 0 on top
  a->refcount.assign(num_blocks, 0);
  *out = a;
  return ok();
}

extern "C" void pkv_alloc_destroy(pkv_alloc* a) { delete a; }

static bool in_pool(const pkv_alloc* a, int32_t id) { return id >= 0 && id < a->num_blocks; }

extern "C" int32_t pkv_alloc_allocate(pkv_alloc* a, int32_t n, int32_t* out_ids) {
  if (a == nullptr) return fail(PKV_ERR_INVALID, "allocate: NULL handle");
  if (n < 0) return fail(PKV_ERR_INVALID, "allocate: negative count");
  if (n > 0 && out_ids == nullptr) return fail(PKV_ERR_INVALID, "allocate: out_ids is NULL");
  if (static_cast<size_t>(n) > a->stack.size())
    return fail(PKV_ERR_POOL_EXHAUSTED, "allocate: need " + std::to_string(n) + " blocks, " +
                                            std::to_string(a->stack.size()) + " free");
  for (int32_t i = 0; i < n; ++i) {
    int32_t id = a->stack.back();
    a->stack.pop_back();
    a->refcount[id] = 1;
    out_ids[i] = id;
  }
  return ok();
}

extern "C" int32_t pkv_alloc_incref(pkv_alloc* a, int32_t n, const int32_t* ids) {
  if (a == nullptr) return fail(PKV_ERR_INVALID, "incref: NULL handle");
  if (n < 0 || (n > 0 && ids == nullptr)) return fail(PKV_ERR_INVALID, "incref: bad ids");
  for (int32_t i = 0; i < n; ++i) {
    if (!in_pool(a, ids[i]))
      return fail(PKV_ERR_INVALID, "incref: block id " + std::to_string(ids[i]) + " outside pool");
    if (a->refcount[ids[i]] < 1)
      return fail(PKV_ERR_INVALID, "incref: block " + std::to_string(ids[i]) + " is free");
  }
  for (int32_t i = 0; i < n; ++i) a->refcount[ids[i]] += 1;
  return ok();
}

extern "C" int32_t pkv_alloc_free(pkv_alloc* a, int32_t n, const int32_t* ids) {
  if (a == nullptr) return fail(PKV_ERR_INVALID, "free: NULL handle");
  if (n < 0 || (n > 0 && ids == nullptr)) return fail(PKV_ERR_INVALID, "free: bad ids");
  for (int32_t i = 0; i < n; ++i)
    if (!in_pool(a, ids[i]))
      return fail(PKV_ERR_INVALID, "free: block id " + std::to_string(ids[i]) + " outside pool");
  // all-or-nothing: every id needs at least as many references as it appears in the call
  std::vector<int32_t> sorted(ids, ids + n);
  std::sort(sorted.begin(), sorted.end());
  for (size_t i = 0; i < sorted.size();) {
    size_t j = i;
    while (j < sorted.size() && sorted[j] == sorted[i]) ++j;
    if (a->refcount[sorted[i]] < static_cast<int32_t>(j - i))
      return fail(PKV_ERR_DOUBLE_FREE, "free: block " + std::to_string(sorted[i]) +
                                           " has refcount " +
                                           std::to_string(a->refcount[sorted[i]]));
    i = j;
  }
  for (int32_t i = 0; i < n; ++i) {
    if (--a->refcount[ids[i]] == 0) a->stack.push_back(ids[i]);
  }
  return ok();
}

extern "C" int32_t pkv_alloc_refcount(const pkv_alloc* a, int32_t id) {
  if (a == nullptr) return fail(PKV_ERR_INVALID, "refcount: NULL handle");
  if (!in_pool(a, id)) return fail(PKV_ERR_INVALID, "refcount: id outside pool");
  return a->refcount[id];
}

extern "C" int32_t pkv_alloc_num_free(const pkv_alloc* a) {
  if (a == nullptr) return fail(PKV_ERR_INVALID, "num_free: NULL handle");
  return static_cast<int32_t>(a->stack.size());
}

extern "C" int32_t pkv_alloc_num_blocks(const pkv_alloc* a) {
  if (a == nullptr) return fail(PKV_ERR_INVALID, "num_blocks: NULL handle");
  return a->num_blocks;
}

extern "C" int32_t pkv_alloc_check_consistent(const pkv_alloc* a) {
  if (a == nullptr) return fail(PKV_ERR_INVALID, "check_consistent: NULL handle");
  std::vector<uint8_t> on_stack(a->num_blocks, 0);
  for (int32_t id : a->stack) {
    if (!in_pool(a, id)) return fail(PKV_ERR_INCONSISTENT, "free stack holds an id outside the pool");
    if (on_stack[id]) return fail(PKV_ERR_INCONSISTENT, "block " + std::to_string(id) + " is on the free stack twice");
    on_stack[id] = 1;
    if (a->refcount[id] != 0)
      return fail(PKV_ERR_INCONSISTENT, "free block " + std::to_string(id) + " is referenced");
  }
  int64_t referenced = 0;
  for (int32_t r : a->refcount) {
    if (r < 0) return fail(PKV_ERR_INCONSISTENT, "negative refcount");
    referenced += (r > 0);
  }
  if (static_cast<int64_t>(a->stack.size()) + referenced != a->num_blocks)
    return fail(PKV_ERR_INCONSISTENT, "free + referenced != total");
  return ok();
}

extern "C" int32_t pkv_alloc_snapshot(const pkv_alloc* a, int32_t* free_stack_out,
                                      int32_t* refcounts_out) {
  if (a == nullptr) return fail(PKV_ERR_INVALID, "snapshot: NULL handle");
  if (free_stack_out != nullptr && !a->stack.empty())
    std::memcpy(free_stack_out, a->stack.data(), a->stack.size() * sizeof(int32_t));
  if (refcounts_out != nullptr && a->num_blocks > 0)
    std::memcpy(refcounts_out, a->refcount.data(), a->refcount.size() * sizeof(int32_t));
  return ok();
}

extern "C" int32_t pkv_slot_mapping(const pkv_alloc* a, const int32_t* bt_row, int32_t n_bt,
                                    int32_t block_size, int32_t start_pos, int32_t n_new,
                                    int32_t* slots_out) {
  if (a == nullptr) return fail(PKV_ERR_INVALID, "slot_mapping: NULL handle");
  if (block_size <= 0 || start_pos < 0 || n_new < 0 || n_bt < 0)
    return fail(PKV_ERR_INVALID, "slot_mapping: bad block_size / start_pos / n_new / n_bt");
  if (n_new == 0) return ok();
  if (bt_row == nullptr || slots_out == nullptr)
    return fail(PKV_ERR_INVALID, "slot_mapping: NULL pointer");
  if (static_cast<int64_t>(a->num_blocks) * block_size > INT32_MAX)
    return fail(PKV_ERR_INVALID, "slot_mapping: pool has more slots than an int32 slot can name");
  if (static_cast<int64_t>(start_pos) + n_new > INT32_MAX)
    return fail(PKV_ERR_INVALID, "slot_mapping: position overflow");
  // validate everything first so a refused call writes nothing
  for (int64_t p = start_pos; p < static_cast<int64_t>(start_pos) + n_new; ++p) {
    int64_t j = p / block_size;
    if (j >= n_bt)
      return fail(PKV_ERR_INVALID, "slot_mapping: position " + std::to_string(p) + " past the block table");
    int32_t blk = bt_row[j];
    if (!in_pool(a, blk))
      return fail(PKV_ERR_INVALID, "slot_mapping: block id " + std::to_string(blk) + " outside pool");
    if (a->refcount[blk] == 0)
      return fail(PKV_ERR_INVALID, "slot_mapping: block " + std::to_string(blk) + " is free");
    if (a->refcount[blk] > 1)
      return fail(PKV_ERR_SHARED_WRITE, "slot_mapping: block " + std::to_string(blk) +
                                            " is shared (refcount " +
                                            std::to_string(a->refcount[blk]) + ")");
  }
  for (int32_t i = 0; i < n_new; ++i) {
    int64_t p = static_cast<int64_t>(start_pos) + i;
    int32_t blk = bt_row[p / block_size];
    slots_out[i] = blk * block_size + static_cast<int32_t>(p % block_size);
  }
  return ok();
}

extern "C" int32_t pkv_slot_mapping_step(const pkv_alloc* a, const int32_t* block_tables_host,
                                         int32_t B, int32_t max_blocks, int32_t block_size,
                                         const int32_t* start_pos, const int32_t* n_new,
                                         int32_t* slots_out) {
  if (a == nullptr) return fail(PKV_ERR_INVALID, "slot_mapping_step: NULL handle");
  if (B < 0 || max_blocks < 0) return fail(PKV_ERR_INVALID, "slot_mapping_step: bad B / max_blocks");
  if (B == 0) return ok();
  if (block_tables_host == nullptr || start_pos == nullptr || n_new == nullptr)
    return fail(PKV_ERR_INVALID, "slot_mapping_step: NULL pointer");
  // validation pass: each call below writes only into a scratch copy-free check
  int64_t total = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (n_new[b] < 0 || start_pos[b] < 0) return fail(PKV_ERR_INVALID, "slot_mapping_step: negative n_new / start_pos");
    total += n_new[b];
  }
  if (total > 0 && slots_out == nullptr) return fail(PKV_ERR_INVALID, "slot_mapping_step: slots_out is NULL");
  for (int32_t b = 0; b < B; ++b) {
    const int32_t* row = block_tables_host + static_cast<int64_t>(b) * max_blocks;
    for (int64_t p = start_pos[b]; p < static_cast<int64_t>(start_pos[b]) + n_new[b]; ++p) {
      const int64_t j = p / block_size;
      if (block_size <= 0 || j >= max_blocks)
        return fail(PKV_ERR_INVALID, "slot_mapping_step: sequence " + std::to_string(b) + " position past its table");
      const int32_t blk = row[j];
      if (!in_pool(a, blk) || a->refcount[blk] == 0)
        return fail(PKV_ERR_INVALID, "slot_mapping_step: sequence " + std::to_string(b) + " block " + std::to_string(blk) + " not live");
      if (a->refcount[blk] > 1)
        return fail(PKV_ERR_SHARED_WRITE, "slot_mapping_step: sequence " + std::to_string(b) + " block " + std::to_string(blk) + " is shared");
    }
  }
  int64_t o = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t st = pkv_slot_mapping(a, block_tables_host + static_cast<int64_t>(b) * max_blocks,
                                        max_blocks, block_size, start_pos[b], n_new[b], slots_out + o);
    if (st != PKV_OK) return st;
    o += n_new[b];
  }
  return ok();
}

namespace pkv {

// Every slot negative (skipped) or in [0, num_slots), no non-negative slot twice. Uses a bitmap
// over the slots' range when that is at most 64 bits per slot (one pass, the usual case for a
// step's slots), else a sorted copy. `what` prefixes the message.
int32_t check_slots(const int32_t* slots, int32_t n, int64_t num_slots, const char* what) {
  int32_t lo = INT32_MAX, hi = -1;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = slots[i];
    if (s < 0) continue;
    if (s >= num_slots)
      return fail(PKV_ERR_INVALID, std::string(what) + ": slot " + std::to_string(s) + " outside the pool");
    lo = std::min(lo, s);
    hi = std::max(hi, s);
  }
  if (hi < 0) return PKV_OK;
  const int64_t range = static_cast<int64_t>(hi) - lo + 1;
  int32_t dup = -1;
  if (range <= 64 * static_cast<int64_t>(n)) {
    static thread_local std::vector<uint64_t> bits;
    bits.assign(static_cast<size_t>((range + 63) / 64), 0);
    for (int32_t i = 0; i < n && dup < 0; ++i) {
      const int32_t s = slots[i];
      if (s < 0) continue;
      const int64_t k = static_cast<int64_t>(s) - lo;
      const uint64_t m = uint64_t(1) << (k & 63);
      if (bits[k >> 6] & m) dup = s;
      bits[k >> 6] |= m;
    }
  } else {
    static thread_local std::vector<int32_t> seen;
    seen.clear();
    for (int32_t i = 0; i < n; ++i)
      if (slots[i] >= 0) seen.push_back(slots[i]);
    std::sort(seen.begin(), seen.end());
    auto d = std::adjacent_find(seen.begin(), seen.end());
    if (d != seen.end()) dup = *d;
  }
  if (dup >= 0)
    return fail(PKV_ERR_INVALID, std::string(what) + ": slot " + std::to_string(dup) + " appears twice");
  return PKV_OK;
}

}  // namespace pkv

extern "C" int32_t pkv_validate_slots(const int32_t* slots_host, int32_t n, int64_t num_slots) {
  if (n < 0 || (n > 0 && slots_host == nullptr))
    return fail(PKV_ERR_INVALID, "validate_slots: bad array");
  const int32_t st = pkv::check_slots(slots_host, n, num_slots, "validate_slots");
  if (st != PKV_OK) return st;
  return ok();
}
