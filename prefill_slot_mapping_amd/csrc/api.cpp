// C ABI of the device path: argument validation, the host work planner, the pinned staging
// ring for work lists, and kernel launches on the caller's stream.
//
// The planner follows the kernel contract of "P3: native paged-KV continuous-batching
// sampler", section "Design > paged.py" (TritonPagedAttention): a flat ragged step described
// by cu_seqlens_q and ctx_lens, with a fixed KV split per context length and no atomics.
// Each query row of sequence b at position pos sees keys 0..pos; a row is "decode" when its
// segment has q_len == 1 and "prefill" otherwise. Routing depends only on the row's own
// segment, so a row's work (and bits) never depend on the rest of the step.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <deque>
#include <atomic>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "common.h"
#include "kernels.h"
#include "plan.h"
#include "planner.h"

using pkv::fail;
using pkv::ok;

namespace {

using pkv::align_up;
using pkv::build_lists;
using pkv::check_step;
using pkv::layout_for;
using pkv::StepShape;

// The kernels move 16-byte vectors through q, the new rows, the pools and the workspace.
bool misaligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool valid_dtype(int32_t dt) { return dt == PKV_F32 || dt == PKV_BF16; }
int elem_bytes(int32_t dt) { return dt == PKV_BF16 ? 2 : 4; }

// ---- pinned staging ring: work lists are built on the host and read by the device ----------
// A ring of pinned buffers per device. Slot n % kRingSlots holds the data of call n until the
// device work that reads it (a host-to-device copy, or the fused append launch, which reads the
// buffer in place through its device mapping) has run; before the host rewrites a slot it
// waits for a fence (an event recorded on the stream of the slot's previous reader) that
// covers that work. Fences are recorded every kFenceEvery calls, not every call: each event
// record costs the stream a few microseconds. A reader left uncovered because its stream was
// not used again before the slot came round is waited for with a device synchronisation.
// All slots live in one pinned arena of kRingSlots equal slots. The arena is allocated by the
// first call on a device and replaced only when a call needs more than a slot holds: then
// every slot's last reader is waited for, and the new slot size is the next power of two at or
// above twice the old one and the request (at least kMinSlotBytes). So a process pays at most
// a few allocations, all before its steps reach their largest size, and none per step after.
constexpr int kRingSlots = 16;
constexpr int kFenceEvery = 4;
constexpr size_t kMinSlotBytes = size_t(1) << 20;

struct Fence {
  hipEvent_t ev;
  hipStream_t stream;
  int64_t covers;  // every call <= covers made on `stream` was enqueued before ev
};

struct DeviceRing {
  std::mutex mu;
  char* host = nullptr;        // pinned arena: kRingSlots slots of slot_cap bytes
  char* dev = nullptr;         // its device mapping (kernels read it in place)
  size_t slot_cap = 0;
  int64_t grows = 0;           // arena (re)allocations so far
  int64_t slot_call[kRingSlots];          // call whose reader last used the slot (-1: none)
  hipStream_t slot_stream[kRingSlots];    // the stream of that reader
  int64_t calls = 0;
  std::deque<Fence> fences;       // in record order
  std::vector<hipEvent_t> spare;  // event objects for reuse
  DeviceRing() {
    for (int i = 0; i < kRingSlots; ++i) {
      slot_call[i] = -1;
      slot_stream[i] = nullptr;
    }
  }
};

std::mutex g_rings_mu;
std::unordered_map<int, DeviceRing*> g_rings;

DeviceRing* ring_for_current_device(int* dev_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  *dev_out = dev;
  std::lock_guard<std::mutex> lk(g_rings_mu);
  auto it = g_rings.find(dev);
  if (it != g_rings.end()) return it->second;
  DeviceRing* r = new DeviceRing();
  g_rings[dev] = r;
  return r;
}

// Returns completed fences at the front of the queue to the spare list.
void drop_completed_fences(DeviceRing* r) {
  while (!r->fences.empty() && hipEventQuery(r->fences.front().ev) == hipSuccess) {
    r->spare.push_back(r->fences.front().ev);
    r->fences.pop_front();
  }
}

// Blocks until the reader of call `call` on `stream` has completed.
hipError_t wait_for_copy(DeviceRing* r, int64_t call, hipStream_t stream) {
  for (const Fence& f : r->fences) {
    if (f.stream == stream && f.covers >= call) {
      hipError_t e = hipEventSynchronize(f.ev);
      if (e != hipSuccess) return e;
      drop_completed_fences(r);
      return hipSuccess;
    }
  }
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return e;
  for (const Fence& f : r->fences) r->spare.push_back(f.ev);
  r->fences.clear();
  return hipSuccess;
}

hipError_t record_fence(DeviceRing* r, hipStream_t stream, int64_t covers) {
  hipEvent_t ev = nullptr;
  if (!r->spare.empty()) {
    ev = r->spare.back();
    r->spare.pop_back();
  } else {
    hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return e;
  }
  hipError_t e = hipEventRecord(ev, stream);
  if (e != hipSuccess) {
    r->spare.push_back(ev);
    return e;
  }
  r->fences.push_back(Fence{ev, stream, covers});
  if (r->fences.size() > 4 * kRingSlots) drop_completed_fences(r);
  return hipSuccess;
}

// Makes every slot of the ring hold at least `bytes` (caller holds r->mu). Waits for every
// slot's last reader before the old arena is released.
hipError_t ring_reserve(DeviceRing* r, size_t bytes) {
  if (bytes <= r->slot_cap && r->host != nullptr) return hipSuccess;
  for (int i = 0; i < kRingSlots; ++i) {
    if (r->slot_call[i] < 0) continue;
    hipError_t e = wait_for_copy(r, r->slot_call[i], r->slot_stream[i]);
    if (e != hipSuccess) return e;
    r->slot_call[i] = -1;
  }
  size_t cap = std::max(kMinSlotBytes, 2 * r->slot_cap);
  while (cap < bytes) cap *= 2;
  if (r->host != nullptr) (void)hipHostFree(r->host);
  r->host = nullptr;
  r->dev = nullptr;
  r->slot_cap = 0;
  void* h = nullptr;
  hipError_t e = hipHostMalloc(&h, cap * kRingSlots, hipHostMallocDefault);
  if (e != hipSuccess) return e;
  void* d = nullptr;
  e = hipHostGetDevicePointer(&d, h, 0);
  if (e != hipSuccess) {
    (void)hipHostFree(h);
    return e;
  }
  r->host = static_cast<char*>(h);
  r->dev = static_cast<char*>(d);
  r->slot_cap = cap;
  r->grows += 1;
  return hipSuccess;
}

// Stages `bytes` of host-built data in the current device's ring (fill(host) writes them) and
// enqueues run(host, dev) on strm, the device work that reads them (through the device mapping
// dev of the staging buffer, or with a copy from host); run returns a status.
// With allow_grow false the ring must already hold `bytes` per slot (no allocation here).
template <typename Fill, typename Run>
int32_t stage_and_run(size_t bytes, hipStream_t strm, const char* what, Fill fill, Run run,
                      bool allow_grow = true) {
  int dev = 0;
  DeviceRing* ring = ring_for_current_device(&dev);
  if (ring == nullptr) return fail(PKV_ERR_HIP, std::string(what) + ": hipGetDevice failed");
  std::lock_guard<std::mutex> lk(ring->mu);
  if (!allow_grow && (ring->host == nullptr || bytes > ring->slot_cap))
    return fail(PKV_ERR_UNSUPPORTED, std::string(what) + ": work lists of " +
                                         std::to_string(bytes) + " bytes exceed a staging slot (" +
                                         std::to_string(ring->slot_cap) + " bytes)");
  hipError_t e = ring_reserve(ring, bytes);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, std::string(what) + ": pinned staging: " + hipGetErrorString(e));
  const int64_t call = ring->calls;
  const int si = static_cast<int>(call % kRingSlots);
  if (ring->slot_call[si] >= 0) {
    e = wait_for_copy(ring, ring->slot_call[si], ring->slot_stream[si]);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, std::string(what) + ": staging wait: " + hipGetErrorString(e));
    ring->slot_call[si] = -1;
  }
  char* host = ring->host + static_cast<size_t>(si) * ring->slot_cap;
  const char* devp = ring->dev + static_cast<size_t>(si) * ring->slot_cap;
  fill(host);
  const int32_t rs = run(static_cast<const char*>(host), devp);
  if (rs != PKV_OK) return rs;
  ring->calls = call + 1;
  ring->slot_call[si] = call;
  ring->slot_stream[si] = strm;
  if (call % kFenceEvery == kFenceEvery - 1) {
    e = record_fence(ring, strm, call);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, std::string(what) + ": fence: " + hipGetErrorString(e));
  }
  return PKV_OK;
}

// Copies `bytes` of host-built data to device memory dst on stream strm through the current
// device's staging ring; fill(host) writes the data into the staging buffer.
template <typename Fill>
int32_t stage_and_copy(void* dst, size_t bytes, hipStream_t strm, const char* what, Fill fill,
                       bool allow_grow = true) {
  return stage_and_run(bytes, strm, what, fill, [&](const char* host, const char*) -> int32_t {
    hipError_t e = hipMemcpyAsync(dst, host, bytes, hipMemcpyHostToDevice, strm);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, std::string(what) + ": list copy: " + hipGetErrorString(e));
    return PKV_OK;
  }, allow_grow);
}

// ---- second stream: a large mixed step's decode pass runs beside its prefill pass -------
// Launched after the prefill pass on one stream, the decode pass cannot start until the last
// prefill workgroup has ended, and the prefill grid leaves more and more compute units idle as
// its shortest items finish. A mixed step with a large prefill grid (more than two workgroups
// per compute unit, so that such a tail exists) and a large decode pass therefore forks: after
// the append, the prefill pass is enqueued first on the caller's stream, then the decode pass
// and its merge on a library-owned stream (one per device, default priority) that waits for
// the caller's stream; the caller's stream waits for them before anything enqueued after the
// call. The decode workgroups then fill compute units as prefill workgroups leave. Below the
// thresholds the two event records and waits cost more than the overlap gains. Enqueueing the
// fork and the join holds a per-device lock, so the events are never re-recorded in between.
// Kernels, work lists and outputs are the same either way, so no output bit depends on it.
// A forked step's prefill pass is two launches of the same kernel: first one round of its
// longest items at one workgroup per compute unit (unused LDS reserved, so that a decode
// workgroup fits beside each: about 220 + 226 registers per SIMD lane), then the rest at full
// occupancy. Measured on the mixed ragged step: 711 against 783 us per step; a first part of
// 81 % or 119 % of a round 727 / 770 us (a part round leaves units idle or adds a tail), two or
// three rounds 731 / 740 us; on the E4M3 mixed step 619-626 against 631-636 us.
constexpr int64_t kForkMinPrefillWgs = 512;
constexpr int64_t kForkMinDecodeWgs = 1024;
constexpr uint32_t kPrefillSharePad = 32768;   // bytes of LDS reserved per prefill workgroup
struct SideStream {
  std::mutex mu;
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  int n_cu = 0;   // compute units of the device
};
std::mutex g_side_mu;
std::unordered_map<int, SideStream*> g_side;

SideStream* side_for_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lk(g_side_mu);
  auto it = g_side.find(dev);
  if (it != g_side.end()) return it->second;
  SideStream* ss = new SideStream();
  if (hipStreamCreateWithFlags(&ss->s, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&ss->fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&ss->join, hipEventDisableTiming) != hipSuccess ||
      hipDeviceGetAttribute(&ss->n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    delete ss;
    return nullptr;
  }
  g_side[dev] = ss;
  return ss;
}

// ---- diagnostics: event pairs around launches -------------------------------------------
struct ProfRecord {
  int kind;
  hipEvent_t a, b;
  int64_t call;   // the attention call (per thread) whose launch it brackets
};
// a drained record: its launch's start and end in ms after the first start of its call
struct ProfDone {
  int kind;
  int64_t call;
  double start, end;
};
std::atomic<int64_t> g_prof_calls{0};
thread_local int64_t t_prof_call = -1;
std::mutex g_prof_mu;
// read without the lock on every launch (the fast path when profiling is off)
std::atomic<bool> g_prof_on{false};
std::atomic<uint32_t> g_prof_kinds{0x1Fu};  // kernel kinds bracketed while profiling is on
std::vector<ProfRecord> g_prof_pending;
std::vector<hipEvent_t> g_prof_free;
constexpr int kProfKinds = 5;  // append, prefill tiles, decode split pass, merge, group items
std::vector<ProfDone> g_prof_done;

hipEvent_t prof_event() {
  if (!g_prof_free.empty()) {
    hipEvent_t e = g_prof_free.back();
    g_prof_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Records the opening event of a launch of `kind`; returns the record index or -1.
int prof_begin(int kind, hipStream_t s) {
  if (!g_prof_on.load(std::memory_order_relaxed) ||
      ((g_prof_kinds.load(std::memory_order_relaxed) >> kind) & 1u) == 0)
    return -1;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  ProfRecord r{kind, prof_event(), prof_event(), t_prof_call};
  if (r.a == nullptr || r.b == nullptr) return -1;
  if (hipEventRecord(r.a, s) != hipSuccess) return -1;
  g_prof_pending.push_back(r);
  return static_cast<int>(g_prof_pending.size()) - 1;
}

void prof_end(int idx, hipStream_t s) {
  if (idx < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  (void)hipEventRecord(g_prof_pending[idx].b, s);
}

// kv_split: a positive multiple of 64, at most 2048 for the split decode pass; the
// phase-consistent mode (tile path only) takes any positive multiple of 64.
int32_t check_heads(int32_t hq, int32_t hkv, int32_t head_dim, int32_t kv_split, int32_t dtype,
                    uint32_t flags) {
  if (!valid_dtype(dtype)) return fail(PKV_ERR_INVALID, "dtype must be PKV_F32 or PKV_BF16");
  if (hq <= 0 || hkv <= 0) return fail(PKV_ERR_INVALID, "head counts must be positive");
  if (hq % hkv != 0) return fail(PKV_ERR_INVALID, "num_q_heads must be a multiple of num_kv_heads");
  const bool tiles_only = (flags & PKV_ATTN_PHASE_CONSISTENT) != 0;
  if (kv_split <= 0 || kv_split % pkv::kDecodeTile != 0 ||
      (!tiles_only && kv_split > pkv::kMaxDecodeSplit))
    return fail(PKV_ERR_INVALID, "kv_split must be a positive multiple of 64, at most 2048 "
                                 "(no upper bound in the phase-consistent mode)");
  if (!pkv::decode_supported(head_dim, hq / hkv))
    return fail(PKV_ERR_UNSUPPORTED, "head_dim must be 64 or 128 and num_q_heads / num_kv_heads "
                                     "one of 1, 2, 4, 8");
  return PKV_OK;
}

int32_t check_flags(uint32_t flags, int32_t hq, int32_t hkv, int32_t head_dim, int32_t dtype) {
  if ((flags & ~static_cast<uint32_t>(PKV_ATTN_PHASE_CONSISTENT)) != 0)
    return fail(PKV_ERR_INVALID, "attention: unknown flag bits");
  if ((flags & PKV_ATTN_PHASE_CONSISTENT) &&
      !pkv::prefill_supported(head_dim, hq / hkv, dtype == PKV_BF16))
    return fail(PKV_ERR_UNSUPPORTED, "attention: the phase-consistent mode runs on bf16 MFMA tiles "
                                     "only (bf16, head_dim 64 or 128)");
  return PKV_OK;
}

StepShape shape_for(const int32_t* ctx, const int32_t* cu, int32_t B, int32_t hq, int32_t hkv,
                    int32_t head_dim, int32_t kv_split, int32_t dtype, uint32_t flags,
                    const int32_t* bt_host = nullptr, int32_t bt_stride = 0,
                    int32_t block_size = 0) {
  StepShape s;
  s.all_mfma = (flags & PKV_ATTN_PHASE_CONSISTENT) != 0;
  s.ctx = ctx;
  s.cu = cu;
  s.B = B;
  s.kv_split = kv_split;
  const int group = hq / hkv;
  s.prefill_on_mfma = pkv::prefill_supported(head_dim, group, dtype == PKV_BF16);
  s.prefill_rows_per_item = pkv::kPrefillMRows / group;
  s.tile_split = s.all_mfma ? kv_split : 0;
  // shared reads: bf16 or E4M3 pools on the split decode pass, groups the group-item kernel
  // serves
  if (bt_host != nullptr && dtype == PKV_BF16 && !s.all_mfma &&
      pkv::decode_groups_supported(head_dim, group)) {
    s.bt_host = bt_host;
    s.bt_stride = bt_stride;
    s.block_size = block_size;
    s.group_rows = pkv::decode_group_rows(group);
    s.hkv = hkv;
  }
  return s;
}

// Validated arguments of a KV append (pkv_write_kv or the append of pkv_write_kv_attention).
int32_t check_write(const void* k_new, const void* v_new, int32_t n_rows, const void* k_cache,
                    const void* v_cache, int32_t num_blocks, int32_t block_size,
                    int32_t num_kv_heads, int32_t head_dim, int32_t dtype, pkv::WriteArgs* a) {
  if (!valid_dtype(dtype)) return fail(PKV_ERR_INVALID, "write_kv: bad dtype");
  if (n_rows < 0 || num_blocks < 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(PKV_ERR_INVALID, "write_kv: bad sizes");
  const int64_t row_bytes = static_cast<int64_t>(num_kv_heads) * head_dim * elem_bytes(dtype);
  if (row_bytes % 16 != 0)
    return fail(PKV_ERR_UNSUPPORTED, "write_kv: num_kv_heads * head_dim * elem_bytes must be a "
                                     "multiple of 16");
  if (n_rows > 0 && (k_new == nullptr || v_new == nullptr || k_cache == nullptr ||
                     v_cache == nullptr))
    return fail(PKV_ERR_INVALID, "write_kv: NULL pointer");
  if (n_rows > 0 && (misaligned16(k_new) || misaligned16(v_new) || misaligned16(k_cache) ||
                     misaligned16(v_cache)))
    return fail(PKV_ERR_INVALID, "write_kv: device pointers must be 16-byte aligned");
  if (static_cast<int64_t>(n_rows) * (row_bytes / 16) > 0xffffffffLL)
    return fail(PKV_ERR_UNSUPPORTED, "write_kv: too many rows in one call");
  a->k_new = k_new;
  a->v_new = v_new;
  a->slots = nullptr;
  a->n_rows = n_rows;
  a->chunks_per_row = static_cast<int32_t>(row_bytes / 16);
  a->n_slots = static_cast<int64_t>(num_blocks) * block_size;
  a->k_cache = const_cast<void*>(k_cache);
  a->v_cache = const_cast<void*>(v_cache);
  return PKV_OK;
}

int32_t launch_write(const pkv::WriteArgs& a, hipStream_t strm) {
  t_prof_call = g_prof_calls.fetch_add(1, std::memory_order_relaxed);
  const int pr = prof_begin(0, strm);
  hipError_t e = pkv::launch_write_kv(a, strm);
  prof_end(pr, strm);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, std::string("write_kv launch: ") + hipGetErrorString(e));
  return PKV_OK;
}

// Validated arguments of an E4M3 append (pkv_write_kv_fp8 or the append of
// pkv_write_kv_attention_fp8).
int32_t check_write_fp8(const void* k_new, const void* v_new, int32_t n_rows,
                        const void* k_cache, const void* v_cache, int32_t num_blocks,
                        int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                        float k_scale, float v_scale, pkv::WriteFp8Args* a) {
  if (n_rows < 0 || num_blocks < 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(PKV_ERR_INVALID, "write_kv_fp8: bad sizes");
  if (!(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return fail(PKV_ERR_INVALID, "write_kv_fp8: scales must be finite and > 0");
  const int64_t row_codes = static_cast<int64_t>(num_kv_heads) * head_dim;
  if (row_codes % 16 != 0)
    return fail(PKV_ERR_UNSUPPORTED, "write_kv_fp8: num_kv_heads * head_dim must be a multiple "
                                     "of 16");
  if (n_rows > 0 && (k_new == nullptr || v_new == nullptr || k_cache == nullptr ||
                     v_cache == nullptr))
    return fail(PKV_ERR_INVALID, "write_kv_fp8: NULL pointer");
  if (n_rows > 0 && (misaligned16(k_new) || misaligned16(v_new) || misaligned16(k_cache) ||
                     misaligned16(v_cache)))
    return fail(PKV_ERR_INVALID, "write_kv_fp8: device pointers must be 16-byte aligned");
  if (static_cast<int64_t>(n_rows) * (row_codes / 16) > 0x7fffffffLL)
    return fail(PKV_ERR_UNSUPPORTED, "write_kv_fp8: too many rows in one call");
  a->k_new = k_new;
  a->v_new = v_new;
  a->slots = nullptr;
  a->n_rows = n_rows;
  a->chunks_per_row = static_cast<int32_t>(row_codes / 16);
  a->n_slots = static_cast<int64_t>(num_blocks) * block_size;
  a->k_inv_scale = 1.0f / k_scale;
  a->v_inv_scale = 1.0f / v_scale;
  a->k_cache = const_cast<void*>(k_cache);
  a->v_cache = const_cast<void*>(v_cache);
  return PKV_OK;
}

int32_t launch_write_fp8(const pkv::WriteFp8Args& a, hipStream_t strm) {
  t_prof_call = g_prof_calls.fetch_add(1, std::memory_order_relaxed);
  const int pr = prof_begin(0, strm);
  hipError_t e = pkv::launch_write_kv_fp8(a, strm);
  prof_end(pr, strm);
  if (e != hipSuccess)
    return fail(PKV_ERR_HIP, std::string("write_kv_fp8 launch: ") + hipGetErrorString(e));
  return PKV_OK;
}

// One attention call, optionally preceded by a KV append whose slots come from host memory
// (wr != nullptr): the slots travel in the same host-to-device copy as the work lists.
int32_t attention_impl(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables_dev, int32_t max_blocks,
                       const int32_t* ctx_lens_host, const int32_t* cu_seqlens_q_host,
                       int32_t B, int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                       int32_t kv_split, int32_t dtype, uint32_t flags, float* out,
                       void* workspace, size_t workspace_bytes, void* stream,
                       pkv::WriteArgs* wr, const int32_t* slots_host,
                       const float* fp8_scales = nullptr, pkv::WriteFp8Args* wr8 = nullptr,
                       bool static_ws = false, const int32_t* block_tables_host = nullptr) {
  // static_ws: the workspace is the library's fixed device scratch (pkv_attention_noalloc):
  // a step that does not fit it, or whose lists do not fit a staging slot, is refused
  // fp8_scales != nullptr: q is bfloat16 and the pools hold E4M3 codes with per-tensor scales
  // {k_scale, v_scale}; rows are routed as for bfloat16 pools, onto the E4M3 kernels
  int32_t st = check_heads(num_q_heads, num_kv_heads, head_dim, kv_split, dtype, flags);
  if (st != PKV_OK) return st;
  st = check_flags(flags, num_q_heads, num_kv_heads, head_dim, dtype);
  if (st != PKV_OK) return st;
  if (fp8_scales != nullptr) {
    if (dtype != PKV_BF16) return fail(PKV_ERR_INVALID, "attention_fp8: q must be bfloat16");
    if (!pkv::decode_fp8_supported(head_dim, num_q_heads / num_kv_heads))
      return fail(PKV_ERR_UNSUPPORTED, "attention_fp8: head_dim 64 or 128 and num_q_heads / "
                                       "num_kv_heads one of 1, 2, 4, 8");
    for (int i = 0; i < 2; ++i)
      if (!(std::isfinite(fp8_scales[i]) && fp8_scales[i] > 0.f))
        return fail(PKV_ERR_INVALID, "attention_fp8: scales must be finite and > 0");
  }
  if (block_size <= 0 || num_blocks <= 0 || max_blocks < 0)
    return fail(PKV_ERR_INVALID, "block_size, num_blocks must be > 0 and max_blocks >= 0");
  if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX)
    return fail(PKV_ERR_UNSUPPORTED, "pool has more slots than int32 can address");
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID, "scale must be finite");
  st = check_step(ctx_lens_host, cu_seqlens_q_host, B, T,
                  static_cast<int64_t>(max_blocks) * block_size);
  if (st != PKV_OK) return st;
  const int32_t n_write = wr != nullptr ? wr->n_rows : (wr8 != nullptr ? wr8->n_rows : 0);
  const int64_t n_slots = wr != nullptr ? wr->n_slots : (wr8 != nullptr ? wr8->n_slots : 0);
  if (n_write > 0) {
    if (slots_host == nullptr) return fail(PKV_ERR_INVALID, "write_kv_attention: slots_host is NULL");
    // range and duplicates: without an order between two rows sent to one slot, the slot's
    // contents after the append would be undefined
    st = pkv::check_slots(slots_host, n_write, n_slots, "write_kv_attention");
    if (st != PKV_OK) return st;
  }
  if (T == 0 && n_write == 0) return ok();
  if (T > 0 && (q == nullptr || k_cache == nullptr || v_cache == nullptr ||
                block_tables_dev == nullptr || out == nullptr))
    return fail(PKV_ERR_INVALID, "attention: NULL device pointer");
  if (T > 0 && (misaligned16(q) || misaligned16(k_cache) || misaligned16(v_cache) ||
                misaligned16(workspace) || (reinterpret_cast<uintptr_t>(out) & 3u) != 0 ||
                (reinterpret_cast<uintptr_t>(block_tables_dev) & 3u) != 0))
    return fail(PKV_ERR_INVALID, "attention: q, pools and workspace must be 16-byte aligned, "
                                 "out and block_tables 4-byte aligned");

  StepShape s = shape_for(ctx_lens_host, cu_seqlens_q_host, B, num_q_heads, num_kv_heads,
                          head_dim, kv_split, dtype, flags, block_tables_host, max_blocks,
                          block_size);
  // the shared splits are found once for the layout and the lists
  pkv::SharedSplits shared;
  if (s.bt_host != nullptr && s.group_rows > 1) {
    shared = pkv::find_shared_splits(s);
    s.shared = &shared;
  }
  const pkv::WorkspaceLayout L = layout_for(s, num_q_heads, head_dim, n_write);
  if (static_ws && L.total > workspace_bytes)
    return fail(PKV_ERR_UNSUPPORTED, "attention_noalloc: the step needs " +
                                         std::to_string(L.total) + " bytes of scratch; the "
                                         "static scratch holds " + std::to_string(workspace_bytes));
  if (workspace_bytes < L.total || (L.total > 0 && workspace == nullptr))
    return fail(PKV_ERR_INVALID, "attention: workspace smaller than the workspace-size query (" +
                                     std::to_string(L.total) + " bytes)");
  if (L.n_decode * num_q_heads > INT32_MAX || L.n_prefill * num_kv_heads > INT32_MAX ||
      L.n_group * num_kv_heads > INT32_MAX)
    return fail(PKV_ERR_UNSUPPORTED, "attention: step too large for one launch");

  hipStream_t strm = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  t_prof_call = g_prof_calls.fetch_add(1, std::memory_order_relaxed);

  // work lists (and fused-append slots) -> pinned staging -> workspace, one async copy ordered
  // before the kernels
  const auto fill = [&](char* host) {
    build_lists(s, L, host);
    if (n_write > 0) std::memcpy(host + L.slots_off, slots_host, sizeof(int32_t) * n_write);
  };
  if (n_write > 0) {
    // one launch copies the work lists (bytes [0, slots_off) of the staging buffer) to the
    // workspace and appends the rows, reading their slots from the staging buffer in place
    st = stage_and_run(L.list_bytes, strm, "write_kv_attention", fill,
                       [&](const char*, const char* dev) -> int32_t {
      pkv::StageArgs sa;
      sa.src = reinterpret_cast<const uint4*>(dev);
      sa.dst = reinterpret_cast<uint4*>(ws);
      sa.n_u4 = static_cast<int32_t>(L.slots_off / 16);
      sa.copy_blocks = static_cast<int32_t>(std::min<size_t>((L.slots_off / 16 + 255) / 256, 64));
      const int32_t* slots_staged = reinterpret_cast<const int32_t*>(dev + L.slots_off);
      const int pr = prof_begin(0, strm);
      hipError_t e;
      if (wr != nullptr) {
        wr->slots = slots_staged;
        e = pkv::launch_stage_write_kv(sa, *wr, strm);
      } else {
        wr8->slots = slots_staged;
        e = pkv::launch_stage_write_kv_fp8(sa, *wr8, strm);
      }
      prof_end(pr, strm);
      if (e != hipSuccess)
        return fail(PKV_ERR_HIP, std::string("write_kv launch: ") + hipGetErrorString(e));
      return PKV_OK;
    });
    if (st != PKV_OK) return st;
  } else if (L.list_bytes > 0) {
    st = stage_and_copy(ws, L.list_bytes, strm, static_ws ? "attention_noalloc" : "attention",
                        fill, !static_ws);
    if (st != PKV_OK) return st;
  }
  if (T == 0) return ok();

  // scores in the base-2 domain: scale * log2(e), times the K scale for E4M3 pools
  const double k_scale = fp8_scales != nullptr ? static_cast<double>(fp8_scales[0]) : 1.0;
  const float scale_log2e =
      static_cast<float>(static_cast<double>(scale) * k_scale * 1.4426950408889634);
  const float v_scale = fp8_scales != nullptr ? fp8_scales[1] : 1.f;
  int32_t bs_log2 = -1;
  for (int sh = 0; sh < 31; ++sh)
    if ((1 << sh) == block_size) bs_log2 = sh;
  const int group = num_q_heads / num_kv_heads;
  float* part_m = reinterpret_cast<float*>(ws + L.part_m_off);
  float* part_l = reinterpret_cast<float*>(ws + L.part_l_off);
  float* part_acc = reinterpret_cast<float*>(ws + L.part_acc_off);

  // a large mixed step forks its decode pass (and merge) onto the second stream
  const bool fork = L.n_prefill * num_kv_heads > kForkMinPrefillWgs &&
                    L.n_decode * num_kv_heads >= kForkMinDecodeWgs;
  // a step with group items and per-row decode items runs the group launch on the second
  // stream beside the per-row launch (joined before the merge): the two launches hold
  // different register budgets, so on one stream the second would wait for the first to drain
  const bool fork_groups = !fork && L.n_group > 0 && L.n_decode > 0;
  SideStream* side = nullptr;
  std::unique_lock<std::mutex> side_lock;
  hipStream_t dstrm = strm;   // per-row decode items (and the merge)
  hipStream_t gstrm = strm;   // group items
  if (fork || fork_groups) {
    side = side_for_current_device();
    if (side == nullptr) return fail(PKV_ERR_HIP, "attention: second stream set-up failed");
    side_lock = std::unique_lock<std::mutex>(side->mu);
    hipError_t e = hipEventRecord(side->fork, strm);
    if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->fork, 0);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, std::string("attention: fork: ") + hipGetErrorString(e));
    gstrm = side->s;
    if (fork) dstrm = side->s;
  }
  // the passes; after a failed launch the join below still runs, so that the caller's stream
  // never runs ahead of work already enqueued on the second stream
  const auto launch_passes = [&]() -> int32_t {
    if (L.n_prefill > 0) {
      pkv::PrefillArgs p;
      p.q = q;
      p.k_cache = k_cache;
      p.v_cache = v_cache;
      p.block_tables = block_tables_dev;
      p.max_blocks = max_blocks;
      p.block_size = block_size;
      p.bs_log2 = bs_log2;
      p.num_blocks = num_blocks;
      p.n_items = static_cast<int32_t>(L.n_prefill);
      p.hq = num_q_heads;
      p.hkv = num_kv_heads;
      p.scale_log2e = std::fabs(scale_log2e);
      p.negate_q = scale < 0.f ? 1 : 0;
      p.v_scale = v_scale;
      p.items = reinterpret_cast<const pkv::PrefillItem*>(ws + L.prefill_off);
      p.out = out;
      p.tile_split = s.tile_split;
      p.part_m = part_m;
      p.part_l = part_l;
      p.part_acc = part_acc;
      const int pr = prof_begin(1, strm);
      // forked step: first one round of the longest items beside the decode pass
      const int64_t n_a = fork && side->n_cu > 0
                              ? std::min<int64_t>(L.n_prefill, side->n_cu / num_kv_heads)
                              : 0;
      const uint32_t pad = kPrefillSharePad;
      hipError_t e = hipSuccess;
      if (n_a > 0) {
        pkv::PrefillArgs pa = p;
        pa.n_items = static_cast<int32_t>(n_a);
        e = pkv::launch_prefill(pa, n_a, head_dim, group, fp8_scales != nullptr, strm, pad);
      }
      if (e == hipSuccess && L.n_prefill > n_a) {
        pkv::PrefillArgs pb = p;
        pb.items = p.items + n_a;
        pb.n_items = static_cast<int32_t>(L.n_prefill - n_a);
        e = pkv::launch_prefill(pb, L.n_prefill - n_a, head_dim, group, fp8_scales != nullptr,
                                strm);
      }
      prof_end(pr, strm);
      if (e != hipSuccess) return fail(PKV_ERR_HIP, std::string("prefill launch: ") + hipGetErrorString(e));
    }
    if (L.n_group > 0) {
      pkv::DecodeArgs d;
      d.q = q;
      d.k_cache = k_cache;
      d.v_cache = v_cache;
      d.block_tables = block_tables_dev;
      d.max_blocks = max_blocks;
      d.block_size = block_size;
      d.bs_log2 = bs_log2;
      d.num_blocks = num_blocks;
      d.hq = num_q_heads;
      d.hkv = num_kv_heads;
      d.kv_split = kv_split;
      d.scale_log2e = scale_log2e;
      d.v_scale = v_scale;
      d.items = nullptr;
      d.groups = reinterpret_cast<const pkv::DecodeGroupItem*>(ws + L.group_off);
      d.group = group;
      d.out = out;
      d.part_m = part_m;
      d.part_l = part_l;
      d.part_acc = part_acc;
      const int pr = prof_begin(4, gstrm);
      hipError_t e =
          pkv::launch_decode_groups(d, L.n_group, head_dim, group, fp8_scales != nullptr, gstrm);
      prof_end(pr, gstrm);
      if (e != hipSuccess) return fail(PKV_ERR_HIP, std::string("decode group launch: ") + hipGetErrorString(e));
    }
    if (L.n_decode > 0) {
      pkv::DecodeArgs d;
      d.q = q;
      d.k_cache = k_cache;
      d.v_cache = v_cache;
      d.block_tables = block_tables_dev;
      d.max_blocks = max_blocks;
      d.block_size = block_size;
      d.bs_log2 = bs_log2;
      d.num_blocks = num_blocks;
      d.hq = num_q_heads;
      d.hkv = num_kv_heads;
      d.kv_split = kv_split;
      d.scale_log2e = scale_log2e;
      d.v_scale = v_scale;
      d.items = reinterpret_cast<const pkv::DecodeItem*>(ws + L.decode_off);
      d.groups = nullptr;
      d.group = group;
      d.out = out;
      d.part_m = part_m;
      d.part_l = part_l;
      d.part_acc = part_acc;
      const int pr = prof_begin(2, dstrm);
      hipError_t e = fp8_scales != nullptr
                         ? pkv::launch_decode_fp8(d, L.n_decode, head_dim, group, dstrm)
                         : pkv::launch_decode(d, L.n_decode, head_dim, group, dtype == PKV_BF16, dstrm);
      prof_end(pr, dstrm);
      if (e != hipSuccess) return fail(PKV_ERR_HIP, std::string("decode launch: ") + hipGetErrorString(e));
    }
    if (fork_groups) {
      // the merge reads the group items' partials
      hipError_t e = hipEventRecord(side->join, gstrm);
      if (e == hipSuccess) e = hipStreamWaitEvent(strm, side->join, 0);
      if (e != hipSuccess) return fail(PKV_ERR_HIP, std::string("attention: join: ") + hipGetErrorString(e));
    }
    if (L.n_merge > 0) {
      pkv::MergeArgs mg;
      mg.items = reinterpret_cast<const pkv::MergeItem*>(ws + L.merge_off);
      mg.hq = num_q_heads;
      mg.n_waves = static_cast<int32_t>(L.n_merge * num_q_heads);
      mg.part_m = part_m;
      mg.part_l = part_l;
      mg.part_acc = part_acc;
      mg.out = out;
      const int pr = prof_begin(3, dstrm);
      hipError_t e = pkv::launch_merge(mg, L.n_merge, head_dim, dstrm);
      prof_end(pr, dstrm);
      if (e != hipSuccess) return fail(PKV_ERR_HIP, std::string("merge launch: ") + hipGetErrorString(e));
    }
    return PKV_OK;
  };
  int32_t rc = launch_passes();
  if (fork_groups && rc != PKV_OK) {
    // a launch failed before the join: the caller's stream still waits for the second stream
    hipError_t e = hipEventRecord(side->join, gstrm);
    if (e == hipSuccess) (void)hipStreamWaitEvent(strm, side->join, 0);
  }
  if (fork) {
    hipError_t e = hipEventRecord(side->join, dstrm);
    if (e == hipSuccess) e = hipStreamWaitEvent(strm, side->join, 0);
    if (e != hipSuccess && rc == PKV_OK)
      rc = fail(PKV_ERR_HIP, std::string("attention: join: ") + hipGetErrorString(e));
  }
  return rc == PKV_OK ? ok() : rc;
}

int32_t workspace_size_impl(const int32_t* ctx_lens_host, const int32_t* cu_seqlens_q_host,
                            int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t kv_split, int32_t dtype, uint32_t flags,
                            int32_t n_write_rows, size_t* bytes, bool fp8 = false,
                            const int32_t* block_tables_host = nullptr, int32_t max_blocks = 0,
                            int32_t block_size = 0) {
  if (bytes == nullptr) return fail(PKV_ERR_INVALID, "workspace_size: bytes is NULL");
  *bytes = 0;
  if (n_write_rows < 0) return fail(PKV_ERR_INVALID, "workspace_size: n_rows must be >= 0");
  int32_t st = check_heads(num_q_heads, num_kv_heads, head_dim, kv_split, dtype, flags);
  if (st != PKV_OK) return st;
  st = check_flags(flags, num_q_heads, num_kv_heads, head_dim, dtype);
  if (st != PKV_OK) return st;
  const int32_t T = (B > 0 && cu_seqlens_q_host != nullptr) ? cu_seqlens_q_host[B] : 0;
  st = check_step(ctx_lens_host, cu_seqlens_q_host, B, T, -1);
  if (st != PKV_OK) return st;
  StepShape s = shape_for(ctx_lens_host, cu_seqlens_q_host, B, num_q_heads, num_kv_heads,
                          head_dim, kv_split, dtype, flags, block_tables_host, max_blocks,
                          block_size);
  if (fp8 && !pkv::decode_fp8_supported(head_dim, num_q_heads / num_kv_heads))
    return fail(PKV_ERR_UNSUPPORTED, "attention_fp8: head_dim 64 or 128 and num_q_heads / "
                                     "num_kv_heads one of 1, 2, 4, 8");
  *bytes = layout_for(s, num_q_heads, head_dim, n_write_rows).total;
  return ok();
}

}  // namespace

namespace pkv {

int32_t staging_setup() {
  int dev = 0;
  DeviceRing* ring = ring_for_current_device(&dev);
  if (ring == nullptr) return fail(PKV_ERR_HIP, "staging set-up: hipGetDevice failed");
  std::lock_guard<std::mutex> lk(ring->mu);
  const hipError_t e = ring_reserve(ring, kMinSlotBytes);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, std::string("staging set-up: ") + hipGetErrorString(e));
  return PKV_OK;
}

int32_t attention_static_scratch(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables_dev, int32_t max_blocks,
                                 const int32_t* ctx_lens_host, const int32_t* cu_seqlens_q_host,
                                 int32_t B, int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 float scale, int32_t kv_split, int32_t dtype, uint32_t flags,
                                 float* out, void* scratch, size_t scratch_bytes, void* stream) {
  return attention_impl(q, k_cache, v_cache, block_tables_dev, max_blocks, ctx_lens_host,
                        cu_seqlens_q_host, B, T, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_blocks, scale, kv_split, dtype, flags, out, scratch, scratch_bytes,
                        stream, nullptr, nullptr, nullptr, nullptr, true);
}

}  // namespace pkv

extern "C" int32_t pkv_write_kv(const void* k_new, const void* v_new, const int32_t* slots_dev,
                                int32_t n_rows, void* k_cache, void* v_cache, int32_t num_blocks,
                                int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                                int32_t dtype, void* stream) {
  pkv::WriteArgs a;
  int32_t st = check_write(k_new, v_new, n_rows, k_cache, v_cache, num_blocks, block_size,
                           num_kv_heads, head_dim, dtype, &a);
  if (st != PKV_OK) return st;
  if (n_rows == 0) return ok();
  if (slots_dev == nullptr) return fail(PKV_ERR_INVALID, "write_kv: NULL pointer");
  a.slots = slots_dev;
  st = launch_write(a, static_cast<hipStream_t>(stream));
  if (st != PKV_OK) return st;
  return ok();
}

extern "C" int32_t pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs_host,
                                   int32_t n_pairs, int32_t num_blocks, int32_t block_size,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dtype) && dtype != PKV_E4M3)
    return fail(PKV_ERR_INVALID, "copy_blocks: dtype must be PKV_F32, PKV_BF16 or PKV_E4M3");
  if (n_pairs < 0 || num_blocks < 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(PKV_ERR_INVALID, "copy_blocks: bad sizes");
  const int64_t block_bytes =
      static_cast<int64_t>(block_size) * num_kv_heads * head_dim *
      (dtype == PKV_E4M3 ? 1 : elem_bytes(dtype));
  if (block_bytes % 16 != 0)
    return fail(PKV_ERR_UNSUPPORTED, "copy_blocks: block bytes must be a multiple of 16");
  if (n_pairs == 0) return ok();
  if (pairs_host == nullptr || k_cache == nullptr || v_cache == nullptr)
    return fail(PKV_ERR_INVALID, "copy_blocks: NULL pointer");
  if (misaligned16(k_cache) || misaligned16(v_cache) || misaligned16(workspace))
    return fail(PKV_ERR_INVALID, "copy_blocks: pools and workspace must be 16-byte aligned");
  if (static_cast<int64_t>(n_pairs) * (block_bytes / 16) > 0xffffffffLL)
    return fail(PKV_ERR_UNSUPPORTED, "copy_blocks: too many chunks in one call");
  const size_t need = align_up(sizeof(int32_t) * 2 * static_cast<size_t>(n_pairs));
  if (workspace == nullptr || workspace_bytes < need)
    return fail(PKV_ERR_INVALID, "copy_blocks: workspace smaller than 8 bytes per pair");
  std::vector<int32_t> dsts, srcs;
  for (int32_t i = 0; i < n_pairs; ++i) {
    const int32_t a = pairs_host[2 * i], b = pairs_host[2 * i + 1];
    if (a < 0 || a >= num_blocks || b < 0 || b >= num_blocks)
      return fail(PKV_ERR_INVALID, "copy_blocks: block id outside the pool");
    srcs.push_back(a);
    dsts.push_back(b);
  }
  std::sort(dsts.begin(), dsts.end());
  std::sort(srcs.begin(), srcs.end());
  if (std::adjacent_find(dsts.begin(), dsts.end()) != dsts.end())
    return fail(PKV_ERR_INVALID, "copy_blocks: a destination block appears twice");
  for (int32_t d : dsts)
    if (std::binary_search(srcs.begin(), srcs.end(), d))
      return fail(PKV_ERR_INVALID, "copy_blocks: a destination block is also a source");
  hipStream_t strm = static_cast<hipStream_t>(stream);
  const size_t bytes = sizeof(int32_t) * 2 * static_cast<size_t>(n_pairs);
  int32_t st = stage_and_copy(workspace, bytes, strm, "copy_blocks",
                              [&](char* host) { std::memcpy(host, pairs_host, bytes); });
  if (st != PKV_OK) return st;
  pkv::CopyArgs c;
  c.k_cache = k_cache;
  c.v_cache = v_cache;
  c.pairs = static_cast<const int32_t*>(workspace);
  c.n_pairs = n_pairs;
  c.chunks_per_block = static_cast<int32_t>(block_bytes / 16);
  hipError_t e = pkv::launch_copy_blocks(c, strm);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, std::string("copy_blocks launch: ") + hipGetErrorString(e));
  return ok();
}

extern "C" int32_t pkv_attention_workspace_size_ex(const int32_t* ctx_lens_host,
                                                   const int32_t* cu_seqlens_q_host, int32_t B,
                                                   int32_t num_q_heads, int32_t num_kv_heads,
                                                   int32_t head_dim, int32_t kv_split,
                                                   int32_t dtype, uint32_t flags, size_t* bytes) {
  return workspace_size_impl(ctx_lens_host, cu_seqlens_q_host, B, num_q_heads, num_kv_heads,
                             head_dim, kv_split, dtype, flags, 0, bytes);
}

extern "C" int32_t pkv_attention_workspace_size(const int32_t* ctx_lens_host,
                                                const int32_t* cu_seqlens_q_host, int32_t B,
                                                int32_t num_q_heads, int32_t num_kv_heads,
                                                int32_t head_dim, int32_t kv_split, int32_t dtype,
                                                size_t* bytes) {
  return pkv_attention_workspace_size_ex(ctx_lens_host, cu_seqlens_q_host, B, num_q_heads,
                                         num_kv_heads, head_dim, kv_split, dtype, 0u, bytes);
}

extern "C" int32_t pkv_write_kv_attention_workspace_size(
    const int32_t* ctx_lens_host, const int32_t* cu_seqlens_q_host, int32_t B,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t kv_split,
    int32_t dtype, uint32_t flags, int32_t n_rows, size_t* bytes) {
  return workspace_size_impl(ctx_lens_host, cu_seqlens_q_host, B, num_q_heads, num_kv_heads,
                             head_dim, kv_split, dtype, flags, n_rows, bytes);
}

extern "C" int32_t pkv_attention_ex(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables_dev, int32_t max_blocks,
                                    const int32_t* ctx_lens_host, const int32_t* cu_seqlens_q_host,
                                    int32_t B, int32_t T, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int32_t num_blocks, float scale, int32_t kv_split,
                                    int32_t dtype, uint32_t flags, float* out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return attention_impl(q, k_cache, v_cache, block_tables_dev, max_blocks, ctx_lens_host,
                        cu_seqlens_q_host, B, T, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_blocks, scale, kv_split, dtype, flags, out, workspace,
                        workspace_bytes, stream, nullptr, nullptr);
}

extern "C" int32_t pkv_attention(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables_dev, int32_t max_blocks,
                                 const int32_t* ctx_lens_host, const int32_t* cu_seqlens_q_host,
                                 int32_t B, int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 float scale, int32_t kv_split, int32_t dtype, float* out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return pkv_attention_ex(q, k_cache, v_cache, block_tables_dev, max_blocks, ctx_lens_host,
                          cu_seqlens_q_host, B, T, num_q_heads, num_kv_heads, head_dim,
                          block_size, num_blocks, scale, kv_split, dtype, 0u, out, workspace,
                          workspace_bytes, stream);
}

extern "C" int32_t pkv_write_kv_attention(
    const void* q, const void* k_new, const void* v_new, const int32_t* slots_host,
    int32_t n_rows, void* k_cache, void* v_cache, const int32_t* block_tables_dev,
    int32_t max_blocks, const int32_t* ctx_lens_host, const int32_t* cu_seqlens_q_host,
    int32_t B, int32_t T, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, float scale, int32_t kv_split, int32_t dtype,
    uint32_t flags, float* out, void* workspace, size_t workspace_bytes, void* stream) {
  pkv::WriteArgs a;
  int32_t st = check_write(k_new, v_new, n_rows, k_cache, v_cache, num_blocks, block_size,
                           num_kv_heads, head_dim, dtype, &a);
  if (st != PKV_OK) return st;
  return attention_impl(q, k_cache, v_cache, block_tables_dev, max_blocks, ctx_lens_host,
                        cu_seqlens_q_host, B, T, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_blocks, scale, kv_split, dtype, flags, out, workspace,
                        workspace_bytes, stream, &a, slots_host);
}

// Host tables for the planner: every read entry in [0, max_blocks) of a row, validated for
// the rows' whole contexts (the device tables are the ones the kernels read).
static int32_t check_host_tables(const int32_t* bt, int32_t max_blocks, int32_t block_size,
                                 const int32_t* ctx, int32_t B) {
  if (B > 0 && bt == nullptr) return fail(PKV_ERR_INVALID, "block_tables_host is NULL");
  if (max_blocks < 0 || block_size <= 0)
    return fail(PKV_ERR_INVALID, "max_blocks must be >= 0 and block_size > 0");
  for (int32_t b = 0; b < B; ++b)
    if (ctx[b] > static_cast<int64_t>(max_blocks) * block_size)
      return fail(PKV_ERR_INVALID, "sequence " + std::to_string(b) +
                                       ": ctx_len exceeds max_blocks * block_size");
  return PKV_OK;
}

extern "C" int32_t pkv_write_kv_attention_shared_workspace_size(
    const int32_t* ctx_lens_host, const int32_t* cu_seqlens_q_host, int32_t B,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t kv_split,
    int32_t dtype, uint32_t flags, int32_t n_rows, const int32_t* block_tables_host,
    int32_t max_blocks, int32_t block_size, size_t* bytes) {
  if (bytes != nullptr) *bytes = 0;
  if (B > 0 && ctx_lens_host != nullptr) {
    const int32_t st = check_host_tables(block_tables_host, max_blocks, block_size,
                                         ctx_lens_host, B);
    if (st != PKV_OK) return st;
  }
  return workspace_size_impl(ctx_lens_host, cu_seqlens_q_host, B, num_q_heads, num_kv_heads,
                             head_dim, kv_split, dtype, flags, n_rows, bytes, false,
                             block_tables_host, max_blocks, block_size);
}

extern "C" int32_t pkv_write_kv_attention_shared(
    const void* q, const void* k_new, const void* v_new, const int32_t* slots_host,
    int32_t n_rows, void* k_cache, void* v_cache, const int32_t* block_tables_dev,
    const int32_t* block_tables_host, int32_t max_blocks, const int32_t* ctx_lens_host,
    const int32_t* cu_seqlens_q_host, int32_t B, int32_t T, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    int32_t kv_split, int32_t dtype, uint32_t flags, float* out, void* workspace,
    size_t workspace_bytes, void* stream) {
  pkv::WriteArgs a;
  int32_t st = check_write(k_new, v_new, n_rows, k_cache, v_cache, num_blocks, block_size,
                           num_kv_heads, head_dim, dtype, &a);
  if (st != PKV_OK) return st;
  if (B > 0 && ctx_lens_host != nullptr) {
    st = check_host_tables(block_tables_host, max_blocks, block_size, ctx_lens_host, B);
    if (st != PKV_OK) return st;
  }
  return attention_impl(q, k_cache, v_cache, block_tables_dev, max_blocks, ctx_lens_host,
                        cu_seqlens_q_host, B, T, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_blocks, scale, kv_split, dtype, flags, out, workspace,
                        workspace_bytes, stream, &a, slots_host, nullptr, nullptr, false,
                        block_tables_host);
}

extern "C" int32_t pkv_write_kv_fp8(const void* k_new, const void* v_new,
                                    const int32_t* slots_dev, int32_t n_rows, void* k_cache,
                                    void* v_cache, int32_t num_blocks, int32_t block_size,
                                    int32_t num_kv_heads, int32_t head_dim, float k_scale,
                                    float v_scale, void* stream) {
  pkv::WriteFp8Args a;
  int32_t st = check_write_fp8(k_new, v_new, n_rows, k_cache, v_cache, num_blocks, block_size,
                               num_kv_heads, head_dim, k_scale, v_scale, &a);
  if (st != PKV_OK) return st;
  if (n_rows == 0) return ok();
  if (slots_dev == nullptr) return fail(PKV_ERR_INVALID, "write_kv_fp8: NULL pointer");
  a.slots = slots_dev;
  st = launch_write_fp8(a, static_cast<hipStream_t>(stream));
  if (st != PKV_OK) return st;
  return ok();
}

extern "C" int32_t pkv_attention_fp8_workspace_size(const int32_t* ctx_lens_host,
                                                    const int32_t* cu_seqlens_q_host,
                                                    int32_t B, int32_t num_q_heads,
                                                    int32_t num_kv_heads, int32_t head_dim,
                                                    int32_t kv_split, uint32_t flags,
                                                    size_t* bytes) {
  return workspace_size_impl(ctx_lens_host, cu_seqlens_q_host, B, num_q_heads, num_kv_heads,
                             head_dim, kv_split, PKV_BF16, flags, 0, bytes, true);
}

extern "C" int32_t pkv_attention_fp8(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables_dev, int32_t max_blocks,
                                     const int32_t* ctx_lens_host,
                                     const int32_t* cu_seqlens_q_host, int32_t B, int32_t T,
                                     int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                     float scale, float k_scale, float v_scale,
                                     int32_t kv_split, uint32_t flags, float* out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  const float scales[2] = {k_scale, v_scale};
  return attention_impl(q, k_cache, v_cache, block_tables_dev, max_blocks, ctx_lens_host,
                        cu_seqlens_q_host, B, T, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_blocks, scale, kv_split, PKV_BF16, flags, out, workspace,
                        workspace_bytes, stream, nullptr, nullptr, scales);
}

extern "C" int32_t pkv_write_kv_attention_fp8_workspace_size(
    const int32_t* ctx_lens_host, const int32_t* cu_seqlens_q_host, int32_t B,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t kv_split,
    uint32_t flags, int32_t n_rows, size_t* bytes) {
  return workspace_size_impl(ctx_lens_host, cu_seqlens_q_host, B, num_q_heads, num_kv_heads,
                             head_dim, kv_split, PKV_BF16, flags, n_rows, bytes, true);
}

extern "C" int32_t pkv_write_kv_attention_fp8(
    const void* q, const void* k_new, const void* v_new, const int32_t* slots_host,
    int32_t n_rows, void* k_cache, void* v_cache, const int32_t* block_tables_dev,
    int32_t max_blocks, const int32_t* ctx_lens_host, const int32_t* cu_seqlens_q_host,
    int32_t B, int32_t T, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, float scale, float k_scale, float v_scale,
    int32_t kv_split, uint32_t flags, float* out, void* workspace, size_t workspace_bytes,
    void* stream) {
  pkv::WriteFp8Args a;
  int32_t st = check_write_fp8(k_new, v_new, n_rows, k_cache, v_cache, num_blocks, block_size,
                               num_kv_heads, head_dim, k_scale, v_scale, &a);
  if (st != PKV_OK) return st;
  const float scales[2] = {k_scale, v_scale};
  return attention_impl(q, k_cache, v_cache, block_tables_dev, max_blocks, ctx_lens_host,
                        cu_seqlens_q_host, B, T, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_blocks, scale, kv_split, PKV_BF16, flags, out, workspace,
                        workspace_bytes, stream, nullptr, slots_host, scales, &a);
}

extern "C" int32_t pkv_write_kv_attention_shared_fp8_workspace_size(
    const int32_t* ctx_lens_host, const int32_t* cu_seqlens_q_host, int32_t B,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t kv_split,
    uint32_t flags, int32_t n_rows, const int32_t* block_tables_host, int32_t max_blocks,
    int32_t block_size, size_t* bytes) {
  if (bytes != nullptr) *bytes = 0;
  if (B > 0 && ctx_lens_host != nullptr) {
    const int32_t st = check_host_tables(block_tables_host, max_blocks, block_size,
                                         ctx_lens_host, B);
    if (st != PKV_OK) return st;
  }
  return workspace_size_impl(ctx_lens_host, cu_seqlens_q_host, B, num_q_heads, num_kv_heads,
                             head_dim, kv_split, PKV_BF16, flags, n_rows, bytes, true,
                             block_tables_host, max_blocks, block_size);
}

extern "C" int32_t pkv_write_kv_attention_shared_fp8(
    const void* q, const void* k_new, const void* v_new, const int32_t* slots_host,
    int32_t n_rows, void* k_cache, void* v_cache, const int32_t* block_tables_dev,
    const int32_t* block_tables_host, int32_t max_blocks, const int32_t* ctx_lens_host,
    const int32_t* cu_seqlens_q_host, int32_t B, int32_t T, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    float k_scale, float v_scale, int32_t kv_split, uint32_t flags, float* out, void* workspace,
    size_t workspace_bytes, void* stream) {
  pkv::WriteFp8Args a;
  int32_t st = check_write_fp8(k_new, v_new, n_rows, k_cache, v_cache, num_blocks, block_size,
                               num_kv_heads, head_dim, k_scale, v_scale, &a);
  if (st != PKV_OK) return st;
  if (B > 0 && ctx_lens_host != nullptr) {
    st = check_host_tables(block_tables_host, max_blocks, block_size, ctx_lens_host, B);
    if (st != PKV_OK) return st;
  }
  const float scales[2] = {k_scale, v_scale};
  return attention_impl(q, k_cache, v_cache, block_tables_dev, max_blocks, ctx_lens_host,
                        cu_seqlens_q_host, B, T, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_blocks, scale, kv_split, PKV_BF16, flags, out, workspace,
                        workspace_bytes, stream, nullptr, slots_host, scales, &a, false,
                        block_tables_host);
}

extern "C" int32_t pkv_profile_set_kinds(uint32_t kinds) {
  if ((kinds & ~0x1Fu) != 0) return fail(PKV_ERR_INVALID, "profile_set_kinds: unknown kind bits");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_kinds.store(kinds, std::memory_order_relaxed);
  return ok();
}

extern "C" int32_t pkv_profile_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (enable) {
    for (auto& r : g_prof_pending) {
      (void)hipEventSynchronize(r.b);
      g_prof_free.push_back(r.a);
      g_prof_free.push_back(r.b);
    }
    g_prof_pending.clear();
    g_prof_done.clear();
  }
  g_prof_on.store(enable != 0, std::memory_order_relaxed);
  return ok();
}

// Waits for the pending records and turns them into ProfDone entries (times relative to the
// first start of each call: launches of one call may run on two streams). Caller holds the
// lock.
static int32_t prof_drain(const char* what) {
  size_t i0 = 0;
  while (i0 < g_prof_pending.size()) {
    size_t i1 = i0 + 1;   // records of one call are contiguous (one thread enqueues a call)
    while (i1 < g_prof_pending.size() && g_prof_pending[i1].call == g_prof_pending[i0].call) ++i1;
    const hipEvent_t ref = g_prof_pending[i0].a;
    for (size_t i = i0; i < i1; ++i) {
      const ProfRecord& r = g_prof_pending[i];
      hipError_t e = hipEventSynchronize(r.b);
      float s_ms = 0.f, e_ms = 0.f;
      if (e == hipSuccess) e = hipEventElapsedTime(&s_ms, ref, r.a);
      if (e == hipSuccess) e = hipEventElapsedTime(&e_ms, ref, r.b);
      if (e != hipSuccess) return fail(PKV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
      g_prof_done.push_back(ProfDone{r.kind, r.call, s_ms, e_ms});
    }
    i0 = i1;
  }
  for (auto& r : g_prof_pending) {
    g_prof_free.push_back(r.a);
    g_prof_free.push_back(r.b);
  }
  g_prof_pending.clear();
  return PKV_OK;
}

extern "C" int32_t pkv_profile_read(int32_t kernel_kind, double* total_ms, int64_t* launches) {
  if (kernel_kind < 0 || kernel_kind >= kProfKinds || total_ms == nullptr || launches == nullptr)
    return fail(PKV_ERR_INVALID, "profile_read: bad arguments");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  const int32_t st = prof_drain("profile_read");
  if (st != PKV_OK) return st;
  double ms = 0.0;
  int64_t n = 0;
  for (const ProfDone& d : g_prof_done)
    if (d.kind == kernel_kind) {
      ms += d.end - d.start;
      n += 1;
    }
  *total_ms = ms;
  *launches = n;
  return ok();
}

extern "C" int32_t pkv_profile_read_span(uint32_t kinds, double* total_ms, int64_t* calls) {
  if ((kinds & ~0x1Fu) != 0 || kinds == 0 || total_ms == nullptr || calls == nullptr)
    return fail(PKV_ERR_INVALID, "profile_read_span: bad arguments");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  const int32_t st = prof_drain("profile_read_span");
  if (st != PKV_OK) return st;
  double ms = 0.0;
  int64_t n = 0;
  size_t i0 = 0;
  while (i0 < g_prof_done.size()) {
    size_t i1 = i0 + 1;
    while (i1 < g_prof_done.size() && g_prof_done[i1].call == g_prof_done[i0].call) ++i1;
    double lo = 0.0, hi = 0.0;
    bool any = false;
    for (size_t i = i0; i < i1; ++i) {
      const ProfDone& d = g_prof_done[i];
      if (((kinds >> d.kind) & 1u) == 0) continue;
      lo = any ? std::min(lo, d.start) : d.start;
      hi = any ? std::max(hi, d.end) : d.end;
      any = true;
    }
    if (any) {
      ms += hi - lo;
      n += 1;
    }
    i0 = i1;
  }
  *total_ms = ms;
  *calls = n;
  return ok();
}

extern "C" int32_t pkv_staging_info(size_t* slot_bytes, int64_t* allocations) {
  int dev = 0;
  DeviceRing* ring = ring_for_current_device(&dev);
  if (ring == nullptr) return fail(PKV_ERR_HIP, "staging_info: hipGetDevice failed");
  std::lock_guard<std::mutex> lk(ring->mu);
  if (slot_bytes != nullptr) *slot_bytes = ring->slot_cap;
  if (allocations != nullptr) *allocations = ring->grows;
  return ok();
}
