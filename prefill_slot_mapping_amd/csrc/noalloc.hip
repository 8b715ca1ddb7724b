// pkv_attention_noalloc: pkv_attention_ex with the library's own device scratch in place of
// the caller's workspace, for callers that cannot allocate device memory during a call (code
// under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The scratch is one file-scope device array per GPU (each GPU the library runs on holds its
// copy until the process ends). Host code never passes the array's name to a kernel: in host
// code that name is only a host-side stand-in. Set-up takes the array's device address with
// hipGetSymbolAddress once per device (on the first call made with that device current) and
// every later call uses that address, as the workspace of the unchanged attention path: work
// lists staged from the host first, then the split partials. Set-up also makes sure the
// device's pinned staging ring exists; after set-up a call allocates nothing.
// Nothing in the scratch needs to start at zero: each call writes its lists before any kernel
// reads them, and every partial before the merge reads it.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>
#include <unordered_map>

#include "common.h"

namespace pkv {
int32_t staging_setup();
int32_t attention_static_scratch(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables_dev, int32_t max_blocks,
                                 const int32_t* ctx_lens_host, const int32_t* cu_seqlens_q_host,
                                 int32_t B, int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 float scale, int32_t kv_split, int32_t dtype, uint32_t flags,
                                 float* out, void* scratch, size_t scratch_bytes, void* stream);
}  // namespace pkv

namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(PKV_NOALLOC_SCRATCH_BYTES);

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::unordered_map<int, void*> g_scratch_ptr;   // device -> address of its scratch copy

// The current device's scratch address, taken once per device; nullptr after a failure
// (the message is set).
void* scratch_for_current_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    pkv::fail(PKV_ERR_HIP, std::string("attention_noalloc: hipGetDevice: ") + hipGetErrorString(e));
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) return it->second;
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || ptr == nullptr) {
    pkv::fail(PKV_ERR_HIP, std::string("attention_noalloc: scratch address: ") +
                               hipGetErrorString(e));
    return nullptr;
  }
  if (pkv::staging_setup() != PKV_OK) return nullptr;
  g_scratch_ptr[dev] = ptr;
  return ptr;
}

}  // namespace

extern "C" int32_t pkv_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* block_tables_dev, int32_t max_blocks,
                                         const int32_t* ctx_lens_host,
                                         const int32_t* cu_seqlens_q_host, int32_t B, int32_t T,
                                         int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size,
                                         int32_t num_blocks, float scale, int32_t kv_split,
                                         int32_t dtype, uint32_t flags, float* out,
                                         void* stream) {
  void* ptr = scratch_for_current_device();
  if (ptr == nullptr) return PKV_ERR_HIP;
  return pkv::attention_static_scratch(q, k_cache, v_cache, block_tables_dev, max_blocks,
                                       ctx_lens_host, cu_seqlens_q_host, B, T, num_q_heads,
                                       num_kv_heads, head_dim, block_size, num_blocks, scale,
                                       kv_split, dtype, flags, out, ptr, kScratchBytes, stream);
}
