// KV append kernel for gfx950 (MI355X).
//
// Source of the operation: "P3: native paged-KV continuous-batching sampler", section
// "Design > paged.py" (PagedKVCache: copy-free append, a write scatters each new K/V row into
// (block, offset) of the pools in place).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "kernels.h"

namespace pkv {

// ---------------------------------------------------------------------------------------
// KV append: row t of k_new / v_new goes to slot slots[t]; a slot row is contiguous in the
// [num_blocks, block_size, Hkv, D] pool at byte offset slot * Hkv * D * elem_bytes.
// ---------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) write_kv_kernel(WriteArgs a) {
  const uint4* __restrict__ kn = static_cast<const uint4*>(a.k_new);
  const uint4* __restrict__ vn = static_cast<const uint4*>(a.v_new);
  uint4* __restrict__ kc = static_cast<uint4*>(a.k_cache);
  uint4* __restrict__ vc = static_cast<uint4*>(a.v_cache);
  const uint32_t chunks = static_cast<uint32_t>(a.chunks_per_row);
  const uint32_t total = static_cast<uint32_t>(a.n_rows) * chunks;
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < total; i += gridDim.x * 256u) {
    const uint32_t row = i / chunks;
    const uint32_t c = i - row * chunks;
    const int32_t s = a.slots[row];
    if (s < 0 || s >= a.n_slots) continue;
    const int64_t dst = static_cast<int64_t>(s) * chunks + c;
    kc[dst] = kn[i];
    vc[dst] = vn[i];
  }
}

hipError_t launch_write_kv(const WriteArgs& a, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(a.n_rows) * a.chunks_per_row;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(write_kv_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                     a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Block copy (copy-on-write): block pairs[2i + 1] of both pools becomes a byte copy of block
// pairs[2i]. A block is chunks_per_block contiguous 16-byte chunks in either pool.
// ---------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) copy_blocks_kernel(CopyArgs a) {
  uint4* __restrict__ kc = static_cast<uint4*>(a.k_cache);
  uint4* __restrict__ vc = static_cast<uint4*>(a.v_cache);
  const uint32_t chunks = static_cast<uint32_t>(a.chunks_per_block);
  const uint32_t total = static_cast<uint32_t>(a.n_pairs) * chunks;
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < total; i += gridDim.x * 256u) {
    const uint32_t pr = i / chunks;
    const uint32_t c = i - pr * chunks;
    const int64_t src = static_cast<int64_t>(a.pairs[2 * pr]) * chunks + c;
    const int64_t dst = static_cast<int64_t>(a.pairs[2 * pr + 1]) * chunks + c;
    kc[dst] = kc[src];
    vc[dst] = vc[src];
  }
}

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(a.n_pairs) * a.chunks_per_block;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace pkv
