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
__device__ __forceinline__ void write_kv_chunks(const WriteArgs& a, uint32_t first,
                                                uint32_t stride) {
  const uint4* __restrict__ kn = static_cast<const uint4*>(a.k_new);
  const uint4* __restrict__ vn = static_cast<const uint4*>(a.v_new);
  uint4* __restrict__ kc = static_cast<uint4*>(a.k_cache);
  uint4* __restrict__ vc = static_cast<uint4*>(a.v_cache);
  const uint32_t chunks = static_cast<uint32_t>(a.chunks_per_row);
  const uint32_t total = static_cast<uint32_t>(a.n_rows) * chunks;
  for (uint32_t i = first; i < total; i += stride) {
    const uint32_t row = i / chunks;
    const uint32_t c = i - row * chunks;
    const int32_t s = a.slots[row];
    if (s < 0 || s >= a.n_slots) continue;
    const int64_t dst = static_cast<int64_t>(s) * chunks + c;
    kc[dst] = kn[i];
    vc[dst] = vn[i];
  }
}

__global__ void __launch_bounds__(256) write_kv_kernel(WriteArgs a) {
  write_kv_chunks(a, blockIdx.x * 256u + threadIdx.x, gridDim.x * 256u);
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
// KV append into E4M3 pools: each bfloat16 element x of a new row is stored as the E4M3 code
// of float32(x * inv_scale) (one float32 multiply), clamped to +-448 before the hardware
// conversion (round to nearest, ties to even), so magnitudes beyond the E4M3 range saturate.
// A thread writes 16 codes (one 16-byte chunk of a pool row) from 32 bytes of the new row.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t quant4(uint32_t b01, uint32_t b23, float inv) {
  const float x0 = fminf(fmaxf(__uint_as_float(b01 << 16) * inv, -448.f), 448.f);
  const float x1 = fminf(fmaxf(__uint_as_float(b01 & 0xffff0000u) * inv, -448.f), 448.f);
  const float x2 = fminf(fmaxf(__uint_as_float(b23 << 16) * inv, -448.f), 448.f);
  const float x3 = fminf(fmaxf(__uint_as_float(b23 & 0xffff0000u) * inv, -448.f), 448.f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  return static_cast<uint32_t>(w);
}

__device__ __forceinline__ uint4 quant16(uint4 lo, uint4 hi, float inv) {
  return make_uint4(quant4(lo.x, lo.y, inv), quant4(lo.z, lo.w, inv), quant4(hi.x, hi.y, inv),
                    quant4(hi.z, hi.w, inv));
}

__device__ __forceinline__ void write_kv_fp8_chunks(const WriteFp8Args& a, uint32_t first,
                                                    uint32_t stride) {
  const uint4* __restrict__ kn = static_cast<const uint4*>(a.k_new);
  const uint4* __restrict__ vn = static_cast<const uint4*>(a.v_new);
  uint4* __restrict__ kc = static_cast<uint4*>(a.k_cache);
  uint4* __restrict__ vc = static_cast<uint4*>(a.v_cache);
  const uint32_t chunks = static_cast<uint32_t>(a.chunks_per_row);
  const uint32_t total = static_cast<uint32_t>(a.n_rows) * chunks;
  for (uint32_t i = first; i < total; i += stride) {
    const uint32_t row = i / chunks;
    const uint32_t c = i - row * chunks;
    const int32_t s = a.slots[row];
    if (s < 0 || s >= a.n_slots) continue;
    const int64_t dst = static_cast<int64_t>(s) * chunks + c;
    kc[dst] = quant16(kn[2 * i], kn[2 * i + 1], a.k_inv_scale);
    vc[dst] = quant16(vn[2 * i], vn[2 * i + 1], a.v_inv_scale);
  }
}

__global__ void __launch_bounds__(256) write_kv_fp8_kernel(WriteFp8Args a) {
  write_kv_fp8_chunks(a, blockIdx.x * 256u + threadIdx.x, gridDim.x * 256u);
}

// ---------------------------------------------------------------------------------------
// Fused staging + append: blocks [0, copy_blocks) copy the step's work lists from the pinned
// staging buffer (read through its device mapping) into the workspace; the other blocks
// scatter the new rows, reading each row's slot from the same staging buffer. One launch
// instead of a host-to-device copy followed by the append.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ bool stage_copy(const StageArgs& st) {
  if (static_cast<int32_t>(blockIdx.x) >= st.copy_blocks) return false;
  const uint32_t stride = static_cast<uint32_t>(st.copy_blocks) * 256u;
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < static_cast<uint32_t>(st.n_u4);
       i += stride)
    st.dst[i] = st.src[i];
  return true;
}

__global__ void __launch_bounds__(256) stage_write_kv_kernel(StageArgs st, WriteArgs a) {
  if (stage_copy(st)) return;
  const uint32_t b = blockIdx.x - static_cast<uint32_t>(st.copy_blocks);
  write_kv_chunks(a, b * 256u + threadIdx.x, (gridDim.x - st.copy_blocks) * 256u);
}

__global__ void __launch_bounds__(256) stage_write_kv_fp8_kernel(StageArgs st, WriteFp8Args a) {
  if (stage_copy(st)) return;
  const uint32_t b = blockIdx.x - static_cast<uint32_t>(st.copy_blocks);
  write_kv_fp8_chunks(a, b * 256u + threadIdx.x, (gridDim.x - st.copy_blocks) * 256u);
}

static uint32_t append_blocks(int64_t total) {
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  return static_cast<uint32_t>(blocks < 1 ? 1 : blocks);
}

hipError_t launch_stage_write_kv(const StageArgs& st, const WriteArgs& a, hipStream_t stream) {
  const uint32_t nb = append_blocks(static_cast<int64_t>(a.n_rows) * a.chunks_per_row);
  hipLaunchKernelGGL(stage_write_kv_kernel, dim3(st.copy_blocks + nb), dim3(256), 0, stream, st,
                     a);
  return hipGetLastError();
}

hipError_t launch_stage_write_kv_fp8(const StageArgs& st, const WriteFp8Args& a,
                                     hipStream_t stream) {
  const uint32_t nb = append_blocks(static_cast<int64_t>(a.n_rows) * a.chunks_per_row);
  hipLaunchKernelGGL(stage_write_kv_fp8_kernel, dim3(st.copy_blocks + nb), dim3(256), 0, stream,
                     st, a);
  return hipGetLastError();
}

hipError_t launch_write_kv_fp8(const WriteFp8Args& a, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(a.n_rows) * a.chunks_per_row;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(write_kv_fp8_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                     stream, a);
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
