// Cache writes: new tokens into their slots, and whole-block copies.
//
// "vLLM 深度解读" (luoboask.github.io), section 7: before attention, each new
// token's K and V rows are stored in place into the paged cache.
// "详解vLLM推理引擎架构：PagedAttention原理与LLM高效部署实践" (tbr8.org),
// section "Copy-on-Write 与内存共享": a block with more than one owner is
// copied into a fresh block before it is written.
//
// Both are pure data movement: one thread per 16-byte chunk, bit-exact, with
// every device-resident index (slot, block id) range-checked before use.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace {

// One thread per 16-byte chunk of one token's [Hkv, D] row.
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, const int64_t* __restrict__ slot_mapping, int64_t n_items,
    int row_chunks, int d_chunks, int num_kv_heads, int block_size, int64_t n_slots) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_items) return;
  const int64_t i = idx / row_chunks;
  const int c = static_cast<int>(idx - i * row_chunks);
  const int64_t slot = slot_mapping[i];
  if (slot < 0 || slot >= n_slots) return;
  const int64_t b = slot / block_size;
  const int o = static_cast<int>(slot - b * block_size);
  const int h = c / d_chunks;
  const int dc = c - h * d_chunks;
  const int64_t dst = ((b * num_kv_heads + h) * block_size + o) * d_chunks + dc;
  k_cache[dst] = key[idx];
  v_cache[dst] = value[idx];
}

// grid.x = pair, grid.y strides over the 16-byte chunks of a block.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ k_cache,
                                                          uint4* __restrict__ v_cache,
                                                          const int64_t* __restrict__ pairs,
                                                          int64_t block_chunks, int num_blocks) {
  const int pr = blockIdx.x;
  const int64_t src = pairs[2 * (int64_t)pr];
  const int64_t dst = pairs[2 * (int64_t)pr + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const uint4* ks = k_cache + src * block_chunks;
  const uint4* vs = v_cache + src * block_chunks;
  uint4* kd = k_cache + dst * block_chunks;
  uint4* vd = v_cache + dst * block_chunks;
  for (int64_t c = (int64_t)blockIdx.y * blockDim.x + threadIdx.x; c < block_chunks;
       c += (int64_t)gridDim.y * blockDim.x) {
    const uint4 kk = ks[c];
    const uint4 vv = vs[c];
    kd[c] = kk;
    vd[c] = vv;
  }
}

}  // namespace

hipError_t launch_reshape_and_cache(const ReshapeLaunch& a) {
  const int d_chunks = a.head_dim * a.elem_bytes / 16;
  const int row_chunks = a.num_kv_heads * d_chunks;
  const int64_t n_items = (int64_t)a.num_tokens * row_chunks;
  const int64_t blocks = (n_items + 255) / 256;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     a.stream, static_cast<const uint4*>(a.key), static_cast<const uint4*>(a.value),
                     static_cast<uint4*>(a.k_cache), static_cast<uint4*>(a.v_cache), a.slot_mapping,
                     n_items, row_chunks, d_chunks, a.num_kv_heads, a.block_size,
                     (int64_t)a.num_blocks * a.block_size);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyLaunch& a) {
  const int64_t block_chunks = (int64_t)a.num_kv_heads * a.block_size * a.head_dim * a.elem_bytes / 16;
  int64_t gy = (block_chunks + 255) / 256;
  if (gy > 64) gy = 64;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(a.num_pairs, static_cast<unsigned>(gy)), dim3(256), 0,
                     a.stream, static_cast<uint4*>(a.k_cache), static_cast<uint4*>(a.v_cache),
                     a.block_pairs, block_chunks, a.num_blocks);
  return hipGetLastError();
}

}  // namespace pa
