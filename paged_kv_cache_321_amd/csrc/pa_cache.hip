// Cache writes: new tokens into their slots, and whole-block copies.
//
// "vLLM 深度解读" (luoboask.github.io), section 7: before attention, each new
// token's K and V rows are stored in place into the paged cache.
// "详解vLLM推理引擎架构：PagedAttention原理与LLM高效部署实践" (tbr8.org),
// section "Copy-on-Write 与内存共享": a block with more than one owner is
// copied into a fresh block before it is written.
//
// Both are data movement: one thread per 16-byte chunk, bit-exact, with every
// device-resident index (slot, block id) range-checked before use.  Into an
// fp8 (E4M3) cache the new rows are encoded on the way (see
// reshape_and_cache_fp8_kernel).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.h"

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

// fp8 cache: one thread per 16 codes of one token's [Hkv, D] row; each element
// x becomes f32_to_e4m3(x * inv_scale) (binary32 multiply, then the nearest
// E4M3 code, ties to even, saturating at 448).
template <typename TS>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const TS* __restrict__ key, const TS* __restrict__ value, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, const int64_t* __restrict__ slot_mapping, int64_t n_items,
    int row_chunks, int d_chunks, int num_kv_heads, int block_size, int64_t n_slots, float k_inv,
    float v_inv) {
  constexpr int QV = Elem<TS>::kVec;  // source elements per 16-byte load
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
  auto encode16 = [&](const TS* src, float inv) {
    float f[16];
#pragma unroll
    for (int j = 0; j < 16 / QV; ++j) Elem<TS>::unpack(*reinterpret_cast<const uint4*>(src + j * QV), f + j * QV);
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = f32_to_e4m3(f[4 * j] * inv) | (f32_to_e4m3(f[4 * j + 1] * inv) << 8) |
             (f32_to_e4m3(f[4 * j + 2] * inv) << 16) | (f32_to_e4m3(f[4 * j + 3] * inv) << 24);
    return make_uint4(w[0], w[1], w[2], w[3]);
  };
  const int64_t src = idx * 16;  // element offset of this chunk in [T, Hkv, D]
  k_cache[dst] = encode16(key + src, k_inv);
  v_cache[dst] = encode16(value + src, v_inv);
}

// Whole-block copies from one pool to another (or within one pool): grid.x
// = pair, grid.y strides over the 16-byte chunks of a block.  Either pool may
// be pinned host memory, which the kernel reads or writes through its unified
// address (a swap to or from host memory).
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* dst_k, uint4* dst_v, const uint4* src_k,
                                                          const uint4* src_v,
                                                          const int64_t* __restrict__ pairs,
                                                          int64_t block_chunks, int num_src_blocks,
                                                          int num_dst_blocks) {
  const int pr = blockIdx.x;
  const int64_t src = pairs[2 * (int64_t)pr];
  const int64_t dst = pairs[2 * (int64_t)pr + 1];
  if (src < 0 || src >= num_src_blocks || dst < 0 || dst >= num_dst_blocks) return;
  const uint4* ks = src_k + src * block_chunks;
  const uint4* vs = src_v + src * block_chunks;
  uint4* kd = dst_k + dst * block_chunks;
  uint4* vd = dst_v + dst * block_chunks;
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
  const int64_t n_slots = (int64_t)a.num_blocks * a.block_size;
  if (a.cache_dtype == kDtypeFp8) {
    const int d_chunks = a.head_dim / 16;
    const int row_chunks = a.num_kv_heads * d_chunks;
    const int64_t n_items = (int64_t)a.num_tokens * row_chunks;
    const dim3 grid(static_cast<unsigned>((n_items + 255) / 256));
    uint4* kc = static_cast<uint4*>(a.k_cache);
    uint4* vc = static_cast<uint4*>(a.v_cache);
    if (a.dtype == kDtypeF32)
      hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<float>, grid, dim3(256), 0, a.stream,
                         static_cast<const float*>(a.key), static_cast<const float*>(a.value), kc, vc,
                         a.slot_mapping, n_items, row_chunks, d_chunks, a.num_kv_heads, a.block_size,
                         n_slots, a.k_inv_scale, a.v_inv_scale);
    else
      hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<uint16_t>, grid, dim3(256), 0, a.stream,
                         static_cast<const uint16_t*>(a.key), static_cast<const uint16_t*>(a.value), kc,
                         vc, a.slot_mapping, n_items, row_chunks, d_chunks, a.num_kv_heads, a.block_size,
                         n_slots, a.k_inv_scale, a.v_inv_scale);
    return hipGetLastError();
  }
  const int elem_bytes = a.dtype == kDtypeF32 ? 4 : 2;
  const int d_chunks = a.head_dim * elem_bytes / 16;
  const int row_chunks = a.num_kv_heads * d_chunks;
  const int64_t n_items = (int64_t)a.num_tokens * row_chunks;
  const int64_t blocks = (n_items + 255) / 256;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     a.stream, static_cast<const uint4*>(a.key), static_cast<const uint4*>(a.value),
                     static_cast<uint4*>(a.k_cache), static_cast<uint4*>(a.v_cache), a.slot_mapping,
                     n_items, row_chunks, d_chunks, a.num_kv_heads, a.block_size, n_slots);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyLaunch& a) {
  const int64_t block_chunks = (int64_t)a.num_kv_heads * a.block_size * a.head_dim * a.elem_bytes / 16;
  int64_t gy = (block_chunks + 255) / 256;
  if (gy > 64) gy = 64;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(a.num_pairs, static_cast<unsigned>(gy)), dim3(256), 0,
                     a.stream, static_cast<uint4*>(a.k_cache), static_cast<uint4*>(a.v_cache),
                     static_cast<const uint4*>(a.src_k_cache ? a.src_k_cache : a.k_cache),
                     static_cast<const uint4*>(a.src_v_cache ? a.src_v_cache : a.v_cache), a.block_pairs,
                     block_chunks, a.src_k_cache ? a.num_src_blocks : a.num_blocks, a.num_blocks);
  return hipGetLastError();
}

}  // namespace pa
