// Decode dispatch and the partition reduce.
//
// A sequence longer than the partition length is cut into partitions of a
// fixed number of tokens (a function of its own length only, so its result
// does not depend on the rest of the batch); each partition leaves the
// triple (running max m_p in log2 units, running sum l_p, unnormalised
// output acc_p) and this kernel merges them:
//   M = max_p m_p,  L = sum_p l_p 2^(m_p - M),  out = sum_p acc_p 2^(m_p - M) / L,
// the same rescaling the online softmax of "vLLM 深度解读" (luoboask.github.io,
// section 3 "PagedAttention CUDA Kernel") applies token by token.

#include "pa_device.h"

namespace pa {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(64) void decode_reduce_kernel(DecodeParams p) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int ctx = p.context_lens[s];
  if (ctx < 0 || ctx > p.max_context_len) return;  // written as NaN by the partition kernel
  const int nparts = parts_for(ctx, p.partition_tokens);
  if (nparts <= 1) return;                          // written by the partition kernel
  const int64_t base = ((int64_t)s * p.num_heads + h) * p.max_parts;
  const float* ml = p.ws_ml + base * 2;
  float mm = -FLT_MAX;
  for (int q = 0; q < nparts; ++q) mm = fmaxf(mm, ml[2 * q]);
  float ll = 0.f;
  for (int q = 0; q < nparts; ++q) ll += ml[2 * q + 1] * fast_exp2(ml[2 * q] - mm);
  for (int d = threadIdx.x; d < D; d += 64) {
    float aa = 0.f;
    for (int q = 0; q < nparts; ++q) aa += p.ws_acc[(base + q) * D + d] * fast_exp2(ml[2 * q] - mm);
    const float o = (ll == 0.f) ? 0.f : aa / ll;
    Elem<T>::store(static_cast<T*>(p.out) + ((int64_t)s * p.num_heads + h) * D + d, o);
  }
}

template <typename T>
hipError_t launch_reduce(const DecodeLaunch& a, const DecodeParams& p) {
  dim3 grid(a.num_heads, a.num_seqs);
  if (a.head_dim == 64)
    hipLaunchKernelGGL((decode_reduce_kernel<T, 64>), grid, dim3(64), 0, a.stream, p);
  else
    hipLaunchKernelGGL((decode_reduce_kernel<T, 128>), grid, dim3(64), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace

static bool use_mfma_path(int dtype, int group) { return dtype == 1 && group >= 2; }

int default_partition_tokens(int /*dtype*/, int /*head_dim*/, int block_size, int /*group*/) {
  // 2048 tokens: 128 pages of 16 or 64 pages of 32 per workgroup.
  const int t = 2048;
  return t - t % block_size;
}

hipError_t launch_decode(const DecodeLaunch& a) {
  DecodeParams p;
  p.out = a.out;
  p.q = a.q;
  p.k_cache = a.k_cache;
  p.v_cache = a.v_cache;
  p.block_tables = a.block_tables;
  p.context_lens = a.context_lens;
  p.ws_ml = a.ws_ml;
  p.ws_acc = a.ws_acc;
  p.block_stride = (int64_t)a.num_kv_heads * a.block_size * a.head_dim;
  p.max_blocks_per_seq = a.max_blocks_per_seq;
  p.num_heads = a.num_heads;
  p.num_blocks = a.num_blocks;
  p.max_context_len = a.max_context_len;
  p.partition_tokens = a.partition_tokens;
  p.max_parts = a.max_parts;
  p.scale_log2e = a.scale * kLog2e;
  const int group = a.num_heads / a.num_kv_heads;
  hipError_t e = use_mfma_path(a.dtype, group) ? launch_partition_mfma(a, p) : launch_partition_valu(a, p);
  if (e != hipSuccess || a.max_parts <= 1) return e;
  return a.dtype == 0 ? launch_reduce<float>(a, p) : launch_reduce<uint16_t>(a, p);
}

}  // namespace pa
