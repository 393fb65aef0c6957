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

// One wave per (head, sequence).  Up to kFewParts partitions, every load of
// the wave goes out at once: lane q reads the (max, sum) pair of partition q,
// and each lane reads its output columns of every partition; the weights then
// reach the column owners by shuffles.  More partitions take a loop that
// reads the pairs 64 at a time and passes their weights through LDS.  Both
// forms add the partitions in the same order, so they give the same bits.
constexpr int kFewParts = 8;

template <typename T, int D>
__global__ __launch_bounds__(64) void decode_reduce_kernel(DecodeParams p) {
  constexpr int E = D / 64;  // output columns per lane
  __shared__ float sw[64];
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int lane = threadIdx.x;
  const int row = query_row(p, s);
  if (row < 0) return;  // not a decode row of this call
  const PrefixChunk pc = prefix_chunk(p, s);
  const SeqSplit sp = split_context(p, p.context_lens[s], pc.blocks, pc.blocks > 0 ? s - pc.chunk : -1);
  if (sp.bad || sp.ctx < p.min_context) return;  // written as NaN by the partition kernel
  const int nparts = sp.nprefix + sp.ntail;
  if (nparts <= 1) return;  // written by the partition kernel
  const int64_t base = ((int64_t)s * p.num_heads + h) * p.max_parts;
  const float2* ml = reinterpret_cast<const float2*>(p.ws_ml) + base;
  const float* acc = p.ws_acc + base * D + lane;
  float aa[E];
#pragma unroll
  for (int e = 0; e < E; ++e) aa[e] = 0.f;
  float ll = 0.f;
  if (nparts <= kFewParts) {
    const float2 v = lane < nparts ? ml[lane] : make_float2(-FLT_MAX, 0.f);
    float a[kFewParts][E];
#pragma unroll
    for (int q = 0; q < kFewParts; ++q)
#pragma unroll
      for (int e = 0; e < E; ++e) a[q][e] = q < nparts ? acc[(int64_t)q * D + 64 * e] : 0.f;
    float mm = v.x;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mm = fmaxf(mm, __shfl_xor(mm, off));
    const float w = lane < nparts ? fast_exp2(v.x - mm) : 0.f;
    ll = v.y * w;
#pragma unroll
    for (int q = 0; q < kFewParts; ++q) {
      const float wq = __shfl(w, q);
      if (q < nparts) {
#pragma unroll
        for (int e = 0; e < E; ++e) aa[e] += a[q][e] * wq;
      }
    }
  } else {
    float mm = -FLT_MAX;
    for (int q = lane; q < nparts; q += 64) mm = fmaxf(mm, ml[q].x);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mm = fmaxf(mm, __shfl_xor(mm, off));
    for (int q0 = 0; q0 < nparts; q0 += 64) {
      const int q = q0 + lane;
      float w = 0.f;
      if (q < nparts) {
        const float2 v = ml[q];
        w = fast_exp2(v.x - mm);
        ll += v.y * w;
      }
      __syncthreads();
      sw[lane] = w;
      __syncthreads();
      const int n = min(64, nparts - q0);
      for (int j = 0; j < n; ++j) {
        const float wj = sw[j];
#pragma unroll
        for (int e = 0; e < E; ++e) aa[e] += acc[(int64_t)(q0 + j) * D + 64 * e] * wj;
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ll += __shfl_xor(ll, off);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float o = (ll == 0.f) ? 0.f : aa[e] * p.v_scale / ll;
    Elem<T>::store(static_cast<T*>(p.out) + ((int64_t)row * p.num_heads + h) * D + lane + 64 * e, o);
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

// Grouped heads with a bf16 query (bf16 or fp8 cache) run on the matrix cores.
static bool use_mfma_path(int dtype, int group) { return dtype == kDtypeBf16 && group >= 2; }

int default_partition_tokens(int dtype, int /*cache_dtype*/, int /*head_dim*/, int block_size, int group,
                             bool shared_prefix, int max_prefix_tokens) {
  // Fixed lengths (never the batch size, so a sequence's result does not
  // depend on the batch): 4096 tokens on the vector path, 8192 on the
  // matrix-core path (both capped at the 256 pages a partition can hold).
  // Fewer, longer workgroups measured faster: on ragged MHA batches (64
  // sequences of 128..4096 tokens, LLaMA-7B shape: 314 us against 348 at
  // 2048; 128 of 1000..8000: 1650 against 1799), the same within 2% on
  // uniform ones; on 16 GQA sequences of 32K tokens (70B shape, 32-token
  // pages) 320 us against 327 at 4096 (bf16) and 167 against 175 (E4M3):
  // 512 workgroups run in one round where 1024 need two at three per CU.
  // Batches of a few long sequences take the batch-shaped length instead
  // (PA_PARTITION_FILL).
  // Shared-prefix decode: a quarter of the longest shared prefix, rounded up
  // to a power of two within [256, 2048] -- each prefix is spread over about
  // four workgroups per kv head (measured best for 1024- and 4096-token
  // prefixes of 4-beam groups).
  int t = use_mfma_path(dtype, group) ? 8192 : 4096;
  if (shared_prefix) {
    t = 256;
    while (t < 2048 && 4 * t < max_prefix_tokens) t *= 2;
  }
  const int cap = kMaxPagesPerPartition * block_size;
  const int u = t < cap ? t : cap;
  return u - u % block_size;
}

int fill_partition_tokens(int dtype, int cache_dtype, int head_dim, int block_size, int group,
                          int num_seqs, int num_kv_heads, int max_context_len) {
  // Batch-shaped: start from the fixed length and halve it, down to 256
  // tokens, while the partition grid (sequences x kv heads x partitions of the
  // longest context) has fewer workgroups than the chip needs to stay busy.
  // Measured on batches of 1..32 sequences of 4K..64K tokens: one workgroup
  // per compute unit on the matrix-core path, four on the vector path, whose
  // workgroups each stream one head and have less work in flight.
  const int64_t target = use_mfma_path(dtype, group) ? 256 : 1024;
  int t = default_partition_tokens(dtype, cache_dtype, head_dim, block_size, group, false, 0);
  while (t > 256 && (int64_t)num_seqs * num_kv_heads * (((int64_t)max_context_len + t - 1) / t) < target)
    t /= 2;
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
  p.seq_order = a.seq_order;
  p.ws_ml = a.ws_ml;
  p.ws_acc = a.ws_acc;
  p.block_stride = (int64_t)a.num_kv_heads * a.block_size * a.head_dim;
  p.max_blocks_per_seq = a.max_blocks_per_seq;
  p.num_seqs = a.num_seqs;
  p.num_heads = a.num_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.num_blocks = a.num_blocks;
  p.max_context_len = a.max_context_len;
  p.partition_tokens = a.partition_tokens;
  p.max_parts = a.max_parts;
  const bool fp8 = a.cache_dtype == kDtypeFp8;
  p.scale_log2e = a.scale * kLog2e * (fp8 ? a.k_scale : 1.f);
  p.v_scale = fp8 ? a.v_scale : 1.f;
  const int group = a.num_heads / a.num_kv_heads;
  p.prefix_leader = a.prefix_leader;
  p.prefix_blocks = a.prefix_blocks;
  p.chunk_seqs = 16 / group;
  p.block_size = a.block_size;
  p.max_prefix_blocks = a.max_prefix_blocks;
  p.max_tail_len = a.max_tail_len;
  p.prefix_parts = a.prefix_parts;
  p.tail_parts = a.tail_parts;
  p.query_start = a.query_start;
  p.num_query_rows = a.num_query_rows;
  p.min_context = a.query_start != nullptr ? 1 : 0;
  p.order_by_length = a.seq_order == nullptr && !a.shared_pages && a.prefix_leader == nullptr &&
                      a.num_seqs > 1 && a.num_seqs <= kOrderedSeqs;
  // Shared-prefix decode always runs on the matrix cores (one 16-column tile
  // holds the query heads of up to 16 / G sequences) and always merges.
  const bool shared = a.prefix_leader != nullptr;
  hipError_t e = shared || use_mfma_path(a.dtype, group) ? launch_partition_mfma(a, p)
                                                         : launch_partition_valu(a, p);
  if (e != hipSuccess || a.max_parts <= 1) return e;
  return a.dtype == kDtypeF32 ? launch_reduce<float>(a, p) : launch_reduce<uint16_t>(a, p);
}

}  // namespace pa
