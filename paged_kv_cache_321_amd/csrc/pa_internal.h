// Internal interface between the validating C entry points (pa_api.cpp) and
// the kernel launchers (pa_cache.hip, pa_decode*.hip, pa_multi_query.hip).  Not part
// of the public ABI.
#ifndef PA_INTERNAL_H_
#define PA_INTERNAL_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Waves per decode workgroup.  The pages of one partition are dealt out to
// the waves round-robin; each wave keeps one page id per lane, so a partition
// holds at most kWaves * 64 pages.
constexpr int kWaves = 4;

// Element type codes (the values of pa_dtype in pa.h).
constexpr int kDtypeF32 = 0;
constexpr int kDtypeBf16 = 1;
constexpr int kDtypeFp8 = 2;
constexpr int kMaxPagesPerPartition = kWaves * 64;

struct DecodeLaunch {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* context_lens;
  const int32_t* seq_order;  // null: the kernels choose (longest first for small batches)
  int num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks;
  int max_context_len;
  float scale;
  int dtype;        // query / output
  int cache_dtype;  // k_cache / v_cache
  float k_scale;    // fp8 caches: a code stands for value * scale
  float v_scale;
  int partition_tokens;  // resolved, > 0
  bool shared_pages;     // pages may be shared: default cache policy, else non-temporal
  int grid_parts;        // ceil(max_context_len / partition_tokens), >= 1
  int max_parts;         // partition slots per (sequence, head): grid_parts, or
                         // prefix_parts + tail_parts with a shared prefix
  float* ws_ml;          // [S, H, max_parts, 2] (running max, running sum); null if max_parts == 1
  float* ws_acc;         // [S, H, max_parts, D] unnormalised outputs; null if max_parts == 1
  // Shared-prefix decode (null for the plain decode): per-sequence group
  // leader and shared leading blocks (read at leaders).
  const int32_t* prefix_leader;
  const int32_t* prefix_blocks;
  // Decode rows of a multi-query batch (null otherwise): sequences with one
  // new query, at q / out row query_start[s].
  const int32_t* query_start;
  int num_query_rows;
  int max_prefix_blocks;  // caller's bounds: prefix_blocks at leaders, context - prefix
  int max_tail_len;
  int prefix_parts;       // ceil(max_prefix_blocks * block_size / partition_tokens)
  int tail_parts;         // ceil(max_tail_len / partition_tokens), >= 1
  hipStream_t stream;
};

struct ReshapeLaunch {
  const void* key;
  const void* value;
  void* k_cache;
  void* v_cache;
  const int64_t* slot_mapping;
  int num_tokens, num_blocks, num_kv_heads, block_size, head_dim;
  int dtype;          // key / value
  int cache_dtype;    // same as dtype (copy) or fp8 (encode)
  float k_inv_scale;  // fp8: fl32(1 / k_scale)
  float v_inv_scale;
  hipStream_t stream;
};

struct CopyLaunch {
  void* k_cache;  // destination pool (and source, for copy_blocks)
  void* v_cache;
  const int64_t* block_pairs;
  int num_pairs, num_blocks, num_kv_heads, block_size, head_dim, elem_bytes;
  hipStream_t stream;
  const void* src_k_cache = nullptr;  // another source pool (swap_blocks), or null
  const void* src_v_cache = nullptr;
  int num_src_blocks = 0;
};

struct MultiQueryLaunch {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* context_lens;
  const int32_t* query_start;
  int num_seqs, num_query_tokens, max_query_len;
  int num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_context_len;
  float scale;
  int cache_dtype;  // bf16 or fp8 (the query is bf16)
  float k_scale, v_scale;
  int partition_tokens;  // resolved, > 0
  int max_parts;         // ceil(max_context_len / partition_tokens), >= 1
  int max_row_blocks;    // ceil(max_query_len * G / rows per block)
  float* ws_ml;          // [T, H, max_parts, 2]; null if max_parts == 1
  float* ws_acc;         // [T, H, max_parts, D]; null if max_parts == 1
  void* work;            // work list: work_capacity 8-byte items (workspace)
  int* work_count;       // (workspace)
  int work_capacity;     // bound on the work items: the grid size per kv head
  bool decode_rows_elsewhere;  // single-query sequences go to the decode kernels
  bool beside_decode;          // the decode kernels run concurrently on another stream
  hipStream_t stream;
};

// Default partition length (tokens) for a shape; a multiple of block_size.
int default_partition_tokens(int dtype, int cache_dtype, int head_dim, int block_size, int group,
                             bool shared_prefix, int max_prefix_tokens);
// Partition length shaped to a pa_decode batch (PA_PARTITION_FILL).
int fill_partition_tokens(int dtype, int cache_dtype, int head_dim, int block_size, int group,
                          int num_seqs, int num_kv_heads, int max_context_len);

hipError_t launch_decode(const DecodeLaunch& a);
// Every host check pa_decode makes on these arguments except the workspace's;
// launches nothing and makes no HIP call.
int decode_check(const void* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                 const int32_t* seq_order, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                 int block_size, int num_blocks, int max_context_len, int dtype, int cache_dtype,
                 float k_scale, float v_scale, int partition_tokens, int flags);
int default_multi_query_partition_tokens(int block_size, int num_seqs, int num_kv_heads, int max_context_len);
int multi_query_rows_per_block();
hipError_t launch_multi_query(const MultiQueryLaunch& a);
hipError_t launch_reshape_and_cache(const ReshapeLaunch& a);
hipError_t launch_copy_blocks(const CopyLaunch& a);

}  // namespace pa

#endif  // PA_INTERNAL_H_
