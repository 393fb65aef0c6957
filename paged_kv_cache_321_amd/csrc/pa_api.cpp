// C entry points of libpa.so: argument validation, workspace carving and
// kernel dispatch.  Every check here runs on the host before any HIP call, so
// each error path is reachable without a GPU.  Semantics are documented in
// include/pa.h.
#include "pa.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pa_internal.h"

namespace {

constexpr int kMaxGridYZ = 65535;

int elem_bytes(int dtype) { return dtype == PA_F32 ? 4 : dtype == PA_BF16 ? 2 : 1; }

bool value_dtype(int dtype) { return dtype == PA_F32 || dtype == PA_BF16; }
bool cache_dtype_ok(int dtype) { return value_dtype(dtype) || dtype == PA_FP8_E4M3; }
bool good_scale(float s) { return isfinite(s) && s > 0.f; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Partitions of n tokens (n >= 0, t > 0), computed in 64 bits so that lengths
// near INT_MAX do not overflow.
int parts_of(int n, int t) { return n <= t ? 1 : (int)(((int64_t)n + t - 1) / t); }

bool supported_head_dim(int d) { return d == 64 || d == 128; }
bool supported_block_size(int bs) { return bs == 16 || bs == 32; }
bool supported_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

int cache_shape_status(int num_blocks, int num_kv_heads, int block_size, int head_dim, int cache_dtype) {
  if (!cache_dtype_ok(cache_dtype)) return PA_ERR_DTYPE;
  if (num_blocks <= 0 || num_kv_heads <= 0 || block_size <= 0 || head_dim <= 0) return PA_ERR_SHAPE;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

// Resolved partition length, or a negative status.
int resolve_partition(int partition_tokens, int dtype, int cache_dtype, int head_dim, int block_size,
                      int group, bool shared_prefix, int max_prefix_tokens) {
  if (partition_tokens == 0)
    return pa::default_partition_tokens(dtype, cache_dtype, head_dim, block_size, group, shared_prefix,
                                        max_prefix_tokens);
  if (partition_tokens < 0 || partition_tokens % block_size != 0) return PA_ERR_SHAPE;
  if (partition_tokens / block_size > pa::kMaxPagesPerPartition) return PA_ERR_UNSUPPORTED;
  return partition_tokens;
}

struct DecodeSizes {
  int status;
  int partition_tokens;
  int grid_parts;    // partitions of the longest context
  int max_parts;     // partition slots per (sequence, head) in the workspace
  size_t ml_bytes;   // offset of the accumulator area, 256-byte aligned
  size_t total;      // 0 when a single partition always suffices
  int prefix_parts;  // shared-prefix decode: grid slots per sequence
  int tail_parts;
};

// With a shared prefix a context is cut at the prefix end: at most
// ceil(max_prefix_blocks * block_size / t) prefix partitions and
// ceil(max_tail_len / t) (at least 1) partitions of the rest.
DecodeSizes decode_sizes(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                         int max_context_len, int dtype, int cache_dtype, int partition_tokens,
                         bool shared_prefix, int max_prefix_blocks = 0, int max_tail_len = 0) {
  DecodeSizes z{PA_OK, 0, 1, 1, 0, 0, 0, 1};
  if (!value_dtype(dtype) || !cache_dtype_ok(cache_dtype)) { z.status = PA_ERR_DTYPE; return z; }
  if (cache_dtype != dtype && !(dtype == PA_BF16 && cache_dtype == PA_FP8_E4M3)) {
    z.status = PA_ERR_UNSUPPORTED;
    return z;
  }
  if (shared_prefix && dtype != PA_BF16) {  // the shared-prefix tile runs on bf16 matrix cores
    z.status = PA_ERR_UNSUPPORTED;
    return z;
  }
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      max_context_len < 0) {
    z.status = PA_ERR_SHAPE;
    return z;
  }
  if (num_heads % num_kv_heads != 0) { z.status = PA_ERR_SHAPE; return z; }
  const int group = num_heads / num_kv_heads;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size) || !supported_group(group)) {
    z.status = PA_ERR_UNSUPPORTED;
    return z;
  }
  if (shared_prefix &&
      (max_prefix_blocks < 0 || max_tail_len < 0 ||
       (int64_t)max_prefix_blocks * block_size > max_context_len || max_tail_len > max_context_len)) {
    z.status = PA_ERR_SHAPE;
    return z;
  }
  const int pt = resolve_partition(partition_tokens, dtype, cache_dtype, head_dim, block_size, group,
                                   shared_prefix, max_prefix_blocks * block_size);
  if (pt < 0) { z.status = pt; return z; }
  z.partition_tokens = pt;
  z.grid_parts = parts_of(max_context_len, pt);
  z.max_parts = z.grid_parts;
  if (shared_prefix) {
    z.prefix_parts = (int)(((int64_t)max_prefix_blocks * block_size + pt - 1) / pt);
    z.tail_parts = parts_of(max_tail_len, pt);
    z.max_parts = z.prefix_parts + z.tail_parts;
    // One-dimensional grid: prefix rows for num_seqs rounded up to a whole
    // number of chunks (at most 16 sequences), tail rows per sequence.
    if (((int64_t)num_seqs + 15) * z.max_parts * num_kv_heads > 0x7fffffffLL) {
      z.status = PA_ERR_UNSUPPORTED;
      return z;
    }
  }
  if (z.max_parts > 1) {
    const uint64_t rows = (uint64_t)num_seqs * (uint64_t)num_heads * (uint64_t)z.max_parts;
    const uint64_t ml = (rows * 2 * sizeof(float) + 255) / 256 * 256;
    z.ml_bytes = (size_t)ml;
    z.total = (size_t)(ml + rows * (uint64_t)head_dim * sizeof(float));
  }
  return z;
}

}  // namespace

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: inconsistent or invalid sizes";
    case PA_ERR_DTYPE:
      return "PA_ERR_DTYPE: dtype must be PA_F32 or PA_BF16, a cache type PA_F32, PA_BF16 or PA_FP8_E4M3";
    case PA_ERR_UNSUPPORTED:
      return "PA_ERR_UNSUPPORTED: head_dim must be 64/128, block_size 16/32, heads per kv head "
             "1/2/4/8, (dtype, cache_dtype) one of (F32, F32), (BF16, BF16), (BF16, FP8_E4M3), "
             "grid within limits, known flags; the shared-prefix decode takes a bf16 query and flags 0";
    case PA_ERR_ALIGN: return "PA_ERR_ALIGN: buffer not aligned (16 bytes for data, element size for indices)";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_LAUNCH: return "PA_ERR_LAUNCH: HIP reported an error after the launch";
    case PA_ERR_VALUE: return "PA_ERR_VALUE: an fp8 cache scale must be finite and > 0";
    case PA_ERR_SCRATCH:
      return "PA_ERR_SCRATCH: the call needs more workspace than the library's static scratch "
             "buffer holds (PA_DECODE_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown pa status";
  }
}

int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int num_tokens, int num_blocks, int num_kv_heads,
                         int block_size, int head_dim, int dtype, int cache_dtype, float k_scale,
                         float v_scale, void* stream) {
  if (!value_dtype(dtype)) return PA_ERR_DTYPE;
  int st = cache_shape_status(num_blocks, num_kv_heads, block_size, head_dim, cache_dtype);
  if (st != PA_OK) return st;
  if (cache_dtype != dtype && cache_dtype != PA_FP8_E4M3) return PA_ERR_UNSUPPORTED;
  const bool fp8 = cache_dtype == PA_FP8_E4M3;
  if (fp8 && (!good_scale(k_scale) || !good_scale(v_scale))) return PA_ERR_VALUE;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (!k_cache || !v_cache) return PA_ERR_NULL;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !slot_mapping) return PA_ERR_NULL;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 8))
    return PA_ERR_ALIGN;
  const int64_t items = (int64_t)num_tokens * num_kv_heads * head_dim * elem_bytes(cache_dtype) / 16;
  if ((items + 255) / 256 > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
  pa::ReshapeLaunch a{key, value, k_cache, v_cache, slot_mapping, num_tokens, num_blocks,
                      num_kv_heads, block_size, head_dim, dtype, cache_dtype,
                      fp8 ? 1.0f / k_scale : 1.f, fp8 ? 1.0f / v_scale : 1.f,
                      static_cast<hipStream_t>(stream)};
  return pa::launch_reshape_and_cache(a) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_pairs, int num_pairs,
                   int num_blocks, int num_kv_heads, int block_size, int head_dim, int cache_dtype,
                   void* stream) {
  int st = cache_shape_status(num_blocks, num_kv_heads, block_size, head_dim, cache_dtype);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return PA_ERR_SHAPE;
  if (!k_cache || !v_cache) return PA_ERR_NULL;
  if (num_pairs == 0) return PA_OK;
  if (!block_pairs) return PA_ERR_NULL;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_pairs, 8)) return PA_ERR_ALIGN;
  pa::CopyLaunch a{k_cache, v_cache, block_pairs, num_pairs, num_blocks, num_kv_heads,
                   block_size, head_dim, elem_bytes(cache_dtype), static_cast<hipStream_t>(stream)};
  return pa::launch_copy_blocks(a) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_swap_blocks(void* dst_k_cache, void* dst_v_cache, const void* src_k_cache, const void* src_v_cache,
                   const int64_t* block_pairs, int num_pairs, int num_src_blocks, int num_dst_blocks,
                   int num_kv_heads, int block_size, int head_dim, int cache_dtype, void* stream) {
  int st = cache_shape_status(num_dst_blocks, num_kv_heads, block_size, head_dim, cache_dtype);
  if (st != PA_OK) return st;
  if (num_src_blocks <= 0 || num_pairs < 0) return PA_ERR_SHAPE;
  if (!dst_k_cache || !dst_v_cache || !src_k_cache || !src_v_cache) return PA_ERR_NULL;
  if (num_pairs == 0) return PA_OK;
  if (!block_pairs) return PA_ERR_NULL;
  if (!aligned(dst_k_cache, 16) || !aligned(dst_v_cache, 16) || !aligned(src_k_cache, 16) ||
      !aligned(src_v_cache, 16) || !aligned(block_pairs, 8))
    return PA_ERR_ALIGN;
  pa::CopyLaunch a{dst_k_cache, dst_v_cache, block_pairs, num_pairs, num_dst_blocks, num_kv_heads,
                   block_size, head_dim, elem_bytes(cache_dtype), static_cast<hipStream_t>(stream)};
  a.src_k_cache = src_k_cache;
  a.src_v_cache = src_v_cache;
  a.num_src_blocks = num_src_blocks;
  return pa::launch_copy_blocks(a) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_decode_partition_tokens(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                               int block_size, int max_context_len, int dtype, int cache_dtype,
                               int policy) {
  if (policy != PA_PARTITION_FIXED && policy != PA_PARTITION_FILL) return PA_ERR_UNSUPPORTED;
  const DecodeSizes z = decode_sizes(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                     max_context_len, dtype, cache_dtype, 0, false);
  if (z.status != PA_OK) return z.status;
  if (policy == PA_PARTITION_FIXED) return z.partition_tokens;
  return pa::fill_partition_tokens(dtype, cache_dtype, head_dim, block_size, num_heads / num_kv_heads,
                                   num_seqs, num_kv_heads, max_context_len);
}

size_t pa_decode_workspace_size(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                int block_size, int max_context_len, int dtype, int cache_dtype,
                                int partition_tokens) {
  const DecodeSizes z = decode_sizes(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                     max_context_len, dtype, cache_dtype, partition_tokens, false);
  return z.status == PA_OK ? z.total : (size_t)-1;
}

size_t pa_decode_shared_prefix_workspace_size(int num_seqs, int num_heads, int num_kv_heads,
                                              int head_dim, int block_size, int max_context_len,
                                              int max_prefix_blocks, int max_tail_len, int dtype,
                                              int cache_dtype, int partition_tokens) {
  const DecodeSizes z = decode_sizes(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                     max_context_len, dtype, cache_dtype, partition_tokens, true,
                                     max_prefix_blocks, max_tail_len);
  return z.status == PA_OK ? z.total : (size_t)-1;
}

}  // extern "C"

namespace {

// Both decode entry points: validation, workspace carving, launch.  The
// shared-prefix form passes its two per-sequence arrays (non-null).
int decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                const int32_t* seq_order, const int32_t* prefix_leader, const int32_t* prefix_blocks,
                bool shared_prefix, int max_prefix_blocks, int max_tail_len, int num_seqs,
                int num_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                int max_context_len, float scale, int dtype, int cache_dtype, float k_scale,
                float v_scale, int partition_tokens, int flags, void* workspace,
                size_t workspace_bytes, void* stream, bool check_only = false) {
  const DecodeSizes z = decode_sizes(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                     max_context_len, dtype, cache_dtype, partition_tokens, shared_prefix,
                                     max_prefix_blocks, max_tail_len);
  if (z.status != PA_OK) return z.status;
  const bool fp8 = cache_dtype == PA_FP8_E4M3;
  if (fp8 && (!good_scale(k_scale) || !good_scale(v_scale))) return PA_ERR_VALUE;
  if (num_blocks <= 0 || max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size < max_context_len) return PA_ERR_SHAPE;
  if (flags & ~(shared_prefix ? 0 : PA_DECODE_SHARED_PAGES)) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL;
  if (shared_prefix && (!prefix_leader || !prefix_blocks)) return PA_ERR_NULL;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(seq_order, 4) ||
      !aligned(prefix_leader, 4) || !aligned(prefix_blocks, 4))
    return PA_ERR_ALIGN;
  if (num_seqs > kMaxGridYZ || num_kv_heads > kMaxGridYZ || num_heads > kMaxGridYZ)
    return PA_ERR_UNSUPPORTED;
  if (check_only) return PA_OK;  // every check but the workspace's passed
  if (z.total > 0) {
    if (!workspace || workspace_bytes < z.total) return PA_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return PA_ERR_ALIGN;
  }
  char* ws = static_cast<char*>(workspace);
  pa::DecodeLaunch a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.seq_order = seq_order;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.scale = scale;
  a.dtype = dtype;
  a.cache_dtype = cache_dtype;
  a.k_scale = fp8 ? k_scale : 1.f;
  a.v_scale = fp8 ? v_scale : 1.f;
  a.partition_tokens = z.partition_tokens;
  a.shared_pages = (flags & PA_DECODE_SHARED_PAGES) != 0;
  a.grid_parts = z.grid_parts;
  a.max_parts = z.max_parts;
  a.ws_ml = z.total ? reinterpret_cast<float*>(ws) : nullptr;
  a.ws_acc = z.total ? reinterpret_cast<float*>(ws + z.ml_bytes) : nullptr;
  a.query_start = nullptr;
  a.num_query_rows = 0;
  a.prefix_leader = shared_prefix ? prefix_leader : nullptr;
  a.prefix_blocks = shared_prefix ? prefix_blocks : nullptr;
  a.max_prefix_blocks = max_prefix_blocks;
  a.max_tail_len = max_tail_len;
  a.prefix_parts = z.prefix_parts;
  a.tail_parts = z.tail_parts;
  a.stream = static_cast<hipStream_t>(stream);
  return pa::launch_decode(a) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

// Workspace of pa_multi_query: the decode kernels' partitions (sequences
// with one query, indexed by sequence) followed by the multi-query
// partitions (indexed by query row).
struct MultiQuerySizes {
  int status;
  int partition_tokens;
  int max_parts;
  size_t ml_bytes;
  size_t total;
  int decode_partition_tokens;
  int decode_grid_parts;
  size_t decode_ml_bytes;
  size_t decode_bytes;  // offset of the multi-query area, 256-byte aligned
  size_t parts_bytes;   // multi-query partition area (0 without cuts)
  int64_t work_capacity;
  size_t work_bytes;    // work list and its count, after the partition area
};

size_t partition_area(uint64_t rows, int head_dim, size_t* ml_bytes) {
  const uint64_t ml = (rows * 2 * sizeof(float) + 255) / 256 * 256;
  *ml_bytes = (size_t)ml;
  return (size_t)((ml + rows * (uint64_t)head_dim * sizeof(float) + 255) / 256 * 256);
}

MultiQuerySizes multi_query_sizes(int num_seqs, int num_query_tokens, int num_heads, int num_kv_heads,
                                  int head_dim, int block_size, int max_context_len, int dtype,
                                  int cache_dtype, int partition_tokens) {
  MultiQuerySizes z{PA_OK, 0, 1, 0, 0, 0, 1, 0, 0, 0, 0, 0};
  if (!value_dtype(dtype) || !cache_dtype_ok(cache_dtype)) { z.status = PA_ERR_DTYPE; return z; }
  // The tiles run on bf16 matrix cores: a bf16 query over a bf16 or fp8 cache.
  if (dtype != PA_BF16 || cache_dtype == PA_F32) { z.status = PA_ERR_UNSUPPORTED; return z; }
  if (num_seqs < 0 || num_query_tokens < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || max_context_len < 0 || num_heads % num_kv_heads != 0) {
    z.status = PA_ERR_SHAPE;
    return z;
  }
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size) ||
      !supported_group(num_heads / num_kv_heads)) {
    z.status = PA_ERR_UNSUPPORTED;
    return z;
  }
  int pt = partition_tokens;
  if (pt == 0) pt = pa::default_multi_query_partition_tokens(block_size, num_seqs, num_kv_heads, max_context_len);
  if (pt < 0 || pt % block_size != 0) { z.status = PA_ERR_SHAPE; return z; }
  z.partition_tokens = pt;
  z.max_parts = parts_of(max_context_len, pt);
  const int dpt = pa::default_partition_tokens(dtype, cache_dtype, head_dim, block_size,
                                               num_heads / num_kv_heads, false, 0);
  z.decode_partition_tokens = dpt;
  z.decode_grid_parts = parts_of(max_context_len, dpt);
  if (z.decode_grid_parts > 1)
    z.decode_bytes = partition_area((uint64_t)num_seqs * num_heads * z.decode_grid_parts, head_dim,
                                    &z.decode_ml_bytes);
  if (z.max_parts > 1)
    z.parts_bytes = partition_area((uint64_t)num_query_tokens * num_heads * z.max_parts, head_dim, &z.ml_bytes);
  // Work items: every row block (at most T * G / 64 plus one partial block per
  // sequence) or, for a sequence of one block, its partitions.
  const int rpb = pa::multi_query_rows_per_block();
  z.work_capacity = ((int64_t)num_query_tokens * (num_heads / num_kv_heads) + rpb - 1) / rpb +
                    (int64_t)num_seqs * (z.max_parts + 1);
  z.work_bytes = (size_t)((z.work_capacity * 8 + 4 + 255) / 256 * 256);
  z.total = num_seqs > 0 && num_query_tokens > 0 ? z.decode_bytes + z.parts_bytes + z.work_bytes : 0;
  return z;
}

}  // namespace

extern "C" {

size_t pa_multi_query_workspace_size(int num_seqs, int num_query_tokens, int num_heads,
                                     int num_kv_heads, int head_dim, int block_size,
                                     int max_context_len, int dtype, int cache_dtype,
                                     int partition_tokens) {
  const MultiQuerySizes z = multi_query_sizes(num_seqs, num_query_tokens, num_heads, num_kv_heads,
                                              head_dim, block_size, max_context_len, dtype,
                                              cache_dtype, partition_tokens);
  return z.status == PA_OK ? z.total : (size_t)-1;
}

int pa_multi_query(void* out, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                   const int32_t* query_start, int num_seqs, int num_query_tokens, int max_query_len,
                   int num_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                   int max_context_len, float scale, int dtype, int cache_dtype, float k_scale,
                   float v_scale, int partition_tokens, int flags, void* workspace,
                   size_t workspace_bytes, const pa_side_stream* side, void* stream) {
  if (flags & ~(PA_MULTI_QUERY_TILES_ONLY | PA_MULTI_QUERY_ONE_STREAM)) return PA_ERR_UNSUPPORTED;
  if (side && (!side->stream || !side->fork_event || !side->join_event)) return PA_ERR_NULL;
  const bool tiles_only = (flags & PA_MULTI_QUERY_TILES_ONLY) != 0;
  const bool one_stream = (flags & PA_MULTI_QUERY_ONE_STREAM) != 0;
  const MultiQuerySizes z = multi_query_sizes(num_seqs, num_query_tokens, num_heads, num_kv_heads,
                                              head_dim, block_size, max_context_len, dtype,
                                              cache_dtype, partition_tokens);
  if (z.status != PA_OK) return z.status;
  const bool fp8 = cache_dtype == PA_FP8_E4M3;
  if (fp8 && (!good_scale(k_scale) || !good_scale(v_scale))) return PA_ERR_VALUE;
  if (max_query_len < 0 || num_blocks <= 0 || max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size < max_context_len) return PA_ERR_SHAPE;
  const int group = num_heads / num_kv_heads;
  const int rpb = pa::multi_query_rows_per_block();
  const int64_t row_blocks = ((int64_t)max_query_len * group + rpb - 1) / rpb;
  if (num_seqs == 0 || num_query_tokens == 0 || row_blocks == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return PA_ERR_NULL;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(query_start, 4))
    return PA_ERR_ALIGN;
  // Work items carry the row-block and partition indices in 16 bits each.
  if (z.work_capacity * num_kv_heads > 0x7fffffffLL || row_blocks > 0x7fff || z.max_parts > 0x7fff ||
      num_seqs > kMaxGridYZ || num_kv_heads > kMaxGridYZ || num_heads > kMaxGridYZ)
    return PA_ERR_UNSUPPORTED;
  if (z.total > 0) {
    if (!workspace || workspace_bytes < z.total) return PA_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return PA_ERR_ALIGN;
  }
  char* ws = static_cast<char*>(workspace);
  pa::MultiQueryLaunch a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.num_seqs = num_seqs;
  a.num_query_tokens = num_query_tokens;
  a.max_query_len = max_query_len;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.scale = scale;
  a.cache_dtype = cache_dtype;
  a.k_scale = fp8 ? k_scale : 1.f;
  a.v_scale = fp8 ? v_scale : 1.f;
  a.partition_tokens = z.partition_tokens;
  a.max_parts = z.max_parts;
  a.max_row_blocks = (int)row_blocks;
  a.ws_ml = z.max_parts > 1 ? reinterpret_cast<float*>(ws + z.decode_bytes) : nullptr;
  a.ws_acc = z.max_parts > 1 ? reinterpret_cast<float*>(ws + z.decode_bytes + z.ml_bytes) : nullptr;
  a.work = ws + z.decode_bytes + z.parts_bytes;
  a.work_count = reinterpret_cast<int*>(ws + z.decode_bytes + z.parts_bytes + z.work_capacity * 8);
  a.work_capacity = (int)z.work_capacity;
  a.decode_rows_elsewhere = !tiles_only;
  a.beside_decode = false;
  a.stream = static_cast<hipStream_t>(stream);
  if (tiles_only) return pa::launch_multi_query(a) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
  // Sequences with a single new query are decode steps: the decode kernels
  // serve them (q / out row query_start[s]); the multi-query kernel skips them.
  pa::DecodeLaunch d;
  d.out = out;
  d.q = q;
  d.k_cache = k_cache;
  d.v_cache = v_cache;
  d.block_tables = block_tables;
  d.max_blocks_per_seq = max_blocks_per_seq;
  d.context_lens = context_lens;
  d.seq_order = nullptr;
  d.num_seqs = num_seqs;
  d.num_heads = num_heads;
  d.num_kv_heads = num_kv_heads;
  d.head_dim = head_dim;
  d.block_size = block_size;
  d.num_blocks = num_blocks;
  d.max_context_len = max_context_len;
  d.scale = scale;
  d.dtype = dtype;
  d.cache_dtype = cache_dtype;
  d.k_scale = a.k_scale;
  d.v_scale = a.v_scale;
  d.partition_tokens = z.decode_partition_tokens;
  d.shared_pages = false;
  d.grid_parts = z.decode_grid_parts;
  d.max_parts = z.decode_grid_parts;
  d.ws_ml = z.decode_bytes ? reinterpret_cast<float*>(ws) : nullptr;
  d.ws_acc = z.decode_bytes ? reinterpret_cast<float*>(ws + z.decode_ml_bytes) : nullptr;
  d.query_start = query_start;
  d.num_query_rows = num_query_tokens;
  d.prefix_leader = nullptr;
  d.prefix_blocks = nullptr;
  d.max_prefix_blocks = 0;
  d.max_tail_len = 0;
  d.prefix_parts = 0;
  d.tail_parts = 1;
  d.stream = a.stream;
  if (max_query_len < 2)  // no sequence has more than one query
    return pa::launch_decode(d) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
  if (one_stream || !side) {
    if (pa::launch_decode(d) != hipSuccess) return PA_ERR_LAUNCH;
    return pa::launch_multi_query(a) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
  }
  // Fork: the multi-query kernels (long workgroups, matrix-core bound) go
  // first on the caller's stream, the decode kernels (cache-read bound) on
  // the side stream; the join makes `stream` wait for both.
  const hipStream_t side_stream = static_cast<hipStream_t>(side->stream);
  const hipEvent_t fork = static_cast<hipEvent_t>(side->fork_event);
  const hipEvent_t join = static_cast<hipEvent_t>(side->join_event);
  if (hipEventRecord(fork, a.stream) != hipSuccess) return PA_ERR_LAUNCH;
  if (hipStreamWaitEvent(side_stream, fork, 0) != hipSuccess) return PA_ERR_LAUNCH;
  d.stream = side_stream;
  a.beside_decode = true;
  const bool mq_ok = pa::launch_multi_query(a) == hipSuccess;
  const bool dec_ok = pa::launch_decode(d) == hipSuccess;
  const bool join_ok = hipEventRecord(join, side_stream) == hipSuccess &&
                       hipStreamWaitEvent(a.stream, join, 0) == hipSuccess;
  return mq_ok && dec_ok && join_ok ? PA_OK : PA_ERR_LAUNCH;
}

int pa_side_stream_create(pa_side_stream* side) {
  if (!side) return PA_ERR_NULL;
  hipStream_t st = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return PA_ERR_LAUNCH;
  if (hipEventCreateWithFlags(&fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&join, hipEventDisableTiming) != hipSuccess) {
    if (fork) (void)hipEventDestroy(fork);
    (void)hipStreamDestroy(st);
    return PA_ERR_LAUNCH;
  }
  side->stream = st;
  side->fork_event = fork;
  side->join_event = join;
  return PA_OK;
}

int pa_side_stream_destroy(pa_side_stream* side) {
  if (!side) return PA_ERR_NULL;
  bool ok = true;
  if (side->join_event) ok = hipEventDestroy(static_cast<hipEvent_t>(side->join_event)) == hipSuccess && ok;
  if (side->fork_event) ok = hipEventDestroy(static_cast<hipEvent_t>(side->fork_event)) == hipSuccess && ok;
  if (side->stream) ok = hipStreamDestroy(static_cast<hipStream_t>(side->stream)) == hipSuccess && ok;
  side->stream = side->fork_event = side->join_event = nullptr;
  return ok ? PA_OK : PA_ERR_LAUNCH;
}

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
              const int32_t* seq_order, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
              int block_size, int num_blocks, int max_context_len, float scale, int dtype,
              int cache_dtype, float k_scale, float v_scale, int partition_tokens, int flags,
              void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     seq_order, nullptr, nullptr, false, 0, 0, num_seqs, num_heads, num_kv_heads, head_dim,
                     block_size, num_blocks, max_context_len, scale, dtype, cache_dtype, k_scale,
                     v_scale, partition_tokens, flags, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace pa {

int decode_check(const void* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                 const int32_t* seq_order, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                 int block_size, int num_blocks, int max_context_len, int dtype, int cache_dtype,
                 float k_scale, float v_scale, int partition_tokens, int flags) {
  return decode_impl(const_cast<void*>(out), q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                     context_lens, seq_order, nullptr, nullptr, false, 0, 0, num_seqs, num_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, max_context_len, 1.f, dtype,
                     cache_dtype, k_scale, v_scale, partition_tokens, flags, nullptr, 0, nullptr, true);
}

}  // namespace pa

extern "C" {

int pa_decode_shared_prefix(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int max_blocks_per_seq,
                            const int32_t* context_lens, const int32_t* prefix_leader,
                            const int32_t* prefix_blocks, int num_seqs, int num_heads,
                            int num_kv_heads, int head_dim, int block_size, int num_blocks,
                            int max_context_len, int max_prefix_blocks, int max_tail_len,
                            float scale, int dtype, int cache_dtype, float k_scale, float v_scale,
                            int partition_tokens, int flags, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, nullptr,
                     prefix_leader, prefix_blocks, true, max_prefix_blocks, max_tail_len, num_seqs,
                     num_heads, num_kv_heads, head_dim,
                     block_size, num_blocks, max_context_len, scale, dtype, cache_dtype, k_scale,
                     v_scale, partition_tokens, flags, workspace, workspace_bytes, stream);
}

}  // extern "C"
