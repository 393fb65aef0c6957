/*
 * pa.h -- C ABI of libpa.so: decode attention over a paged KV cache on AMD
 * MI355X (gfx950).
 *
 * What is computed comes from these pages:
 *  [tbr8]     "详解vLLM推理引擎架构：PagedAttention原理与LLM高效部署实践"
 *             (tbr8.org/?p=10846): "PagedAttention 的核心思想" (K/V split into
 *             fixed-size blocks of 16 or 32 tokens, reached through a per-sequence
 *             block table) and "Copy-on-Write 与内存共享" (a shared block is
 *             copied to a fresh one before it is written).
 *  [luoboask] "vLLM 深度解读" (luoboask.github.io/fde-learning/opensource/vllm/):
 *             section 3 "PagedAttention CUDA Kernel" (one query per sequence and
 *             head; scores scale * q.k over every context token found through the
 *             block table; softmax; weighted sum of V), section 7 (each new token's
 *             K/V is stored into the cache, then paged attention runs).
 *
 * Layouts (row-major; element type `dtype` = float or bf16 for q, out, key and
 * value; `cache_dtype` for the caches: the same as dtype, or PA_FP8_E4M3):
 *   q, out          [num_seqs, num_heads, head_dim]
 *   key, value      [num_tokens, num_kv_heads, head_dim]
 *   k_cache, v_cache[num_blocks, num_kv_heads, block_size, head_dim]
 *                   (one (block, kv_head) page is a contiguous block_size x
 *                   head_dim tile)
 *   block_tables    int32 [num_seqs, max_blocks_per_seq]; entry j of row s is
 *                   the physical block holding tokens j*block_size ..
 *                   (j+1)*block_size-1 of sequence s
 *   context_lens    int32 [num_seqs]
 *   slot_mapping    int64 [num_tokens]; slot = block * block_size + offset
 *   block_pairs     int64 [num_pairs, 2]; (src, dst) physical block ids
 *
 * Conventions shared by every entry point:
 *  - Every buffer pointer is a DEVICE pointer.  The caller owns every buffer
 *    and every stream; the library allocates no device memory and keeps no
 *    state between calls (pa_decode_noalloc's static scratch buffer aside).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *    null stream).  A return of PA_OK means the kernels were enqueued.
 *  - A negative return means nothing was launched, except PA_ERR_LAUNCH, which
 *    reports a failure seen by hipGetLastError after the launch.
 *  - Arguments are validated on the host before any HIP call, so every error
 *    path below is reachable without a GPU.
 *  - Values that live in device memory (table entries, context lengths, slots,
 *    block pairs) cannot be checked on the host without a synchronisation.
 *    Their preconditions are listed per call; the kernels bound-check them and
 *    never access memory outside the buffers: a violated precondition gives the
 *    documented result (a skipped write, or NaN in the affected output row),
 *    not a fault.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  PA_FP8_E4M3 is a cache type only: OCP 8-bit floating point
 * E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, S.1111.111 = NaN, largest finite 448), one float scale per cache:
 * a code c stands for value(c) * scale.  ([tbr8] section "量化集成与部署"
 * offers an fp8 KV cache without fixing the format; this is the reading used.) */
typedef enum pa_dtype { PA_F32 = 0, PA_BF16 = 1, PA_FP8_E4M3 = 2 } pa_dtype;

/* pa_multi_query flags */
enum {
  /* Serve every sequence, single-query ones included, in the multi-query
   * tiles instead of routing sequences with one new query through the decode
   * kernels.  Saves the decode launch for batches that have no decode steps
   * (speculative verification); never changes what is computed. */
  PA_MULTI_QUERY_TILES_ONLY = 1,
  /* Launch every kernel on the caller's stream, even when a side stream is
   * given; the results are the same bits either way. */
  PA_MULTI_QUERY_ONE_STREAM = 2
};

/* A second stream for pa_multi_query, with the two events that fork it from
 * and join it back to the caller's stream: HIP handles (hipStream_t,
 * hipEvent_t) on one device, owned by the caller.  pa_side_stream_create
 * makes them (a non-blocking stream of default priority, two events with
 * timing disabled) and pa_side_stream_destroy releases them; a caller may also
 * fill the fields with handles of its own.  One handle serves one call at a
 * time: calls that overlap (from several host threads) need a handle each. */
typedef struct pa_side_stream {
  void* stream;
  void* fork_event;
  void* join_event;
} pa_side_stream;

/* pa_side_stream_create -- create the stream and events of *side on the
 * current device.  PA_ERR_NULL for a null side, PA_ERR_LAUNCH if HIP fails
 * (nothing is left allocated then). */
int pa_side_stream_create(pa_side_stream* side);

/* pa_side_stream_destroy -- destroy what pa_side_stream_create made (after the
 * work queued on it is done, as for any HIP stream) and zero the fields.
 * PA_ERR_NULL for a null side; null fields are skipped. */
int pa_side_stream_destroy(pa_side_stream* side);

/* pa_decode flags */
enum {
  /* Physical blocks may be shared by several sequences of the batch (prefix
   * sharing, beams).  Pages are then read with the default cache policy so
   * that later readers of a shared page can hit in cache; without the flag
   * pages are read with the non-temporal hint (each page read once). */
  PA_DECODE_SHARED_PAGES = 1
};

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL                        */
  PA_ERR_SHAPE = -2,       /* a size is negative/zero where it must not be, or  */
                           /* sizes are inconsistent (num_heads % num_kv_heads, */
                           /* max_blocks_per_seq * block_size < max_context_len)*/
  PA_ERR_DTYPE = -3,       /* dtype is not PA_F32 or PA_BF16                    */
  PA_ERR_UNSUPPORTED = -4, /* head_dim not 64/128, block_size not 16/32, group  */
                           /* size num_heads/num_kv_heads not 1/2/4/8, or a grid */
                           /* dimension over the hardware limit                 */
  PA_ERR_ALIGN = -5,       /* a floating-point buffer is not 16-byte aligned, or*/
                           /* an index buffer is not aligned to its element size*/
  PA_ERR_WORKSPACE = -6,   /* workspace missing or smaller than required        */
  PA_ERR_LAUNCH = -7,      /* the HIP runtime reported an error after launch    */
  PA_ERR_VALUE = -8,       /* a scale of an fp8 cache is not finite and > 0     */
  PA_ERR_SCRATCH = -9      /* pa_decode_noalloc: the call needs more workspace  */
                           /* than the static scratch buffer holds              */
} pa_status;

/*
 * pa_reshape_and_cache -- store new tokens' K and V rows into their cache slots.
 * ([luoboask] section 7: the K/V of each new token is written into the paged
 * cache in place before attention.)
 *
 * For every token i with 0 <= slot_mapping[i] < num_blocks*block_size:
 *   b = slot / block_size, o = slot % block_size, and for every kv head h
 *   k_cache[b, h, o, :] = key[i, h, :]  and  v_cache[b, h, o, :] = value[i, h, :]
 * -- a bit-exact copy when cache_dtype == dtype.  With cache_dtype ==
 * PA_FP8_E4M3 each element x is stored as the E4M3 code nearest to
 * x * fl32(1 / k_scale) (v_scale for values), computed in binary32, ties to the
 * even code, magnitudes >= 448 saturating to 448, NaN to a NaN code.
 * Negative slots mean "no write" (padding).  Slots at or past
 * num_blocks*block_size violate the precondition and are skipped.
 * Precondition: the non-negative slots are distinct (otherwise which token lands
 * in a slot is unspecified).  num_tokens == 0 is a no-op.  dtype is PA_F32 or
 * PA_BF16; k_scale and v_scale are read only for an fp8 cache (finite, > 0,
 * else PA_ERR_VALUE).
 */
int pa_reshape_and_cache(const void* key, const void* value,
                         void* k_cache, void* v_cache,
                         const int64_t* slot_mapping,
                         int num_tokens, int num_blocks, int num_kv_heads,
                         int block_size, int head_dim, int dtype, int cache_dtype,
                         float k_scale, float v_scale, void* stream);

/*
 * pa_copy_blocks -- copy whole cache blocks, K and V, src -> dst.
 * ([tbr8] "Copy-on-Write 与内存共享": before a block with more than one owner is
 * written, its content is copied to a freshly allocated block.)
 *
 * For every pair p: k_cache[dst] = k_cache[src] and v_cache[dst] = v_cache[src]
 * over all kv heads and all block_size slots (bit-exact).
 * Preconditions: 0 <= src, dst < num_blocks (pairs outside are skipped); the dst
 * ids are distinct and no dst is also a src (otherwise the result depends on
 * the order of the copies).  num_pairs == 0 is a no-op.
 */
int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_pairs,
                   int num_pairs, int num_blocks, int num_kv_heads,
                   int block_size, int head_dim, int cache_dtype, void* stream);

/*
 * pa_swap_blocks -- copy whole cache blocks, K and V, from one pool to another:
 * swap a preempted request's blocks out to host memory, or back in.
 * ([tbr8] scheduler section: when GPU memory runs short, the KV cache of
 * low-priority requests is swapped out to CPU memory and swapped back in
 * later, with --swap-space setting the CPU memory for it; [luoboask] section 4
 * "Scheduler": a SWAPPED queue whose requests are swapped back in when blocks
 * are free.)
 *
 * For every pair p = (src, dst): dst_k_cache[dst] = src_k_cache[src] and
 * dst_v_cache[dst] = src_v_cache[src] over all kv heads and slots (bit-exact);
 * both pools have the [blocks, num_kv_heads, block_size, head_dim] layout of
 * cache_dtype.  Either pool (and block_pairs) may live in host memory allocated
 * pinned with hipHostMalloc: the copy kernel reads and writes it through its
 * unified address, one launch for any number of scattered blocks.
 * Preconditions: 0 <= src < num_src_blocks, 0 <= dst < num_dst_blocks (pairs
 * outside are skipped); dst ids distinct; the pools do not overlap.
 * num_pairs == 0 is a no-op.
 */
int pa_swap_blocks(void* dst_k_cache, void* dst_v_cache,
                   const void* src_k_cache, const void* src_v_cache,
                   const int64_t* block_pairs, int num_pairs,
                   int num_src_blocks, int num_dst_blocks, int num_kv_heads,
                   int block_size, int head_dim, int cache_dtype, void* stream);

/* pa_decode_partition_tokens policies */
enum {
  /* The fixed length pa_decode uses for partition_tokens == 0: it depends on
   * the shape only (dtypes, block size, heads per kv head), never on the
   * batch, so a sequence's output does not depend on its batch. */
  PA_PARTITION_FIXED = 0,
  /* A length shaped to the batch: the fixed one, halved (down to 256 tokens)
   * while the batch's sequences x kv heads x partitions would leave the chip
   * short of workgroups.  Faster for a few long sequences (one 32K-token
   * grouped-query sequence: about 2x); the same as the fixed length for full
   * batches.  A sequence's output may then change, within float32
   * accumulation rounding, when the batch around it changes. */
  PA_PARTITION_FILL = 1
};

/*
 * pa_decode_partition_tokens -- the partition length (tokens, a positive
 * multiple of block_size) that `policy` picks for a pa_decode call of these
 * sizes, to be passed as partition_tokens to pa_decode_workspace_size and
 * pa_decode.  Host only: touches no device and no memory.  Returns a negative
 * status for sizes pa_decode_workspace_size would reject, and
 * PA_ERR_UNSUPPORTED for an unknown policy.
 * (Splitting a long context over workgroups and merging their partial softmax
 * results is the partitioning of [luoboask] section 3; the pages fix no
 * partition length.)
 */
int pa_decode_partition_tokens(int num_seqs, int num_heads, int num_kv_heads,
                               int head_dim, int block_size, int max_context_len,
                               int dtype, int cache_dtype, int policy);

/*
 * pa_decode_workspace_size -- bytes of device workspace pa_decode needs for
 * these sizes.  Long contexts are cut into partitions of `partition_tokens`
 * tokens (0 = the library's default for this shape); each partition leaves a
 * partial result (running max, running sum, unnormalised output) in float32
 * that a second kernel merges.  Returns 0 when no sequence can need more than
 * one partition (then pa_decode accepts workspace == NULL), and (size_t)-1 for
 * arguments pa_decode would reject.
 */
size_t pa_decode_workspace_size(int num_seqs, int num_heads, int num_kv_heads,
                                int head_dim, int block_size, int max_context_len,
                                int dtype, int cache_dtype, int partition_tokens);

/*
 * pa_decode -- single-query decode attention over the paged cache.
 * ([luoboask] section 3; [tbr8] "PagedAttention 的核心思想".)
 *
 * For every sequence s with L = context_lens[s] and every query head h, with
 * G = num_heads / num_kv_heads and kv head g = h / G (contiguous groups):
 *   K_t = k_cache[block_tables[s, t / block_size], g, t % block_size, :]
 *   V_t likewise, for t = 0 .. L-1 (for an fp8 cache: the codes' values times
 *   k_scale, resp. v_scale)
 *   w   = softmax_t(scale * dot(q[s, h, :], K_t))
 *   out[s, h, :] = sum_t w_t * V_t
 * accumulated in float32 and rounded to dtype (round-to-nearest-even for
 * bf16).  Supported (dtype, cache_dtype): (F32, F32), (BF16, BF16),
 * (BF16, FP8_E4M3); k_scale and v_scale are read only for an fp8 cache.
 * L == 0 gives an all-zero row.  Slots past L in the last block and table
 * entries past ceil(L / block_size) are never read, so they may hold anything
 * (NaN included).
 *
 * Arguments: max_blocks_per_seq is the row stride of block_tables;
 * max_context_len is an upper bound on every context_lens[s] (it sizes the
 * grid); num_blocks is the pool size; scale is usually 1/sqrt(head_dim);
 * partition_tokens: 0 = default, else a multiple of block_size, at most
 * 256 * block_size.  flags: 0 or PA_DECODE_SHARED_PAGES (any other bit gives
 * PA_ERR_UNSUPPORTED); the flag changes only the cache policy of the loads,
 * never the result.  The way a sequence is partitioned depends only on its own
 * length, so a sequence's output does not depend on the other sequences of the
 * batch or on which physical blocks hold its pages.
 * seq_order: NULL, or a device int32 [num_seqs] permutation of 0..num_seqs-1
 * giving the order in which sequences are dispatched; longest contexts first
 * shortens the tail of a ragged batch.  It never changes a result.  With NULL,
 * a batch of at most 256 sequences without PA_DECODE_SHARED_PAGES is
 * dispatched longest context first (ties by index), ranked in the kernel from
 * context_lens; other batches in index order.
 * Precondition: a permutation (entries outside [0, num_seqs) are skipped, and a
 * row whose index is missing is left unwritten).
 * workspace: device buffer of at least pa_decode_workspace_size(...) bytes with
 * 16-byte alignment (NULL allowed when that size is 0).
 * Preconditions (device values): 0 <= context_lens[s] <= max_context_len and
 * 0 <= block_tables[s, j] < num_blocks for j < ceil(L / block_size).  A row that
 * breaks them is written as NaN instead of being computed.
 */
int pa_decode(void* out, const void* q,
              const void* k_cache, const void* v_cache,
              const int32_t* block_tables, int max_blocks_per_seq,
              const int32_t* context_lens, const int32_t* seq_order,
              int num_seqs, int num_heads, int num_kv_heads, int head_dim,
              int block_size, int num_blocks, int max_context_len,
              float scale, int dtype, int cache_dtype, float k_scale, float v_scale,
              int partition_tokens, int flags,
              void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the static scratch buffer pa_decode_noalloc uses (32 MiB per GPU). */
#define PA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate memory:
 * code being captured into a HIP graph, tight serving loops, harnesses that
 * forbid hipMalloc.  It takes pa_decode's arguments without the workspace and
 * computes the same result with the same kernels (the same bits as pa_decode
 * with the same partition_tokens); the partial results of cut contexts go to
 * a static device buffer of PA_DECODE_NOALLOC_SCRATCH_BYTES bytes that the
 * library holds on every GPU it runs on until the process ends.  The call
 * allocates nothing: no hipMalloc, no hipFree, no allocating library routine.
 *
 * The buffer's device address is looked up on a GPU's first call that needs
 * it, with that GPU current (the GPU holding the call's buffers must be the
 * current device, as for every entry point).
 * Errors: the statuses of pa_decode, and PA_ERR_SCRATCH (nothing launched)
 * when pa_decode_workspace_size(...) for these arguments exceeds
 * PA_DECODE_NOALLOC_SCRATCH_BYTES -- e.g. at the default partitioning, 64
 * sequences x 64 heads (8 kv heads) x 32K-token contexts in 16-token pages
 * fit and 128 do not; in 32-token pages 128 fit and 256 do not.
 * All calls on one GPU share its buffer and nothing in it has to start at
 * zero: calls that overlap on one GPU (on different streams, or from several
 * threads) race on it and give unspecified results; serialise them.
 */
int pa_decode_noalloc(void* out, const void* q,
                      const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int max_blocks_per_seq,
                      const int32_t* context_lens, const int32_t* seq_order,
                      int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                      int block_size, int num_blocks, int max_context_len,
                      float scale, int dtype, int cache_dtype, float k_scale, float v_scale,
                      int partition_tokens, int flags, void* stream);

/*
 * pa_decode_shared_prefix_workspace_size -- bytes of device workspace
 * pa_decode_shared_prefix needs for these sizes and bounds (0 when nothing can
 * need a merge: no prefix and every context within one partition); (size_t)-1
 * for arguments it would reject.  partition_tokens: 0 = the call's default.
 */
size_t pa_decode_shared_prefix_workspace_size(int num_seqs, int num_heads, int num_kv_heads,
                                              int head_dim, int block_size, int max_context_len,
                                              int max_prefix_blocks, int max_tail_len,
                                              int dtype, int cache_dtype, int partition_tokens);

/*
 * pa_decode_shared_prefix -- pa_decode for a batch whose sequences share
 * leading cache blocks (beams forked from one sequence, or requests with a
 * common prompt), reading each shared page once for several sequences.
 * ([tbr8] "Copy-on-Write 与内存共享": beams and parallel samples of one request
 * share their common prefix, their block-table entries naming the same physical
 * pages until one of them writes; "Prefix Caching（前缀缓存）": requests with the
 * same system prompt share its blocks.)
 *
 * The result is the one pa_decode defines for the same q, caches, block_tables
 * and context_lens (the grouping below changes only which workgroup reads a
 * page, not what is computed; rounding may differ from pa_decode's within the
 * usual float32 accumulation error).
 *
 * Grouping (device int32 arrays [num_seqs]):
 *   prefix_leader[s]  the first sequence L of s's group (L == s for the first
 *                     member, or a sequence served alone); members of a group
 *                     are consecutive: L, L+1, ...
 *   prefix_blocks[L]  read at group leaders only: the number n of leading
 *                     block-table entries that every member of the group holds
 *                     in common (the shared blocks, each full: n * block_size
 *                     <= every member's context length).  0 = no sharing.
 * Members are served in chunks of 16 / G consecutive sequences counted from L
 * (G = num_heads / num_kv_heads): one workgroup computes the shared part of a
 * chunk, so each shared page is read once per chunk; a member's tokens past
 * the prefix are read by one of its chunk's prefix workgroups when they fit one
 * partition, else by its own workgroups; a merge kernel combines the partial
 * results.  An entry that does not describe such a chunk (L < 0, L > s,
 * prefix_leader[L] != L, or the first sequence of s's chunk in another group)
 * makes s a sequence served alone (its prefix is 0), with the same result.
 *
 * Host bounds, which size the grid (like max_context_len):
 *   max_prefix_blocks >= prefix_blocks[L] of every group, and
 *   max_tail_len      >= context_lens[s] - (its shared prefix in tokens) for
 *                        every s (the whole context for a sequence served alone),
 * with max_prefix_blocks * block_size and max_tail_len at most max_context_len
 * (else PA_ERR_SHAPE).
 * Preconditions (device values, as for pa_decode, plus): the bounds above; for
 * every member s of a group with n > 0, block_tables[s, j] == block_tables[c, j]
 * for j < n, where c is the first sequence of s's chunk; n * block_size <=
 * context_lens[s].  A member that breaks them gets a NaN row (if the first
 * sequence of a chunk has an out-of-range table entry, the whole chunk's rows
 * are NaN).
 *
 * Arguments not listed here mean what they mean for pa_decode.  dtype must be
 * PA_BF16 (cache PA_BF16 or PA_FP8_E4M3); G may be 1, 2, 4 or 8; flags must be
 * 0.  partition_tokens cuts the shared prefix and the rest of each context
 * separately (0 = default: a quarter of max_prefix_blocks * block_size rounded
 * up to a power of two, within [256, 2048]).  workspace: at least
 * pa_decode_shared_prefix_workspace_size(...) bytes, 16-byte aligned (NULL
 * allowed when that is 0).
 */
int pa_decode_shared_prefix(void* out, const void* q,
                            const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int max_blocks_per_seq,
                            const int32_t* context_lens,
                            const int32_t* prefix_leader, const int32_t* prefix_blocks,
                            int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                            int block_size, int num_blocks, int max_context_len,
                            int max_prefix_blocks, int max_tail_len,
                            float scale, int dtype, int cache_dtype, float k_scale, float v_scale,
                            int partition_tokens, int flags,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_multi_query_workspace_size -- bytes of device workspace pa_multi_query
 * needs: the partitions of cut contexts and room for the list of work items
 * it builds on the device each call for batches of more than 64 sequences
 * (smaller batches find their items in the kernels; the size does not depend
 * on that) (0 when there are no sequences or no query tokens);
 * (size_t)-1 for arguments it would reject.  partition_tokens: 0 = the
 * default pa_multi_query picks for the same shape (see there).
 */
size_t pa_multi_query_workspace_size(int num_seqs, int num_query_tokens, int num_heads,
                                     int num_kv_heads, int head_dim, int block_size,
                                     int max_context_len, int dtype, int cache_dtype,
                                     int partition_tokens);

/*
 * pa_multi_query -- causal attention of several new query tokens per sequence
 * over the paged cache: a chunk of a long prompt processed between decode steps,
 * or drafted tokens being verified.  ([tbr8] "Chunked Prefill（分块预填充）": a long
 * prefill is cut into chunks interleaved with decoding; "结合 Speculative Decoding
 * 加速": the large model checks N drafted tokens in one pass.)
 *
 * query_start: device int32 [num_seqs + 1]; sequence s owns rows
 * query_start[s] .. query_start[s+1] - 1 of q and out ([num_query_tokens,
 * num_heads, head_dim], bf16).  With n = its row count and L = context_lens[s]
 * (cached tokens, the n new ones included: their K/V were stored with
 * pa_reshape_and_cache), row query_start[s] + i is the token at position
 * p = L - n + i and, for every query head h (kv head h / G),
 *   out[row, h, :] = sum_{t <= p} softmax_t(scale * dot(q[row, h, :], K_t)) * V_t
 * with K_t, V_t reached through block_tables as for pa_decode (E4M3 caches times
 * k_scale / v_scale).  Accumulation in float32, output rounded to bf16 (RNE).
 * A sequence with n == 1 is a decode step.
 *
 * dtype must be PA_BF16 (cache PA_BF16 or PA_FP8_E4M3); G = num_heads /
 * num_kv_heads in {1, 2, 4, 8}; head_dim 64 or 128; block_size 16 or 32.
 * max_query_len >= every n and max_context_len >= every L (host bounds that size
 * the grid); ceil(max_query_len * G / 64) and the number of partitions of
 * max_context_len must each stay below 2^15 (else PA_ERR_UNSUPPORTED).  A sequence with n == 1 is a decode step and runs through
 * pa_decode's kernels (with their partitioning) unless flags holds
 * PA_MULTI_QUERY_TILES_ONLY (other flag bits than the two above:
 * PA_ERR_UNSUPPORTED).
 * Streams: when a batch has decode rows and longer chunks and `side` is not
 * NULL, the decode kernels (bound by the cache reads) run on side->stream
 * beside the multi-query kernels (bound by the matrix cores) on `stream`.
 * side->stream is forked from `stream` and joined back to it with the two
 * events, so the call is ordered on `stream` like a single launch.  With
 * side == NULL or PA_MULTI_QUERY_ONE_STREAM every launch goes to `stream`.
 * The side handle must be on the device of the call and serve no other call
 * at the same time.
 * partition_tokens (0 = chosen from the
 * shape: the smallest of 512, 1024 and 2048 for which num_seqs * num_kv_heads
 * * ceil(max_context_len / partition_tokens) <= 1024, else 2048; otherwise a
 * positive multiple of block_size): a sequence with n > 1 whose n * G rows
 * fit in 64 has its context cut into partitions of this many tokens, merged
 * by a second kernel; longer chunks are not cut.  The cut changes the
 * rounding of a row's result, so a caller that needs rows bitwise
 * independent of the rest of the batch passes a fixed partition_tokens (and
 * query ranges that cover every row of q: where rows belong to no sequence,
 * a short sequence may run uncut, with the same result up to rounding).
 * workspace: at least pa_multi_query_workspace_size(...) bytes, 16-byte
 * aligned.
 * Preconditions (device values): query_start ranges inside [0, num_query_tokens],
 * non-decreasing, n <= max_query_len (a sequence breaking these is skipped and
 * its rows are left unwritten; overlapping ranges give unspecified rows);
 * n <= L <= max_context_len (all rows of a sequence breaking these are NaN)
 * and table entries in [0, num_blocks) for the pages of the context (a bad
 * entry makes NaN every row that attends to its page, and possibly other rows
 * of the same sequence: those that share the bad row's block of 64 or 128
 * rows).  Rows of no sequence are left unwritten.
 */
int pa_multi_query(void* out, const void* q,
                   const void* k_cache, const void* v_cache,
                   const int32_t* block_tables, int max_blocks_per_seq,
                   const int32_t* context_lens, const int32_t* query_start,
                   int num_seqs, int num_query_tokens, int max_query_len,
                   int num_heads, int num_kv_heads, int head_dim,
                   int block_size, int num_blocks, int max_context_len,
                   float scale, int dtype, int cache_dtype, float k_scale, float v_scale,
                   int partition_tokens, int flags,
                   void* workspace, size_t workspace_bytes,
                   const pa_side_stream* side, void* stream);

/* pa_status_string -- static, human-readable name of a status code. */
const char* pa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
