// Device-side pieces shared by the decode kernels: element access, the
// launch parameter block, the partition arithmetic and the workgroup epilogue
// that merges the waves' online-softmax states.
#ifndef PA_DEVICE_H_
#define PA_DEVICE_H_

#include <float.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {

constexpr float kLog2e = 1.4426950408889634f;

// Lazy online-softmax rescaling threshold (log2 units): weights computed
// against a stale reference max stay below 2^8 = 256.
constexpr float kRescaleLog2 = 8.f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// bf16 is handled as raw uint16_t bits: widening puts the 16 bits on top of a
// binary32 word (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even binary32 -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load with the non-temporal hint.  Cache pages are read once per
// decode step, so their lines should not displace others; on MI355X random
// 4-8 KiB page reads measured 6.35-6.60 TB/s with the hint against
// 5.80-5.97 TB/s without.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return __builtin_bit_cast(uint4, v);
}

// Page load: non-temporal unless pages may be shared between sequences.
template <bool kNonTemporal>
__device__ __forceinline__ uint4 load_page16(const void* p) {
  if constexpr (kNonTemporal) return load_stream16(p);
  return *reinterpret_cast<const uint4*>(p);
}

// Sum over groups of LPT consecutive lanes (LPT a power of two); every lane
// of a group receives the group's total.  Steps inside a 16-lane row use DPP
// (quad permutes, half-row and row mirrors), so they fold into the adds.
template <int LPT>
__device__ __forceinline__ float row_sum(float x) {
  auto dpp = [](float v, int ctrl) -> float {
    switch (ctrl) {  // the control word must be a constant at each call site
      case 0xB1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
      case 0x4E: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
      case 0x141: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
      default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    }
  };
  if constexpr (LPT >= 2) x += dpp(x, 0xB1);   // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (LPT >= 4) x += dpp(x, 0x4E);   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (LPT >= 8) x += dpp(x, 0x141);  // row_half_mirror: quads of an 8-lane half swap
  if constexpr (LPT >= 16) x += dpp(x, 0x140); // row_mirror: the two halves of a row swap
  if constexpr (LPT >= 32) x += __shfl_xor(x, 16);
  if constexpr (LPT >= 64) x += __shfl_xor(x, 32);
  return x;
}

template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static constexpr int kVec = 4;  // elements per 16-byte load
  __device__ static __forceinline__ void unpack(const uint4& r, float* f) {
    f[0] = __uint_as_float(r.x);
    f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z);
    f[3] = __uint_as_float(r.w);
  }
  __device__ static __forceinline__ void store(float* p, float v) { *p = v; }
};

// OCP E4M3 codes (gfx950's fp8 format: bias 7, largest finite 448, no
// infinities).  Widening uses v_cvt_pk_f32_fp8, exact for every code.
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* f) {
  const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
  const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
  f[0] = lo.x;
  f[1] = lo.y;
  f[2] = hi.x;
  f[3] = hi.y;
}

// Nearest finite E4M3 code of x, ties to even, |x| >= 448 saturating to 448,
// NaN to 0x7F (with the sign of x).  Written on the binary32 bit pattern:
// below 2^-6 the code is the integer nearest x * 2^9; above, the 23-bit
// mantissa is rounded to 3 bits in place (a carry moves into the exponent) and
// the exponent is re-biased from 127 to 7.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;       // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;      // >= 448 (and inf): saturate
  if (a < 0x3c800000u) {                          // < 2^-6: multiples of 2^-9
    return sign | static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.f));
  }
  const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
  const uint32_t code = (r >> 20) - (120u << 3);
  return sign | (code > 0x7eu ? 0x7eu : code);
}

template <>
struct Elem<uint8_t> {
  static constexpr int kVec = 16;
  __device__ static __forceinline__ void unpack(const uint4& r, float* f) {
    fp8x4_to_f32(r.x, f);
    fp8x4_to_f32(r.y, f + 4);
    fp8x4_to_f32(r.z, f + 8);
    fp8x4_to_f32(r.w, f + 12);
  }
};

template <>
struct Elem<uint16_t> {
  static constexpr int kVec = 8;
  __device__ static __forceinline__ void unpack(const uint4& r, float* f) {
    f[0] = bf16_lo(r.x);
    f[1] = bf16_hi(r.x);
    f[2] = bf16_lo(r.y);
    f[3] = bf16_hi(r.y);
    f[4] = bf16_lo(r.z);
    f[5] = bf16_hi(r.z);
    f[6] = bf16_lo(r.w);
    f[7] = bf16_hi(r.w);
  }
  __device__ static __forceinline__ void store(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }
};

struct DecodeParams {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* seq_order;  // null = natural order
  float* ws_ml;
  float* ws_acc;
  int64_t block_stride;  // elements between consecutive physical blocks
  int max_blocks_per_seq;
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int num_blocks;
  int max_context_len;
  int partition_tokens;
  int max_parts;
  float scale_log2e;  // softmax scale * log2(e), times k_scale for fp8 caches
  float v_scale;      // multiplies the output (1 unless the cache holds fp8 codes)
  // Shared-prefix decode only (prefix_leader == null otherwise).
  const int32_t* prefix_leader;  // [num_seqs] first member of the sequence's group
  const int32_t* prefix_blocks;  // [num_seqs] shared leading blocks, read at group leaders
  int chunk_seqs;                // members one prefix workgroup serves (16 / G)
  int block_size;
  int max_prefix_blocks;         // caller's bound on prefix_blocks
  int max_tail_len;              // caller's bound on context_len - shared prefix
  int prefix_parts;              // grid rows per sequence for prefix partitions
  int tail_parts;                // grid rows per sequence for the rest
  // Decode rows of a multi-query batch (query_start == null otherwise): only
  // sequences with exactly one new query are served, at q / out row
  // query_start[s], and a context must hold that query (min_context = 1).
  const int32_t* query_start;
  int num_query_rows;
  int min_context;
  int order_by_length;  // no seq_order, pages not shared, at most kOrderedSeqs sequences
};

// q / out row of sequence s: s itself, or in a multi-query batch its one
// query's row (-1: the sequence has another number of queries, or an invalid
// range, and is not served by the decode kernels).
__device__ __forceinline__ int query_row(const DecodeParams& p, int s) {
  if (p.query_start == nullptr) return s;
  const int t0 = p.query_start[s];
  const int t1 = p.query_start[s + 1];
  return (t1 - t0 == 1 && t0 >= 0 && t1 <= p.num_query_rows) ? t0 : -1;
}

// Without a caller's order, a batch of at most kOrderedSeqs sequences whose
// pages are not shared is dispatched longest context first (equal lengths:
// lower index first), so that with mixed lengths no long sequence starts
// after the short ones have taken the CUs (decode rows of a chunked-prefill
// batch, 64 sequences of 128-4096 tokens, alone: 439.5 -> 421.9 us).  Shared
// pages keep the caller's order, which places the sequences that read the
// same pages next to each other.  Each wave selects the sequence of rank z
// itself, bit by bit from the top of the length over wave ballots (lane i
// holds sequences i, 64 + i, ...); sequences the decode kernels do not serve
// (another number of queries) rank last.  Every lane of the wave must be
// active.
constexpr int kOrderedSeqs = 256;
__device__ __forceinline__ int ranked_sequence(const DecodeParams& p, int z) {
  constexpr int K = kOrderedSeqs / 64;
  const int lane = threadIdx.x & 63;
  int key[K];
  uint64_t m[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int s = 64 * k + lane;
    key[k] = 0;
    m[k] = 0;
    if (64 * k < p.num_seqs) {  // uniform
      const bool in = s < p.num_seqs;
      if (in && query_row(p, s) >= 0) key[k] = 1 + min(max(p.context_lens[s], 0), p.max_context_len);
      m[k] = __ballot(in);
    }
  }
  int r = z;
  for (int bit = 31 - __clz(p.max_context_len + 1); bit >= 0; --bit) {
    uint64_t ones[K];
    int c = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      ones[k] = 0;
      if (64 * k < p.num_seqs) {
        ones[k] = __ballot((key[k] >> bit) & 1) & m[k];
        c += __popcll(ones[k]);
      }
    }
    const bool high = r < c;  // rank z lies among the sequences with this bit set
    if (!high) r -= c;
#pragma unroll
    for (int k = 0; k < K; ++k) m[k] = high ? ones[k] : m[k] & ~ones[k];
  }
  // m: the sequences of the selected length; z is the r-th of them.
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int cnt = __popcll(m[k]);
    if (r < cnt) {
      const bool hit = ((m[k] >> lane) & 1) && __popcll(m[k] & ((1ull << lane) - 1)) == r;
      return 64 * k + __builtin_ctzll(__ballot(hit));
    }
    r -= cnt;
  }
  return -1;
}

// Sequence served by grid slot z (the caller may reorder dispatch); -1 if the
// order array names no valid sequence there.
__device__ __forceinline__ int sequence_of(const DecodeParams& p, int z) {
  if (p.seq_order == nullptr) return p.order_by_length ? ranked_sequence(p, z) : z;
  const int s = p.seq_order[z];
  return (s >= 0 && s < p.num_seqs) ? s : -1;
}
__device__ __forceinline__ int parts_for(int ctx, int partition_tokens) {
  return ctx <= partition_tokens ? 1 : (ctx + partition_tokens - 1) / partition_tokens;
}

// Where one workgroup's work lies: partition `part` of sequence `s`, its
// token range [tok0, tok1) and the pages dealt to this wave.  A context
// length outside [0, max_context_len] marks the row bad (written as NaN).
struct PartitionRange {
  int ctx, nparts, tok0, tok1, pg0, npg, nk;
  bool ctx_bad;
};

__device__ __forceinline__ PartitionRange partition_range(const DecodeParams& p, int s, int part,
                                                          int wave, int block_size) {
  PartitionRange r;
  r.ctx = p.context_lens[s];
  r.ctx_bad = r.ctx < p.min_context || r.ctx > p.max_context_len;
  r.nparts = r.ctx_bad ? 1 : parts_for(r.ctx, p.partition_tokens);
  r.tok0 = part * p.partition_tokens;
  r.tok1 = r.ctx_bad ? r.tok0 : min(r.ctx, r.tok0 + p.partition_tokens);
  r.pg0 = r.tok0 / block_size;
  r.npg = r.tok1 > r.tok0 ? (r.tok1 - r.tok0 + block_size - 1) / block_size : 0;
  r.nk = r.npg > wave ? (r.npg - wave + kWaves - 1) / kWaves : 0;  // <= 64
  return r;
}

// Physical ids of this wave's pages (page pg0 + wave + k*kWaves for lane k),
// one per lane.  Ids outside [0, num_blocks) are replaced by 0 and reported.
__device__ __forceinline__ int load_page_ids(const DecodeParams& p, int s, const PartitionRange& r,
                                             int wave, int lane, bool* any_bad) {
  int id = 0;
  bool bad = false;
  if (lane < r.nk) {
    id = p.block_tables[(int64_t)s * p.max_blocks_per_seq + r.pg0 + wave + lane * kWaves];
    bad = id < 0 || id >= p.num_blocks;
    if (bad) id = 0;
  }
  *any_bad = __any(bad);
  return id;
}

// Shared-prefix decode.  Sequence s names the first member L of its group in
// prefix_leader[s]; the group's members hold the same physical blocks in their
// first prefix_blocks[L] table entries.  Members are served in chunks of
// chunk_seqs consecutive sequences counted from L, and one workgroup reads each
// shared page once for a whole chunk.  A sequence whose entry does not describe
// such a chunk (L out of range or not its own leader, or the first sequence of
// its chunk in another group) is served alone, which computes the same result.
// Every kernel derives this from the same device values, so they agree.
struct PrefixChunk {
  int leader;  // the group's first member (s itself when served alone)
  int chunk;   // first member of s's chunk (s itself when served alone)
  int blocks;  // shared leading blocks, 0 = none
};
__device__ __forceinline__ PrefixChunk prefix_chunk(const DecodeParams& p, int s) {
  PrefixChunk c{s, s, 0};
  if (p.prefix_leader == nullptr) return c;
  const int lead = p.prefix_leader[s];
  if (lead < 0 || lead > s || p.prefix_leader[lead] != lead) return c;
  const int first = lead + (s - lead) / p.chunk_seqs * p.chunk_seqs;
  if (p.prefix_leader[first] != lead) return c;
  const int nb = p.prefix_blocks[lead];
  if (nb <= 0) return c;
  c.leader = lead;
  c.chunk = first;
  c.blocks = nb;
  return c;
}
// How a sequence's context is cut: the shared prefix [0, prefix) into nprefix
// partitions (computed by its chunk's workgroups, partition slots 0 ..
// nprefix-1), the rest [prefix, ctx) into ntail partitions (its own
// workgroups, slots nprefix ..).  A chunk member (index `member` in its
// chunk, -1 when served alone) whose rest fits one partition is folded: its
// chunk's workgroup of prefix partition member % nprefix reads it too (for
// that member's columns only), into the same slot, and ntail is 0.  Without
// a prefix this is the plain partitioning.  A bad row (context length out of
// range, shorter than the declared prefix, or past the caller's prefix or
// tail bound) has one partition and is written as NaN.
struct SeqSplit {
  int ctx, prefix, nprefix, ntail;
  bool bad;
  bool folded;
};
__device__ __forceinline__ SeqSplit split_context(const DecodeParams& p, int ctx, int prefix_blocks,
                                                  int member) {
  SeqSplit r;
  r.ctx = ctx;
  r.folded = false;
  const int64_t pre = (int64_t)prefix_blocks * p.block_size;
  r.bad = ctx < 0 || ctx > p.max_context_len || pre > ctx;
  if (p.prefix_leader != nullptr)  // the caller's bounds size the grid
    r.bad = r.bad || prefix_blocks > p.max_prefix_blocks || ctx - pre > p.max_tail_len;
  r.prefix = r.bad ? 0 : (int)pre;
  const int pt = p.partition_tokens;
  if (r.bad) {
    r.nprefix = 0;
    r.ntail = 1;
  } else if (r.prefix == 0) {
    r.nprefix = 0;
    r.ntail = parts_for(ctx, pt);
  } else {
    r.nprefix = (r.prefix + pt - 1) / pt;
    r.ntail = (ctx - r.prefix + pt - 1) / pt;
    r.folded = member >= 0 && r.ntail == 1;
    if (r.folded) r.ntail = 0;
  }
  return r;
}
// Page range of the tokens [tok0, tok1) (tok0 a multiple of block_size) and
// this wave's share of it.
__device__ __forceinline__ PartitionRange token_range(int ctx, int nparts, int tok0, int tok1, bool bad,
                                                      int wave, int block_size) {
  PartitionRange r;
  r.ctx = ctx;
  r.ctx_bad = bad;
  r.nparts = nparts;
  r.tok0 = tok0;
  r.tok1 = bad ? tok0 : tok1;
  r.pg0 = tok0 / block_size;
  r.npg = r.tok1 > r.tok0 ? (r.tok1 - r.tok0 + block_size - 1) / block_size : 0;
  r.nk = r.npg > wave ? (r.npg - wave + kWaves - 1) / kWaves : 0;
  return r;
}
// Epilogue: the kWaves partial states of each query head of the group sit in
// LDS (sm_acc [kWaves][G][D], sm_m / sm_l [kWaves][G]); merge them with the
// log-sum-exp rule and write either the final row (single partition, at q /
// out row `row`) or the partition's (max, sum, accumulator) triple to the
// workspace (indexed by sequence).
template <typename T, int D, int G>
__device__ __forceinline__ void merge_waves_and_store(const DecodeParams& p, const float* sm_acc,
                                                      const float* sm_m, const float* sm_l, int s,
                                                      int kvh, int part, int nparts, int row) {
  for (int idx = threadIdx.x; idx < G * D; idx += kWaves * 64) {
    const int g = idx / D;
    const int d = idx % D;
    float mm = -FLT_MAX;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, sm_m[w * G + g]);
    float ll = 0.f, aa = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = fast_exp2(sm_m[w * G + g] - mm);
      ll += sm_l[w * G + g] * wt;
      aa += sm_acc[(w * G + g) * D + d] * wt;
    }
    const int64_t sh = (int64_t)s * p.num_heads + (int64_t)kvh * G + g;
    if (nparts == 1) {
      const float o = (ll == 0.f) ? 0.f : aa * p.v_scale / ll;
      Elem<T>::store(static_cast<T*>(p.out) + ((int64_t)row * p.num_heads + (int64_t)kvh * G + g) * D + d, o);
    } else {
      const int64_t slot = sh * p.max_parts + part;
      p.ws_acc[slot * D + d] = aa;
      if (d == 0) {
        p.ws_ml[slot * 2] = mm;
        p.ws_ml[slot * 2 + 1] = ll;
      }
    }
  }
}

// Kernel launchers of the two decode-partition variants (one per file).
hipError_t launch_partition_valu(const DecodeLaunch& a, const DecodeParams& p);
hipError_t launch_partition_mfma(const DecodeLaunch& a, const DecodeParams& p);

}  // namespace pa

#endif  // PA_DEVICE_H_
