// gfx950 kernels for decode attention over a paged KV cache.
//
// What is computed: "vLLM 深度解读" (luoboask.github.io), section 3
// "PagedAttention CUDA Kernel" -- for each (sequence, query head), scores
// scale * q.k for every context token reached through the block table, a
// softmax over them kept as a running (max, sum) pair, and the weighted sum of
// V; section 7 -- new tokens' K/V are stored into their cache slots first;
// "详解vLLM推理引擎架构：PagedAttention原理与LLM高效部署实践" (tbr8.org),
// "Copy-on-Write 与内存共享" -- whole-block copies before a shared block is
// written.
//
// How (MI355X-first, not the page's CUDA sketch):
//  * Cache layout [num_blocks, num_kv_heads, block_size, head_dim]: a
//    (block, kv head) page is one contiguous block_size x head_dim tile.  Each
//    wave reads a page with 16-byte loads, one token row per D/VEC lanes, so a
//    load instruction moves 1 KiB of contiguous memory straight into the
//    registers that consume it (no LDS round trip: nothing is reused).
//  * Scores are reduced across the lanes of a token row with xor shuffles; the
//    online softmax state (max, sum, accumulator) is kept per row, so no
//    cross-row traffic happens inside the page loop; rows and waves are merged
//    once per partition.
//  * The next page's loads are in flight while the current page is consumed
//    (two register buffers).  Page ids of a wave's pages sit one per lane and
//    are read with readlane, so the table walk costs one coalesced load.
//  * Long contexts are cut into partitions of a fixed number of tokens (a
//    function of the sequence's own length only); a second kernel merges the
//    partitions' (max, sum, accumulator) with the log-sum-exp rule.
//  * exp is exp2 (v_exp_f32) with log2(e) folded into the query scale.

#include <float.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

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
  float* ws_ml;
  float* ws_acc;
  int64_t block_stride;  // elements between consecutive physical blocks
  int max_blocks_per_seq;
  int num_heads;
  int num_blocks;
  int max_context_len;
  int partition_tokens;
  int max_parts;
  float scale_log2e;
};

__device__ __forceinline__ int parts_for(int ctx, int partition_tokens) {
  return ctx <= partition_tokens ? 1 : (ctx + partition_tokens - 1) / partition_tokens;
}

// One workgroup = kWaves waves = one (partition, kv head, sequence); it serves
// the G query heads that share the kv head.
template <typename T, int D, int BS, int G>
__global__ __launch_bounds__(kWaves * 64) void decode_partition_kernel(DecodeParams p) {
  using E = Elem<T>;
  constexpr int VEC = E::kVec;
  constexpr int LPT = D / VEC;   // lanes per token row
  constexpr int TPL = 64 / LPT;  // token rows per wave-wide load
  constexpr int NLD = BS / TPL;  // loads per page
  static_assert(D % VEC == 0 && 64 % LPT == 0 && BS % TPL == 0, "tile shape");

  const int part = blockIdx.x;
  const int kvh = blockIdx.y;
  const int s = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row = lane / LPT;
  const int col = lane % LPT;

  const int ctx = p.context_lens[s];
  const bool ctx_bad = ctx < 0 || ctx > p.max_context_len;
  const int nparts = ctx_bad ? 1 : parts_for(ctx, p.partition_tokens);
  if (part >= nparts) return;  // uniform over the workgroup

  const int tok0 = part * p.partition_tokens;
  const int tok1 = ctx_bad ? tok0 : min(ctx, tok0 + p.partition_tokens);
  const int pg0 = tok0 / BS;
  const int npg = (tok1 - tok0 + BS - 1) / BS;
  const int nk = npg > wave ? (npg - wave + kWaves - 1) / kWaves : 0;  // <= 64

  // Physical ids of this wave's pages, one per lane.
  int my_id = 0;
  bool id_bad = false;
  if (lane < nk) {
    my_id = p.block_tables[(int64_t)s * p.max_blocks_per_seq + pg0 + wave + lane * kWaves];
    id_bad = my_id < 0 || my_id >= p.num_blocks;
    if (id_bad) my_id = 0;
  }
  const bool bad = ctx_bad || __any(id_bad);

  // Query rows of the group, pre-scaled by scale * log2(e).
  float qf[G][VEC];
  {
    const T* qb = static_cast<const T*>(p.q) + ((int64_t)s * p.num_heads + (int64_t)kvh * G) * D + col * VEC;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint4 r = *reinterpret_cast<const uint4*>(qb + g * D);
      E::unpack(r, qf[g]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) qf[g][e] *= p.scale_log2e;
    }
  }

  float m[G], l[G], acc[G][VEC];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -FLT_MAX;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[g][e] = 0.f;
  }

  const T* kbase = static_cast<const T*>(p.k_cache) + (int64_t)kvh * BS * D + row * D + col * VEC;
  const T* vbase = static_cast<const T*>(p.v_cache) + (int64_t)kvh * BS * D + row * D + col * VEC;

  auto load_page = [&](int k, uint4 (&kr)[NLD], uint4 (&vr)[NLD]) {
    const int64_t phys = __builtin_amdgcn_readlane(my_id, k);
    const T* kp = kbase + phys * p.block_stride;
    const T* vp = vbase + phys * p.block_stride;
#pragma unroll
    for (int i = 0; i < NLD; ++i) kr[i] = *reinterpret_cast<const uint4*>(kp + i * TPL * D);
#pragma unroll
    for (int i = 0; i < NLD; ++i) vr[i] = *reinterpret_cast<const uint4*>(vp + i * TPL * D);
  };

  auto consume_page = [&](int k, const uint4 (&kr)[NLD], uint4 (&vr)[NLD]) {
    const int t0 = (pg0 + wave + k * kWaves) * BS;  // logical token of slot 0
    const bool full = t0 + BS <= tok1;
    float sc[G][NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      float kf[VEC];
      E::unpack(kr[i], kf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) a = fmaf(qf[g][e], kf[e], a);
        sc[g][i] = a;
      }
    }
#pragma unroll
    for (int off = 1; off < LPT; off <<= 1) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < NLD; ++i) sc[g][i] += __shfl_xor(sc[g][i], off);
    }
    bool valid[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) valid[i] = full || (t0 + i * TPL + row < tok1);
    if (!full) {
      // Slots past the context may hold anything (NaN included): drop them
      // by selection, never by multiplying with a zero weight.
#pragma unroll
      for (int i = 0; i < NLD; ++i)
        if (!valid[i]) vr[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    float pw[G][NLD];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = m[g];
#pragma unroll
      for (int i = 0; i < NLD; ++i)
        if (valid[i]) mx = fmaxf(mx, sc[g][i]);
      const float alpha = fast_exp2(m[g] - mx);
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        pw[g][i] = valid[i] ? fast_exp2(sc[g][i] - mx) : 0.f;
        psum += pw[g][i];
      }
      l[g] = l[g] * alpha + psum;
      m[g] = mx;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[g][e] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      float vf[VEC];
      E::unpack(vr[i], vf);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[g][e] = fmaf(pw[g][i], vf[e], acc[g][e]);
    }
  };

  if (!bad && nk > 0) {
    uint4 ka[NLD], va[NLD], kb[NLD], vb[NLD];
    load_page(0, ka, va);
    for (int k = 0; k < nk; k += 2) {
      if (k + 1 < nk) load_page(k + 1, kb, vb);
      consume_page(k, ka, va);
      if (k + 1 < nk) {
        if (k + 2 < nk) load_page(k + 2, ka, va);
        consume_page(k + 1, kb, vb);
      }
    }
  }

  // Merge the token rows of the wave (lanes with the same col).
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(m[g], off);
      const float lo = __shfl_xor(l[g], off);
      const float mn = fmaxf(m[g], mo);
      const float a = fast_exp2(m[g] - mn);
      const float b = fast_exp2(mo - mn);
      l[g] = l[g] * a + lo * b;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[g][e] = acc[g][e] * a + __shfl_xor(acc[g][e], off) * b;
      m[g] = mn;
    }
  }

  // Merge the waves through LDS.
  __shared__ float sm_acc[kWaves][G][D];
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  if (row == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < VEC; ++e) sm_acc[wave][g][col * VEC + e] = acc[g][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      sm_m[wave][g] = bad ? 0.f : m[g];
      sm_l[wave][g] = bad ? __builtin_nanf("") : l[g];
    }
  }
  __syncthreads();

  for (int idx = tid; idx < G * D; idx += kWaves * 64) {
    const int g = idx / D;
    const int d = idx % D;
    float mm = -FLT_MAX;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, sm_m[w][g]);
    float ll = 0.f, aa = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = fast_exp2(sm_m[w][g] - mm);
      ll += sm_l[w][g] * wt;
      aa += sm_acc[w][g][d] * wt;
    }
    const int64_t sh = (int64_t)s * p.num_heads + (int64_t)kvh * G + g;
    if (nparts == 1) {
      const float o = (ll == 0.f) ? 0.f : aa / ll;
      E::store(static_cast<T*>(p.out) + sh * D + d, o);
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

// Merge of the partitions of one (sequence, head): log-sum-exp combination of
// the partial (max, sum, accumulator) triples, then normalisation and the cast.
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_reduce_kernel(DecodeParams p) {
  using E = Elem<T>;
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int ctx = p.context_lens[s];
  if (ctx < 0 || ctx > p.max_context_len) return;  // written as NaN by the partition kernel
  const int nparts = parts_for(ctx, p.partition_tokens);
  if (nparts <= 1) return;
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
    E::store(static_cast<T*>(p.out) + ((int64_t)s * p.num_heads + h) * D + d, o);
  }
}

// ---------------------------------------------------------------------------
// Cache writes
// ---------------------------------------------------------------------------

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

template <typename T, int D, int BS, int G>
hipError_t launch_decode_t(const DecodeLaunch& a, const DecodeParams& p) {
  dim3 grid(a.max_parts, a.num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_partition_kernel<T, D, BS, G>), grid, dim3(kWaves * 64), 0, a.stream, p);
  if (a.max_parts > 1) {
    hipLaunchKernelGGL((decode_reduce_kernel<T, D>), dim3(a.num_heads, a.num_seqs), dim3(64), 0,
                       a.stream, p);
  }
  return hipGetLastError();
}

template <typename T, int D, int BS>
hipError_t dispatch_group(const DecodeLaunch& a, const DecodeParams& p) {
  switch (a.num_heads / a.num_kv_heads) {
    case 1: return launch_decode_t<T, D, BS, 1>(a, p);
    case 2: return launch_decode_t<T, D, BS, 2>(a, p);
    case 4: return launch_decode_t<T, D, BS, 4>(a, p);
    case 8: return launch_decode_t<T, D, BS, 8>(a, p);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int D>
hipError_t dispatch_bs(const DecodeLaunch& a, const DecodeParams& p) {
  return a.block_size == 16 ? dispatch_group<T, D, 16>(a, p) : dispatch_group<T, D, 32>(a, p);
}

template <typename T>
hipError_t dispatch_d(const DecodeLaunch& a, const DecodeParams& p) {
  return a.head_dim == 64 ? dispatch_bs<T, 64>(a, p) : dispatch_bs<T, 128>(a, p);
}

}  // namespace

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
  return a.dtype == 0 ? dispatch_d<float>(a, p) : dispatch_d<uint16_t>(a, p);
}

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
