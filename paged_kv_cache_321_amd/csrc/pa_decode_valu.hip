// Decode partition kernel on the vector ALUs: used when every page serves one
// query head (no grouping), for fp32 caches, and as the general fallback.
// Caches may hold bf16, fp32 or E4M3 fp8 codes (16 per 16-byte load, widened
// with v_cvt_pk_f32_fp8; k_scale is folded into the score scale and v_scale
// into the final normalisation).
//
// What is computed: "vLLM 深度解读" (luoboask.github.io), section 3
// "PagedAttention CUDA Kernel" -- per (sequence, query head), scale * q.k for
// every context token reached through the block table, a softmax kept as a
// running (max, sum) pair, and the weighted sum of V.
//
// How (MI355X-first, not the page's CUDA sketch):
//  * A (block, kv head) page is one contiguous block_size x head_dim tile.
//    Each wave reads it with 16-byte loads, one token row per D/VEC lanes, so
//    a load instruction moves 1 KiB of contiguous memory straight into the
//    registers that consume it (nothing is reused, so no LDS round trip).
//  * bf16 scores use v_dot2_f32_bf16 on packed pairs; the partial scores are
//    summed across the lanes of a token row with DPP adds; the
//    online-softmax state (max, sum, accumulator) is kept per row, so no
//    cross-row traffic happens inside the page loop; rows and waves are merged
//    once per partition.
//  * Page loads carry the non-temporal hint (each page is read once), unless
//    the caller says pages may be shared between sequences.
//  * The next page's loads are in flight while the current page is consumed
//    (two register buffers).  The page ids of a wave sit one per lane and are
//    read with readlane, so the table walk is one coalesced load.
//  * exp is exp2 (v_exp_f32) with log2(e) folded into the query scale.

#include "pa_device.h"

namespace pa {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// a.x * b.x + a.y * b.y + c over packed bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// One workgroup = kWaves waves = one (partition, kv head, sequence); it serves
// the G query heads that share the kv head.  TQ is the query/output element
// type (float or bf16 bits), TC the cache element type (the same, or E4M3
// codes with a bf16 query).
template <typename TQ, typename TC, int D, int BS, int G, bool NONTEMPORAL>
__global__ __launch_bounds__(kWaves * 64) void decode_partition_valu_kernel(DecodeParams p) {
  using E = Elem<TC>;
  constexpr int VEC = E::kVec;  // cache elements per 16-byte load
  constexpr int LPT = D / VEC;   // lanes per token row
  constexpr int TPL = 64 / LPT;  // token rows per wave-wide load
  constexpr int NLD = BS / TPL;  // loads per page
  static_assert(D % VEC == 0 && 64 % LPT == 0 && BS % TPL == 0, "tile shape");

  const int part = blockIdx.x;
  const int kvh = blockIdx.y;
  const int s = sequence_of(p, blockIdx.z);
  if (s < 0) return;  // uniform over the workgroup
  const int qrow = query_row(p, s);
  if (qrow < 0) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row = lane / LPT;
  const int col = lane % LPT;

  const PartitionRange r = partition_range(p, s, part, wave, BS);
  if (part >= r.nparts) return;  // uniform over the workgroup
  const int tok1 = r.tok1;
  const int nk = r.nk;
  bool ids_bad;
  const int my_id = load_page_ids(p, s, r, wave, lane, &ids_bad);
  const bool bad = r.ctx_bad || ids_bad;

  // Query rows of the group (this lane's VEC columns): with bf16 query and
  // cache the pairs stay packed for v_dot2 (the scale is applied to the
  // reduced score); otherwise they are widened and pre-scaled.
  constexpr bool kDot2 = sizeof(TQ) == 2 && sizeof(TC) == 2;
  constexpr int QVEC = Elem<TQ>::kVec;  // query elements per 16-byte load
  static_assert(VEC % QVEC == 0, "query load");
  float qf[G][VEC];
  uint32_t qw[G][4];
  {
    const TQ* qb = static_cast<const TQ*>(p.q) + ((int64_t)qrow * p.num_heads + (int64_t)kvh * G) * D + col * VEC;
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int c = 0; c < VEC / QVEC; ++c) {
        const uint4 q4 = *reinterpret_cast<const uint4*>(qb + g * D + c * QVEC);
        if (c == 0) {
          qw[g][0] = q4.x;
          qw[g][1] = q4.y;
          qw[g][2] = q4.z;
          qw[g][3] = q4.w;
        }
        Elem<TQ>::unpack(q4, qf[g] + c * QVEC);
      }
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

  const TC* kbase = static_cast<const TC*>(p.k_cache) + (int64_t)kvh * BS * D + row * D + col * VEC;
  const TC* vbase = static_cast<const TC*>(p.v_cache) + (int64_t)kvh * BS * D + row * D + col * VEC;

  auto load_page = [&](int k, uint4 (&kr)[NLD], uint4 (&vr)[NLD]) {
    const int64_t phys = __builtin_amdgcn_readlane(my_id, k);
    const TC* kp = kbase + phys * p.block_stride;
    const TC* vp = vbase + phys * p.block_stride;
#pragma unroll
    for (int i = 0; i < NLD; ++i) kr[i] = load_page16<NONTEMPORAL>(kp + i * TPL * D);
#pragma unroll
    for (int i = 0; i < NLD; ++i) vr[i] = load_page16<NONTEMPORAL>(vp + i * TPL * D);
  };

  auto consume_page = [&](int k, const uint4 (&kr)[NLD], uint4 (&vr)[NLD]) {
    const int t0 = (r.pg0 + wave + k * kWaves) * BS;  // logical token of slot 0
    const bool full = t0 + BS <= tok1;
    float sc[G][NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      if constexpr (kDot2) {
        const uint32_t kw[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float a = 0.f;
#pragma unroll
          for (int w = 0; w < 4; ++w) a = dot2_bf16(qw[g][w], kw[w], a);
          sc[g][i] = a;
        }
      } else {
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
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        sc[g][i] = row_sum<LPT>(sc[g][i]);
        if constexpr (kDot2) sc[g][i] *= p.scale_log2e;
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
  __shared__ float sm_acc[kWaves * G * D];
  __shared__ float sm_m[kWaves * G];
  __shared__ float sm_l[kWaves * G];
  if (row == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < VEC; ++e) sm_acc[(wave * G + g) * D + col * VEC + e] = acc[g][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      sm_m[wave * G + g] = bad ? 0.f : m[g];
      sm_l[wave * G + g] = bad ? __builtin_nanf("") : l[g];
    }
  }
  __syncthreads();
  merge_waves_and_store<TQ, D, G>(p, sm_acc, sm_m, sm_l, s, kvh, part, r.nparts, qrow);
}

template <typename TQ, typename TC, int D, int BS, int G>
hipError_t launch_t(const DecodeLaunch& a, const DecodeParams& p) {
  dim3 grid(a.grid_parts, a.num_kv_heads, a.num_seqs);
  if (a.shared_pages)
    hipLaunchKernelGGL((decode_partition_valu_kernel<TQ, TC, D, BS, G, false>), grid, dim3(kWaves * 64), 0,
                       a.stream, p);
  else
    hipLaunchKernelGGL((decode_partition_valu_kernel<TQ, TC, D, BS, G, true>), grid, dim3(kWaves * 64), 0,
                       a.stream, p);
  return hipGetLastError();
}

template <typename TQ, typename TC, int D, int BS>
hipError_t by_group(const DecodeLaunch& a, const DecodeParams& p) {
  switch (a.num_heads / a.num_kv_heads) {
    case 1: return launch_t<TQ, TC, D, BS, 1>(a, p);
    case 2: return launch_t<TQ, TC, D, BS, 2>(a, p);
    case 4: return launch_t<TQ, TC, D, BS, 4>(a, p);
    case 8: return launch_t<TQ, TC, D, BS, 8>(a, p);
    default: return hipErrorInvalidValue;
  }
}

template <typename TQ, typename TC, int D>
hipError_t by_block(const DecodeLaunch& a, const DecodeParams& p) {
  return a.block_size == 16 ? by_group<TQ, TC, D, 16>(a, p) : by_group<TQ, TC, D, 32>(a, p);
}

template <typename TQ, typename TC>
hipError_t by_dim(const DecodeLaunch& a, const DecodeParams& p) {
  return a.head_dim == 64 ? by_block<TQ, TC, 64>(a, p) : by_block<TQ, TC, 128>(a, p);
}

}  // namespace

hipError_t launch_partition_valu(const DecodeLaunch& a, const DecodeParams& p) {
  if (a.cache_dtype == kDtypeFp8) return by_dim<uint16_t, uint8_t>(a, p);
  return a.dtype == kDtypeF32 ? by_dim<float, float>(a, p) : by_dim<uint16_t, uint16_t>(a, p);
}

}  // namespace pa
