// Decode partition kernel on the matrix cores, for a bf16 query where several
// query heads share a kv head (grouped-query attention, G = H / Hkv > 1); the
// cache holds bf16 or E4M3 fp8 codes (widened to bf16 in registers, exactly).
//
// What is computed is the same as the vector kernel ("vLLM 深度解读",
// luoboask.github.io, section 3 "PagedAttention CUDA Kernel"): per query head,
// softmax over scale * q.k of every context token reached through the block
// table, then the weighted sum of V.  With grouping, one kv page serves G
// query heads, so the two products become dense tiles:
//
//   S^T [tokens x heads] = K_page [tokens x D] . Q_group^T [D x heads]
//   O^T [D x heads]     += V_page^T [D x tokens] . P^T [tokens x heads]
//
// both on v_mfma_f32_16x16x32_bf16 (16x16x16 for 16-token pages), with the
// head dimension of the tile padded to 16 (zero query rows).
//
// Operand layouts (checked on gfx950): A lane i holds row i%16, k = 8*(i/16)+j;
// B lane i holds column i%16, the same k; the f32 result lane i holds rows
// 4*(i/16)+j of column i%16.  Therefore
//  * K goes from HBM straight into the A operand (lane i reads 16 bytes of
//    token i%16), no staging;
//  * the S^T result already sits where the B operand of the PV product wants
//    P^T (tokens along k in the same slots), after a round-to-nearest-even
//    cast to bf16 -- no data movement;
//  * V is the one operand that needs a transpose: each wave writes its page
//    to LDS (rows swizzled so the transposed reads hit distinct banks, rows
//    past the context written as zeros so NaN in unused slots can never reach
//    the product) and reads V^T back as the A operand with gfx950's
//    transposing LDS read, four k slots per instruction.
// The online softmax runs on the S^T tile: each lane holds 4 tokens of one
// head per 16-token tile; the max over tokens takes two cross-lane steps.  The
// reference max is moved lazily (only when exceeded by more than 2^8), which
// keeps the accumulator rescale off the common path; numerator and
// denominator share the same reference, so the ratio is unchanged.

#include "pa_device.h"
#include "pa_mfma.h"

namespace pa {
namespace {

// TC: cache element type, bf16 bits (uint16_t) or E4M3 codes (uint8_t); the
// query is bf16 either way and the products run on bf16 MFMA (E4M3 widens to
// bf16 exactly).
//
// SHARED (shared-prefix decode): the 16 columns of the tile are the query
// heads of up to 16 / G sequences that hold the same leading pages (a beam
// group, or requests with a common prompt), so each shared page is read once
// for all of them.  The grid is one-dimensional, kv head fastest: the first
// num_seqs * prefix_parts rows are prefix partitions of the chunk starting at
// sequence row / prefix_parts, the rest serve each sequence's tokens past its
// shared prefix (tail_parts rows per sequence).  Prefix workgroups read the
// most pages, so they are dispatched first.  Both leave partition results
// that the reduce kernel merges; the softmax algebra is the same as for one
// sequence's partitions, since each column keeps its own running max and sum.
template <typename TC, int D, int BS, int G, bool NONTEMPORAL, bool SHARED>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(SHARED && BS == 16 ? 4 : 3))) void decode_partition_mfma_kernel(DecodeParams p) {
  constexpr bool kFp8 = sizeof(TC) == 1;
  constexpr int NT = BS / 16;       // 16-token tiles per page
  constexpr int NC = D / 32;        // 32-wide steps of the QK contraction
  constexpr int NM = D / 16;        // 16-wide output tiles along head_dim
  constexpr int ROWB = D * 2;       // bytes of one bf16 token row (LDS page)
  constexpr int NCH = ROWB / 16;    // 16-byte bf16 chunks per row
  constexpr int CROWB = D * (int)sizeof(TC);  // bytes of one cache token row
  constexpr int CNCH = CROWB / 16;  // 16-byte cache chunks per row
  constexpr int RPL = 64 / CNCH;    // rows per row-contiguous wave load of V
  constexpr int NV = BS / RPL;      // V loads per lane per page
  constexpr int NKL = kFp8 ? D / 64 : NC;  // K loads per 16-token tile
  constexpr int PAGEB = BS * ROWB;  // bytes of one bf16 page in LDS
  constexpr int NCOL = SHARED ? 16 : G;  // tile columns that carry results
  constexpr int R = 16 / G;               // sequences per prefix chunk
  constexpr int EPI = (kWaves * NCOL * D + 2 * kWaves * NCOL) * 4 + 2 * 16 * 4;
  constexpr int SMEM = kWaves * PAGEB > EPI ? kWaves * PAGEB : EPI;
  static_assert((G >= 2 || SHARED) && G <= 16 && NCH >= 8 && BS % RPL == 0, "tile shape");

  int part = blockIdx.x;
  const int kvh = SHARED ? (int)(blockIdx.x % p.num_kv_heads) : (int)blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  int s;                 // sequence whose table row supplies the page ids
  int qrow = 0;          // its q / out row (decode)
  PartitionRange r;
  int my_id;
  bool bad;              // this wave's pages cannot be read: its columns become NaN
  int col_seq = -1;      // sequence of this lane's column l16 (-1: padding)
  int col_total = 1;     // partitions of that sequence
  bool col_bad = false;  // that sequence's table disagrees with the chunk's (NaN row)
  int slot;              // partition slot of this workgroup's results (< max_parts)
  // Shared prefix: the chunk members whose tokens past the prefix this
  // workgroup reads after the prefix (bit i: member i), with their contexts.
  uint32_t hosted = 0;
  int member_ctx = 0;    // lane i < R: context length of member i
  int chunk0 = 0;        // first sequence of the chunk
  int pre_tokens = 0;    // shared prefix length
  if constexpr (!SHARED) {
    slot = part;
    s = sequence_of(p, blockIdx.z);
    if (s < 0) return;  // uniform over the workgroup
    qrow = query_row(p, s);
    if (qrow < 0) return;
    r = partition_range(p, s, part, wave, BS);
    if (part >= r.nparts) return;  // uniform over the workgroup
    bool ids_bad;
    my_id = load_page_ids(p, s, r, wave, lane, &ids_bad);
    bad = r.ctx_bad || ids_bad;
    col_seq = l16 < G ? s : -1;
  } else {
    const int pt = p.partition_tokens;
    const int row = blockIdx.x / p.num_kv_heads;
    const int nwin = (p.num_seqs + R - 1) / R;
    const int prefix_rows = R * nwin * p.prefix_parts;
    if (row < prefix_rows) {
      // Prefix workgroup of the chunk that starts at sequence z.  Rows come
      // in R classes, z % R = 0 first: groups whose leaders sit at multiples
      // of R (beams of equal width) have all their chunk starts in the first
      // class, and the rows that are no chunk start (one load to see) come
      // after them.
      const int cls = row / (nwin * p.prefix_parts);
      const int rem = row % (nwin * p.prefix_parts);
      const int z = rem / p.prefix_parts * R + cls;
      part = rem % p.prefix_parts;
      if (z >= p.num_seqs) return;
      // The prologue's reads are dependent (leader, then the chunk, then the
      // members and the page ids), and under the walk's load each level costs
      // microseconds.  Rows of the first class (the chunk starts of groups
      // that sit at multiples of R, e.g. beams) therefore issue every read
      // that needs z alone at once: the leader entry, the prefix length at z
      // (the chunk's own when z leads its group), the members' leader entries
      // and contexts, and the page ids of the partition and the members'
      // entries for the same pages as if the prefix filled it.  Each is used
      // only where the checks below would have read it.  Other rows read one
      // level at a time.
      const bool spec = cls == 0;
      const int m = z + l16;
      const bool m_in = l16 < R && m < p.num_seqs;
      const int spec_lanes = (pt / BS + kWaves - 1) / kWaves;  // pages per wave of a full partition
      const int64_t jspec = (int64_t)part * (pt / BS) + wave + lane * kWaves;
      const bool j_in = lane < spec_lanes && jspec < p.max_blocks_per_seq;
      const int lead = p.prefix_leader[z];
      int z_blocks = 0, m_lead = -1, m_ctx = 0, spec_id = 0;
      int other[R > 1 ? R - 1 : 1] = {};
      if (spec) {
        z_blocks = p.prefix_blocks[z];
        if (m_in) {
          m_lead = p.prefix_leader[m];
          m_ctx = p.context_lens[m];
        }
        if (j_in) {
          spec_id = p.block_tables[(int64_t)z * p.max_blocks_per_seq + jspec];
#pragma unroll
          for (int i = 1; i < R; ++i)
            if (z + i < p.num_seqs) other[i - 1] = p.block_tables[(int64_t)(z + i) * p.max_blocks_per_seq + jspec];
        }
      }
      if (lead < 0 || lead > z || (z - lead) % R != 0) return;
      // A leader's own chunk: prefix_chunk's reads are the leader entry and
      // the prefix length at z, both in hand.
      const PrefixChunk pc =
          spec && lead == z ? PrefixChunk{z, z, z_blocks > 0 ? z_blocks : 0} : prefix_chunk(p, z);
      if (pc.blocks == 0 || pc.chunk != z) return;
      // A prefix past the caller's bound: every member is a bad row, which
      // its own workgroup writes.
      if (pc.blocks > p.max_prefix_blocks) return;
      const int pre = pc.blocks * BS;
      const int npre = (pre + pt - 1) / pt;
      if (part >= npre) return;
      s = z;
      slot = part;
      r = token_range(pre, npre, part * pt, min(pre, part * pt + pt), false, wave, BS);
      // Lane i < R checks member z + i: same group, and a context that holds
      // the prefix (the same test its own workgroups make).
      bool member = false;
      bool host = false;
      int total = 0;
      if (!spec && m_in) {
        m_lead = p.prefix_leader[m];
        m_ctx = p.context_lens[m];
      }
      if (m_in && m_lead == pc.leader) {
        const SeqSplit sp = split_context(p, m_ctx, pc.blocks, l16);
        member = !sp.bad;
        host = member && sp.folded && l16 % npre == part;
        total = sp.nprefix + sp.ntail;
        member_ctx = sp.ctx;
      }
      const uint32_t members = static_cast<uint32_t>(__ballot(member)) & 0xffffu;
      hosted = static_cast<uint32_t>(__ballot(host)) & 0xffffu;
      chunk0 = z;
      pre_tokens = pre;
      const int mi = l16 / G;
      col_seq = (members >> mi) & 1u ? z + mi : -1;
      col_total = __shfl(total, mi);
      bool ids_bad;
      if (spec) {
        // The partition's pages are the first r.nk <= spec_lanes of each wave's.
        bool badid = false;
        my_id = 0;
        if (lane < r.nk) {
          badid = spec_id < 0 || spec_id >= p.num_blocks;
          my_id = badid ? 0 : spec_id;
        }
        ids_bad = __any(badid);
      } else {
        my_id = load_page_ids(p, z, r, wave, lane, &ids_bad);
      }
      bad = ids_bad;
      // Every member must name the same physical pages.
      uint32_t differ = 0;
      if (lane < r.nk) {
        const int64_t j = r.pg0 + wave + lane * kWaves;
#pragma unroll
        for (int i = 1; i < R; ++i) {
          if (!((members >> i) & 1u)) continue;
          const int e = spec ? other[i - 1] : p.block_tables[(int64_t)(z + i) * p.max_blocks_per_seq + j];
          if (e != my_id) differ |= 1u << i;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) differ |= __shfl_xor(differ, off);
      col_bad = ((differ >> mi) & 1u) != 0;
    } else {
      // Sequence s's own workgroups: its tokens past the shared prefix.
      s = (row - prefix_rows) / p.tail_parts;
      part = (row - prefix_rows) % p.tail_parts;
      const PrefixChunk pc = prefix_chunk(p, s);
      const SeqSplit sp = split_context(p, p.context_lens[s], pc.blocks, pc.blocks > 0 ? s - pc.chunk : -1);
      if (part >= sp.ntail) return;  // none, or folded into a prefix workgroup
      const int t0 = sp.prefix + part * pt;
      r = token_range(sp.ctx, sp.nprefix + sp.ntail, t0, min(sp.ctx, t0 + pt), sp.bad, wave, BS);
      bool ids_bad;
      my_id = load_page_ids(p, s, r, wave, lane, &ids_bad);
      bad = sp.bad || ids_bad;
      col_seq = l16 < G ? s : -1;
      col_total = sp.nprefix + sp.ntail;
      slot = sp.nprefix + part;
    }
  }
  int tok1 = r.tok1;
  int nk = r.nk;
  bool col_on = true;  // this lane's column takes part in the current page range

  // B operand of S^T = K Q^T: for bf16 caches lane holds Q[head l16][32c +
  // 8 g4 .. +7]; for fp8 caches, whose 16-byte K loads carry 16 columns, step
  // c = 2kk + h holds columns 64kk + 16 g4 + 8h .. +7 (the K operand uses the
  // same column order, so the contraction is unchanged).  Zero for padding
  // columns.
  bf16x8_t qb[NC];
  {
    const int q_seq = SHARED ? (col_seq >= 0 ? col_seq : s) : qrow;
    const int q_head = kvh * G + (SHARED ? l16 % G : (l16 < G ? l16 : 0));
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) + ((int64_t)q_seq * p.num_heads + q_head) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int col0 = kFp8 ? 64 * (c >> 1) + 16 * g4 + 8 * (c & 1) : 32 * c + 8 * g4;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (col_seq >= 0) v = *reinterpret_cast<const uint4*>(qp + col0);
      qb[c] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  f32x4_t acc[NM];  // O^T[d = 16 m + 4 g4 + j][head l16]
#pragma unroll
  for (int m = 0; m < NM; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -FLT_MAX;  // running max of head l16 (same in the 4 lanes of a head)
  float l_run = 0.f;       // this lane's share of the running sum

  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  unsigned char* vbuf = smem + wave * PAGEB;

  const TC* kc = static_cast<const TC*>(p.k_cache) + (int64_t)kvh * BS * D;
  const TC* vc = static_cast<const TC*>(p.v_cache) + (int64_t)kvh * BS * D;
  // A operand of S^T: token l16; bf16: 8 columns at 32c + 8 g4; fp8: 16 columns
  // at 64kk + 16 g4.
  const int k_off = l16 * D + (kFp8 ? 16 : 8) * g4;
  const int v_row = lane / CNCH;               // row-contiguous V load
  const int v_ch = lane % CNCH;
  const int v_off = v_row * D + v_ch * (16 / (int)sizeof(TC));

  auto load_k = [&](int k, uint4 (&kr)[NT][NKL]) {
    const int64_t phys = __builtin_amdgcn_readlane(my_id, k);
    const TC* kp = kc + phys * p.block_stride + k_off;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int c = 0; c < NKL; ++c)
        kr[tt][c] = load_page16<NONTEMPORAL>(kp + tt * 16 * D + (kFp8 ? 64 : 32) * c);
  };
  auto load_v = [&](int k, uint4 (&vr)[NV]) {
    const int64_t phys = __builtin_amdgcn_readlane(my_id, k);
    const TC* vp = vc + phys * p.block_stride + v_off;
#pragma unroll
    for (int n = 0; n < NV; ++n) vr[n] = load_page16<NONTEMPORAL>(vp + n * RPL * D);
  };
  auto stage_v = [&](int k, const uint4 (&vr)[NV]) {
    const int t0 = (r.pg0 + wave + k * kWaves) * BS;
    const bool full = t0 + BS <= tok1;
    wave_lds_fence();
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      const int row = n * RPL + v_row;
      const bool keep = full || t0 + row < tok1;
      if constexpr (kFp8) {
        // 16 codes -> 16 bf16: LDS chunks 2 v_ch and 2 v_ch + 1 of the row.
        uint4 a = fp8x8_to_bf16x8(vr[n].x, vr[n].y);
        uint4 b = fp8x8_to_bf16x8(vr[n].z, vr[n].w);
        if (!keep) a = b = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(vbuf + row * ROWB + (((2 * v_ch) ^ swz<ROWB>(row)) << 4)) = a;
        *reinterpret_cast<uint4*>(vbuf + row * ROWB + (((2 * v_ch + 1) ^ swz<ROWB>(row)) << 4)) = b;
      } else {
        uint4 v = vr[n];
        if (!keep) v = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(vbuf + row * ROWB + ((v_ch ^ swz<ROWB>(row)) << 4)) = v;
      }
    }
    wave_lds_fence();
  };
  // V^T operand: four k slots per transposed LDS read (vt4 in pa_mfma.h).
  auto vt4 = [&](int tb, int d0) -> s16x4_t { return pa::vt4<ROWB>(vbuf, l16, tb, d0); };

  auto scores = [&](const uint4 (&kr)[NT][NKL], f32x4_t (&st)[NT]) {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      st[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        uint4 ka;
        if constexpr (kFp8) {
          const uint4& w = kr[tt][c >> 1];
          ka = (c & 1) ? fp8x8_to_bf16x8(w.z, w.w) : fp8x8_to_bf16x8(w.x, w.y);
        } else {
          ka = kr[tt][c];
        }
        st[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka), qb[c], st[tt], 0,
                                                         0, 0);
      }
    }
  };

  auto softmax_pv = [&](int k, const f32x4_t (&st)[NT]) {
    const int t0 = (r.pg0 + wave + k * kWaves) * BS;
    const bool full = t0 + BS <= tok1;
    // Scores of token 16 tt + 4 g4 + j for head l16; masked past the context.
    float sv[NT][4];
    float mx = m_run;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool valid = col_on && (full || (t0 + 16 * tt + 4 * g4 + j < tok1));
        sv[tt][j] = valid ? st[tt][j] * p.scale_log2e : -__builtin_inff();
        mx = fmaxf(mx, sv[tt][j]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // Lazy rescaling: the reference max moves only when a score exceeds it
    // by more than 2^kRescaleLog2, so weights stay <= 2^kRescaleLog2 and the
    // accumulators are rescaled on few pages (a wave-uniform branch).
    if (__any(mx > m_run + kRescaleLog2)) {
      const float alpha = fast_exp2(m_run - mx);
      m_run = mx;
      l_run *= alpha;
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[m] *= alpha;
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int j = 0; j < 4; ++j) sv[tt][j] = fast_exp2(sv[tt][j] - m_run);
    // The weights are rounded to bf16 for the PV product; the running sum
    // adds the same rounded weights, so numerator and denominator agree (a
    // constant V row comes back exactly).

    if constexpr (BS == 32) {
      // P^T as the B operand: k slot j of lane group g4 is token 4 g4 + j
      // (j < 4, first tile) or 16 + 4 g4 + j - 4 (second tile).
      uint4 pbits;
      pbits.x = pack_bf16x2(sv[0][0], sv[0][1]);
      pbits.y = pack_bf16x2(sv[0][2], sv[0][3]);
      pbits.z = pack_bf16x2(sv[1][0], sv[1][1]);
      pbits.w = pack_bf16x2(sv[1][2], sv[1][3]);
      l_run = bf16x2_acc(pbits.w, bf16x2_acc(pbits.z, bf16x2_acc(pbits.y, bf16x2_acc(pbits.x, l_run))));
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pbits);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const s16x4_t lo = vt4(4 * g4, 16 * m);       // tokens 4 g4 .. +3
        const s16x4_t hi = vt4(16 + 4 * g4, 16 * m);  // tokens 16 + 4 g4 .. +3
        const s16x8_t va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, va), pb, acc[m], 0, 0,
                                                         0);
      }
    } else {
      // 16-token pages: k slot j of lane group g4 is token 4 g4 + j.
      uint2 pbits;
      pbits.x = pack_bf16x2(sv[0][0], sv[0][1]);
      pbits.y = pack_bf16x2(sv[0][2], sv[0][3]);
      l_run = bf16x2_acc(pbits.y, bf16x2_acc(pbits.x, l_run));
      const s16x4_t pb = __builtin_bit_cast(s16x4_t, pbits);
#pragma unroll
      for (int m = 0; m < NM; ++m)
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt4(4 * g4, 16 * m), pb, acc[m], 0, 0, 0);
    }
  };

  // One K and one V register buffer: the next page's V is requested as soon
  // as this page's V sits in LDS, the next K as soon as the QK products have
  // consumed this page's K, so one page per wave is always in flight.  (Two
  // buffer pairs, two pages in flight, measured no faster on any workload
  // here and cost a wave per SIMD of occupancy.)
  // Page ranges: this workgroup's own, then (shared prefix) the tokens past
  // the prefix of each member it hosts, from that member's table row, for
  // that member's columns only (their running max and sum carry on).
  bool walk = !bad;
  for (;;) {
    if (walk && nk > 0) {
      uint4 kr[NT][NKL], vr[NV];
      load_k(0, kr);
      load_v(0, vr);
      for (int k = 0; k < nk; ++k) {
        stage_v(k, vr);
        if (k + 1 < nk) load_v(k + 1, vr);
        f32x4_t st[NT];
        scores(kr, st);
        if (k + 1 < nk) load_k(k + 1, kr);
        softmax_pv(k, st);
      }
    }
    if (!SHARED || hosted == 0 || bad) break;
    const int i = __builtin_ctz(hosted);
    hosted &= hosted - 1;
    const int ctx_i = __shfl(member_ctx, i);
    r = token_range(ctx_i, 1, pre_tokens, ctx_i, false, wave, BS);
    tok1 = r.tok1;
    nk = r.nk;
    bool ids_bad;
    my_id = load_page_ids(p, chunk0 + i, r, wave, lane, &ids_bad);
    col_on = l16 / G == i;
    col_bad = col_bad || (ids_bad && col_on);  // the member's row becomes NaN
    walk = !ids_bad;
  }

  // The four lanes of a head each hold a share of its running sum.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  __syncthreads();  // every wave is done with its page buffer: reuse the LDS
  float* sm_acc = reinterpret_cast<float*>(smem);
  float* sm_m = sm_acc + kWaves * NCOL * D;
  float* sm_l = sm_m + kWaves * NCOL;
  if (l16 < NCOL) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) sm_acc[(wave * NCOL + l16) * D + 16 * m + 4 * g4 + j] = acc[m][j];
    if (g4 == 0) {
      sm_m[wave * NCOL + l16] = bad ? 0.f : m_run;
      sm_l[wave * NCOL + l16] = bad || col_bad ? __builtin_nanf("") : l_run;
    }
  }
  if constexpr (!SHARED) {
    __syncthreads();
    merge_waves_and_store<uint16_t, D, G>(p, sm_acc, sm_m, sm_l, s, kvh, part, r.nparts, qrow);
  } else {
    int* sm_seq = reinterpret_cast<int*>(sm_l + kWaves * NCOL);
    int* sm_total = sm_seq + 16;
    if (wave == 0 && g4 == 0) {
      sm_seq[l16] = col_seq;
      sm_total[l16] = col_total;
    }
    __syncthreads();
    // Merge the waves per column; a sequence with one partition in all gets
    // its final row, otherwise the partition slot.
    for (int idx = tid; idx < NCOL * D; idx += kWaves * 64) {
      const int c = idx / D;
      const int d = idx % D;
      const int seq = sm_seq[c];
      if (seq < 0) continue;
      float mm = -FLT_MAX;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, sm_m[w * NCOL + c]);
      float ll = 0.f, aa = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float wt = fast_exp2(sm_m[w * NCOL + c] - mm);
        ll += sm_l[w * NCOL + c] * wt;
        aa += sm_acc[(w * NCOL + c) * D + d] * wt;
      }
      const int64_t sh = (int64_t)seq * p.num_heads + (int64_t)kvh * G + c % G;
      if (sm_total[c] == 1) {
        const float o = (ll == 0.f) ? 0.f : aa * p.v_scale / ll;
        Elem<uint16_t>::store(static_cast<uint16_t*>(p.out) + sh * D + d, o);
      } else {
        const int64_t at = sh * p.max_parts + slot;
        p.ws_acc[at * D + d] = aa;
        if (d == 0) {
          p.ws_ml[at * 2] = mm;
          p.ws_ml[at * 2 + 1] = ll;
        }
      }
    }
  }
}

template <typename TC, int D, int BS, int G, bool SHARED>
hipError_t launch_t(const DecodeLaunch& a, const DecodeParams& p) {
  const int R = 16 / G;
  const dim3 grid = SHARED ? dim3(((a.num_seqs + R - 1) / R * R * a.prefix_parts + a.num_seqs * a.tail_parts) *
                                      a.num_kv_heads,
                                  1, 1)
                          : dim3(a.grid_parts, a.num_kv_heads, a.num_seqs);
  if constexpr (SHARED) {
    hipLaunchKernelGGL((decode_partition_mfma_kernel<TC, D, BS, G, true, true>), grid, dim3(kWaves * 64), 0,
                       a.stream, p);
  } else if (a.shared_pages) {
    hipLaunchKernelGGL((decode_partition_mfma_kernel<TC, D, BS, G, false, false>), grid, dim3(kWaves * 64), 0,
                       a.stream, p);
  } else {
    hipLaunchKernelGGL((decode_partition_mfma_kernel<TC, D, BS, G, true, false>), grid, dim3(kWaves * 64), 0,
                       a.stream, p);
  }
  return hipGetLastError();
}

template <typename TC, int D, int BS>
hipError_t by_group(const DecodeLaunch& a, const DecodeParams& p) {
  if (a.prefix_leader != nullptr) {
    switch (a.num_heads / a.num_kv_heads) {
      case 1: return launch_t<TC, D, BS, 1, true>(a, p);
      case 2: return launch_t<TC, D, BS, 2, true>(a, p);
      case 4: return launch_t<TC, D, BS, 4, true>(a, p);
      case 8: return launch_t<TC, D, BS, 8, true>(a, p);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.num_heads / a.num_kv_heads) {
    case 2: return launch_t<TC, D, BS, 2, false>(a, p);
    case 4: return launch_t<TC, D, BS, 4, false>(a, p);
    case 8: return launch_t<TC, D, BS, 8, false>(a, p);
    default: return hipErrorInvalidValue;
  }
}

template <typename TC, int D>
hipError_t by_block(const DecodeLaunch& a, const DecodeParams& p) {
  return a.block_size == 16 ? by_group<TC, D, 16>(a, p) : by_group<TC, D, 32>(a, p);
}

template <typename TC>
hipError_t by_dim(const DecodeLaunch& a, const DecodeParams& p) {
  return a.head_dim == 64 ? by_block<TC, 64>(a, p) : by_block<TC, 128>(a, p);
}

}  // namespace

hipError_t launch_partition_mfma(const DecodeLaunch& a, const DecodeParams& p) {
  return a.cache_dtype == kDtypeFp8 ? by_dim<uint8_t>(a, p) : by_dim<uint16_t>(a, p);
}

}  // namespace pa
