// Multi-query paged attention on the matrix cores: several new query tokens per
// sequence -- a chunk of a long prompt, or drafted tokens being verified --
// each attending causally to the sequence's cached context ("详解vLLM推理引擎
// 架构" (tbr8.org), sections "Chunked Prefill（分块预填充）" and "结合 Speculative
// Decoding 加速").  The new tokens' K/V are already in the cache; query i of a
// sequence with q_len new tokens and L cached tokens sits at position
// L - q_len + i and sees tokens 0 .. L - q_len + i.
//
// Rows.  For one kv head, a sequence contributes q_len * G rows (row r is query
// r / G with query head kvh * G + r % G).  A workgroup takes a block of 64 rows
// and each of its 4 waves owns 16 of them as the 16 columns of
//   S^T [tokens x rows] = K [tokens x D] . Q^T [D x rows],
//   O^T [D x rows]     += V^T [D x tokens] . P^T [tokens x rows]
// (the decode kernel's formulation), so one K/V step staged in LDS feeds 64
// rows.  A step is 32 tokens: two 16-token pages or one 32-token page.  Pages
// go from the cache straight into a ring of two or three LDS stages (buffer
// loads with the lds bit, one or two steps ahead).  bf16 chunks land where the
// matrix cores read them: K row-major with 16-byte chunks swizzled by the
// token, so the 16 rows one A-operand read touches hit distinct banks, and V
// in the transposed-read layout of pa_mfma.h.  E4M3 V codes land as stored
// and each step is widened (exactly) into a bf16 tile in that layout; E4M3 K
// codes at D = 128 land swizzled and the QK product widens them in registers
// (at D = 64 they are widened into a tile like V).  Each
// column keeps its own running max and sum, moved lazily (only when a score
// exceeds the reference by more than 2^8).
//
// Sequences with exactly one new query are decode steps; unless told
// otherwise, the entry point runs them through the decode kernels (which
// stream their pages at the HBM rate) and this kernel skips them.
//
// Partitions.  A sequence whose rows fit one block (speculative verification,
// short chunks) would give too few workgroups on a long context, so its
// context is cut into partitions of partition_tokens tokens whose
// (max, sum, accumulator) triples the reduce kernel merges; a sequence with
// more rows is parallel enough through its row blocks and is not cut.  Given
// partition_tokens, the cut depends on the sequence alone; the default
// partition_tokens follows the batch's shape (its host-side bounds), so a
// caller that needs rows bitwise independent of the batch fixes it.

#include <type_traits>

#include "pa_device.h"
#include "pa_lds_dma.h"
#include "pa_mfma.h"

namespace pa {
namespace {

constexpr int kMqWaves = 4;                   // waves per workgroup, 16 rows each
constexpr int kRowsPerBlock = kMqWaves * 16;
constexpr int kStepTokens = 32;               // tokens staged in LDS per step

struct MultiQueryParams {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;
  float* ws_ml;
  float* ws_acc;
  int64_t block_stride;  // elements between consecutive physical blocks
  int max_blocks_per_seq;
  int num_seqs;
  int num_query_tokens;
  int num_heads;
  int num_kv_heads;
  int num_blocks;
  int max_context_len;
  int max_query_len;
  int partition_tokens;
  int max_parts;       // partition slots per row (workspace)
  int max_row_blocks;  // row blocks of the longest allowed chunk
  int2* work;          // work items (sequence, row block index << 16 | partition)
  int* work_count;     // number of work items
  int work_capacity;   // items the list holds (the grid's bound)
  int find_items;      // the workgroups find their own items (at most 64 sequences;
                       // no list, no schedule launch)
  int decode_rows_elsewhere;  // sequences with one query run in the decode kernels
  int stream_rows;     // single-block sequences of at most this many rows run in the
                       // streaming kernel (0: none), the others in the ring kernel
  int one_ring;        // the two-tile ring kernel takes the 64-row blocks too (the
                       // one-tile kernel is not launched)
  int whole_contexts;  // no sequence is cut into partitions (no merge launch)
  float scale_log2e;   // softmax scale * log2(e), times k_scale for fp8 caches
  float v_scale;       // multiplies the output (1 unless the cache holds fp8 codes)
};

// The work of row block `rbi` (in dispatch order) of sequence s.
struct MqBlock {
  int t0;       // first q / out row of the sequence
  int qlen;     // new query tokens
  int ctx;      // cached tokens, the new ones included
  int rows;     // qlen * G
  int rpb;      // rows per block: 64, or 128 for a sequence of more than 128 rows
  int rb;       // row block: rows rb * rpb .. rb * rpb + rpb - 1
  int kv_end;   // tokens seen by the block's last query
  int nparts;   // context partitions
  int nrb;      // row blocks of the sequence
  bool skip;    // no such block, or an invalid query range: nothing is written
  bool bad;     // bad context length: the block's rows are written as NaN
};

// A work item's second word holds a row-block index in its upper 16 bits and
// a partition index in the lower 16 (the host keeps both below 2^15).  The
// word is packed and unpacked as unsigned, so no index reads back negative.
__device__ __forceinline__ int pack_row_block(int rbi) { return (int)((uint32_t)rbi << 16); }
__device__ __forceinline__ int row_block_of(int word) { return (int)((uint32_t)word >> 16); }

template <int G>
__device__ __forceinline__ MqBlock mq_block(const MultiQueryParams& p, int s, int rbi) {
  MqBlock b{};
  const int t0 = p.query_start[s];
  const int t1 = p.query_start[s + 1];
  b.skip = t0 < 0 || t1 < t0 || t1 > p.num_query_tokens || t1 - t0 > p.max_query_len;
  if (b.skip) return b;
  b.t0 = t0;
  b.qlen = t1 - t0;
  if (b.qlen == 1 && p.decode_rows_elsewhere) {  // a decode row: served by the decode kernels
    b.skip = true;
    return b;
  }
  b.rows = b.qlen * G;
  // Long chunks take 128-row blocks (two 16-row tiles per wave: each K and
  // V operand read from LDS feeds two products); sequences of at most 128
  // rows keep 64-row blocks, so every sequence of one block has at most 64
  // rows and only those are cut into partitions.
  b.rpb = b.rows > 2 * kRowsPerBlock ? 2 * kRowsPerBlock : kRowsPerBlock;
  const int nrb = (b.rows + b.rpb - 1) / b.rpb;
  b.nrb = nrb;
  if (rbi >= nrb) {
    b.skip = true;
    return b;
  }
  b.rb = nrb - 1 - rbi;  // later queries see more tokens: dispatch them first
  b.ctx = p.context_lens[s];
  b.bad = b.ctx < 0 || b.ctx > p.max_context_len || b.qlen > b.ctx;
  b.nparts = 1;
  if (b.bad) return b;
  const int last_row = min(b.rows, (b.rb + 1) * b.rpb) - 1;
  b.kv_end = b.ctx - b.qlen + last_row / G + 1;
  if (nrb == 1 && b.kv_end > p.partition_tokens && !p.whole_contexts)
    b.nparts = (b.kv_end + p.partition_tokens - 1) / p.partition_tokens;
  return b;
}

// Work item `item` of the list multi_query_schedule_kernel writes (the same
// items; the second class longest first), found by the workgroup itself when
// the batch has at most 64 sequences: wave 0 counts the items of sequence
// `lane`, scans the counts, and the lane whose range holds `item` publishes it
// through LDS.  Every thread of the workgroup calls it; false: no such item.
// Measured against both classes in sequence order on the 70B-shaped
// verification batch: E4M3 32 sequences 78.9 -> 69.9 us, 64 sequences 151.5
// -> 142.7, 16 sequences 45.6 -> 44.3, 4 queries 73.5 -> 68.4; bf16 32
// sequences 101.5 -> 99.1, 64 sequences 230.9 -> 197.4.  (Ranking the lengths
// with a 64-step loop over the lanes instead cost 2-5 us per call.)
template <int G>
__device__ __forceinline__ bool find_item(const MultiQueryParams& p, int item, int2* w) {
  __shared__ int2 found;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int n = 0;
    bool single = false;
    int rest = 0;  // tokens of the last partition of a cut sequence
    if (lane < p.num_seqs) {
      const MqBlock b = mq_block<G>(p, lane, 0);
      if (!b.skip) {
        single = b.nrb == 1;
        n = single ? b.nparts : b.nrb;
        if (single && n > 1) rest = b.kv_end - (n - 1) * p.partition_tokens;
      }
    }
    // The list's two classes: n0 items of sequence `lane` in the first, and
    // its last partition, when it is cut, in the second.
    const bool last = single && n > 1;
    const int n0 = n - (last ? 1 : 0);
    int incl0 = n0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v0 = __shfl_up(incl0, off);
      if (lane >= off) incl0 += v0;
    }
    const int start0 = incl0 - n0;
    const int total0 = __shfl(incl0, 63);
    if (lane == 0) found = make_int2(-1, 0);
    if (n0 > 0 && item >= start0 && item < start0 + n0)
      found = make_int2(lane, single ? item - start0 : pack_row_block(item - start0));
    // Second class, longest first (equal lengths: lower sequence first): the
    // item's rank r is selected bit by bit from the top with wave-uniform
    // ballots, keeping the lanes whose length agrees with the selected bits.
    uint64_t m = __ballot(last);
    int r = item - total0;
    if (r >= 0 && r < __popcll(m)) {
      for (int bit = 31 - __clz(p.partition_tokens); bit >= 0; --bit) {
        const uint64_t ones = __ballot((rest >> bit) & 1) & m;
        const int c = __popcll(ones);
        if (r < c) {
          m = ones;
        } else {
          r -= c;
          m &= ~ones;
        }
      }
      // m: the lanes of the selected length; the item is the r-th of them.
      if (((m >> lane) & 1) && __popcll(m & ((1ull << lane) - 1)) == r) found = make_int2(lane, n - 1);
    }
  }
  __syncthreads();
  *w = found;
  return w->x >= 0;
}

// K rows (ROWB bytes) in LDS: 16-byte chunk c of token `tok` is stored at
// chunk c ^ kswz<ROWB>(tok).  One A-operand read has 16 lanes read 16
// consecutive tokens at the same logical chunk; the swizzle gives them
// distinct banks whether 8 or 16 lanes (32 or 64 4-byte banks) are served
// per cycle: 256-byte rows take 16 chunk positions, 128-byte rows (alternating
// bank halves) 8 positions distinct over each 8 tokens and each parity.
// E4M3 K codes at D = 128 (128-byte rows, 8 chunks) in the ring stage: chunk
// c of token `tok` is stored at chunk c ^ kswz8(tok).  An operand read has 16
// lanes read 8 bytes of 16 consecutive tokens at the same logical chunk; row
// parity picks the bank half and the swizzle one of 8 positions, so the 32
// lanes served together hit all 64 banks once.
__device__ __forceinline__ int kswz8(int tok) { return (tok >> 1) & 7; }

template <int ROWB>
__device__ __forceinline__ int kswz(int tok) {
  static_assert(ROWB == 128 || ROWB == 256, "128- or 256-byte rows");
  return ROWB == 256 ? (tok & 15) : ((tok & 7) ^ ((tok >> 3) & 1));
}

// Max over the four lanes l, l ^ 16, l ^ 32, l ^ 48 that hold one column of an
// MFMA result: v_permlane32_swap exchanges the wave's 32-lane halves and
// v_permlane16_swap the odd and even 16-lane rows (gfx950), both in the VALU.
// The maxima take v_max_f32 directly: for fmaxf the compiler first quiets
// each input it cannot prove canonical (a lane swap's result, a running max),
// one instruction per input; scores are never signalling NaNs, so the plain
// instruction gives the same values.
__device__ __forceinline__ float max_of(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ float column_max(float x) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max_of(__uint_as_float(h[0]), __uint_as_float(h[1]));
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_of(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// The column maxima of two MFMA results at once: the first half swap leaves
// a's four-lane groups merged in lanes 0-31 and b's in lanes 32-63, so one
// row swap finishes both, and a last half swap hands each its maxima in all
// lanes (three swaps and two maxima for the two, against two swaps and two
// maxima for each alone).
__device__ __forceinline__ void column_max2(float& a, float& b) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  float x = max_of(__uint_as_float(h[0]), __uint_as_float(h[1]));
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max_of(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto g = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(g[0]);
  b = __uint_as_float(g[1]);
}

// Bytes of the ring kernel's LDS: STAGES (K, V) stages of one step as stored
// in the cache, plus for E4M3 the widened bf16 tile(s) (V only at D = 128,
// where the QK product widens K in registers).
template <typename TC, int D, int STAGES, int STEP = kStepTokens>
constexpr int ring_lds_bytes() {
  constexpr int raw_tile = STEP * D * (int)sizeof(TC);
  constexpr int bf16_tile = STEP * D * 2;
  return STAGES * 2 * raw_tile + (sizeof(TC) == 1 ? (D == 128 ? 1 : 2) * bf16_tile : 0);
}

// V tiles of the ring: each 1 KiB holds R = 1024 / ROWB consecutive
// tokens chunk-major, 16-byte chunk c of the block's token r at slot c R + r.
// The 4 consecutive tokens that a 16-lane transposed read takes at one column
// then sit in 64 contiguous bytes (distinct banks), and the read's column
// offset is an immediate (16 R bytes per chunk), where the row-major layout
// needs a swizzle that depends on both the token and the column.
template <int ROWB>
__device__ __forceinline__ int vslot_cm(int tok, int ch) {
  constexpr int R = 1024 / ROWB;
  return (tok / R) * 1024 + (ch * R + tok % R) * 16;
}

// Four k slots of the V^T A operand from a chunk-major V stage: lane l16
// receives column d0 + l16 of tokens tb .. tb + 3 (tb a multiple of 4, d0 of
// 16), as vt4 does for the row-major layout.
template <int ROWB>
__device__ __forceinline__ s16x4_t vt4_cm(const unsigned char* tile, int l16, int tb, int d0) {
  constexpr int R = 1024 / ROWB;
  const int t = tb + (l16 >> 2);
  const int lane_off = (t / R) * 1024 + (((l16 & 3) >> 1) * R + t % R) * 16 + ((l16 & 1) << 3);
  const unsigned char* a = tile + lane_off + (d0 >> 3) * R * 16;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)a);
}

// NCT: 16-row tiles per wave (1: 64-row blocks, 2: 128-row blocks, and the
// 64-row ones too when it is the batch's only ring launch); the kernel serves
// only the sequences whose blocks it takes.  STEP: tokens staged per step (32
// or 64).
// Register targets: four waves per SIMD for one tile (the 64-token E4M3
// kernel needs more than 128 registers and settles at three), three for two
// tiles.  The two-tile E4M3 kernel, asked for two, took 180 registers; at
// three it fits in 168 (chunk-only prefill batch over E4M3: 230 -> 199 us).
template <typename TC, int D, int BS, int G, int STAGES, int NCT, int STEP = kStepTokens>
__global__ __launch_bounds__(kMqWaves * 64) __attribute__((amdgpu_waves_per_eu(NCT == 1 ? 4 : 3))) void multi_query_kernel(MultiQueryParams p) {
  constexpr bool kFp8 = sizeof(TC) == 1;
  constexpr int PPS = STEP / BS;             // pages per step
  constexpr int NC = D / 32;                 // 32-wide steps of the QK contraction
  constexpr int NM = D / 16;                 // 16-wide output tiles along D
  constexpr int ROWB = D * 2;                // bytes of one bf16 row in LDS
  constexpr int NCH = ROWB / 16;             // 16-byte bf16 chunks per row
  constexpr int CCH = D * (int)sizeof(TC) / 16;  // 16-byte cache chunks per row
  constexpr int CHUNKS = STEP * CCH;         // 16-byte cache chunks per step (K or V)
  constexpr int PER_T = (CHUNKS + kMqWaves * 64 - 1) / (kMqWaves * 64);
  constexpr int NTT = STEP / 16;             // 16-token tiles per step
  constexpr int TILEB = STEP * ROWB;         // bytes of one step's bf16 K (or V) in LDS
  constexpr int CROWB = D * (int)sizeof(TC);  // bytes of one cache row
  constexpr int RTILEB = STEP * CROWB;       // bytes of one step's K (or V) as in the cache
  // A ring of STAGES (K, V) stages filled by direct LDS loads STAGES - 1
  // steps ahead.  bf16 caches land in the swizzled layouts the matrix cores
  // read; E4M3 caches land as they are and each step is widened into one
  // bf16 (K, V) tile after the ring.
  constexpr int NSTAGE = STAGES;
  // E4M3 at D = 128: the QK product reads K codes straight from the stage
  // (8 codes per lane, widened in registers), so only V is widened in LDS.
  constexpr bool kKRaw = kFp8 && D == 128;
  constexpr int LDS_BYTES = ring_lds_bytes<TC, D, NSTAGE, STEP>();
  static_assert(LDS_BYTES == NSTAGE * 2 * RTILEB + (kFp8 ? (kKRaw ? 1 : 2) * TILEB : 0), "ring layout");
  constexpr int RPB = kRowsPerBlock * NCT;   // rows per block
  static_assert(STEP % BS == 0 && STEP % 32 == 0 && NCH >= 8, "tile shape");
  static_assert(kFp8 || CHUNKS % (kMqWaves * 64) == 0, "a bf16 step is whole wave loads");
  static_assert(CHUNKS * 16 == RTILEB, "a step is CHUNKS 16-byte chunks");
  static_assert(CHUNKS % 64 == 0 && 64 / CCH <= BS, "a wave's chunks of a step lie in one page");
  static_assert(NSTAGE >= 2, "ring depth");

  const int kvh = blockIdx.x % p.num_kv_heads;
  const int item = blockIdx.x / p.num_kv_heads;
  int2 w;
  if (p.find_items) {
    if (!find_item<G>(p, item, &w)) return;  // uniform over the workgroup
  } else {
    if (item >= *p.work_count) return;  // uniform over the workgroup
    w = p.work[item];
  }
  const int s = w.x;
  const int rbi = row_block_of(w.y);
  const int part = w.y & 0xffff;
  const MqBlock b = mq_block<G>(p, s, rbi);
  if (b.skip || part >= b.nparts) return;
  // The two-tile kernel takes 128-row blocks, and the 64-row ones when it is
  // the only ring launch (its waves 0 and 1 then hold the rows); the one-tile
  // kernel takes 64-row blocks.
  if (b.rpb != RPB && !(NCT == 2 && p.one_ring && b.rpb == kRowsPerBlock)) return;
  if (b.nrb == 1 && b.rows <= p.stream_rows) return;  // the streaming kernel's

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < kMqWaves);
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  // This lane's rows: column l16 of each of the wave's NCT tiles.  A wave
  // whose rows all lie past the block's rows (a short chunk, a decoding
  // sequence) only helps stage the tiles.
  const int rows_end = min(b.rows, (b.rb + 1) * b.rpb);  // past the block's last row
  const int wrow0 = b.rb * b.rpb + wave * 16 * NCT;
  const bool wave_rows = wrow0 < rows_end;
  bool row_ok[NCT];
  int head[NCT], last_seen[NCT];
  int64_t qrow[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int r = wrow0 + 16 * ct + l16;
    row_ok[ct] = r < rows_end;
    const int qi = row_ok[ct] ? r / G : 0;
    head[ct] = kvh * G + (row_ok[ct] ? r % G : 0);
    qrow[ct] = b.t0 + qi;
    last_seen[ct] = b.ctx - b.qlen + qi;  // the row sees tokens 0 .. last_seen
  }

  const int pt = p.partition_tokens;
  const int tok0 = b.nparts > 1 ? part * pt : 0;
  const int tok1 = b.bad ? tok0 : (b.nparts > 1 ? min(b.kv_end, tok0 + pt) : b.kv_end);
  const int pg0 = tok0 / BS;
  const int npg = tok1 > tok0 ? (tok1 - tok0 + BS - 1) / BS : 0;
  const int nsteps = (npg + PPS - 1) / PPS;
  // The two-tile kernel's waves (long, matrix-core bound) take the SIMD
  // before other kernels' waves that are ready in the same cycle, the
  // side-stream decode rows mostly waiting on memory.  Chunked-prefill batch
  // (LLaMA-13B shape) with 16 / 32 / 64 / 128 decodes: 238.9 -> 231.1,
  // 359.8 -> 356.3, 545.8 -> 543.6, 984.9 -> 985.6 us; E4M3 370.3 -> 367.1.
  if constexpr (NCT == 2) __builtin_amdgcn_s_setprio(3);

  // B operand of S^T: Q[row l16 of tile ct][32c + 8 g4 .. +7]; zero for rows
  // past the block.
  bf16x8_t qb[NCT][NC];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) + (qrow[ct] * p.num_heads + head[ct]) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (row_ok[ct]) v = *reinterpret_cast<const uint4*>(qp + 32 * c + 8 * g4);
      // Consumed here, so that the compiler waits for the load before the
      // step loop rather than at its first use inside it, where its wait
      // would also drain the page loads in flight.
      asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
      qb[ct][c] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  f32x4_t acc[NCT][NM];  // O^T[d = 16 m + 4 g4 + j][row l16 of tile ct]
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[ct][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[NCT];  // running max of the row (same in its 4 lanes)
  float l_run[NCT];  // this lane's share of the running sum
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    m_run[ct] = -FLT_MAX;
    l_run[ct] = 0.f;
  }

  // Stage i: K tile at ring + 2 i RTILEB, V tile right after it.  In the
  // tiles the matrix cores read (the stages for bf16, the widened tile for
  // E4M3), K rows hold 16-byte chunk ch at position ch ^ kswz<ROWB>(token);
  // V is chunk-major per 1 KiB (vslot_cm): the bf16 stages and the widened
  // E4M3 tile, and the E4M3 codes as stored.
  __shared__ __attribute__((aligned(16))) unsigned char ring[LDS_BYTES];
  unsigned char* const wide = ring + NSTAGE * 2 * RTILEB;  // E4M3: the widened tile(s)
  unsigned char* const wide_v = wide + (kKRaw ? 0 : TILEB);  // E4M3: the widened V tile

  const TC* kc = static_cast<const TC*>(p.k_cache) + (int64_t)kvh * BS * D;
  const TC* vc = static_cast<const TC*>(p.v_cache) + (int64_t)kvh * BS * D;
  const int32_t* table = p.block_tables + (int64_t)s * p.max_blocks_per_seq;

  // Physical page ids come from the block table through scalar loads: the
  // table is read-only here, so a wave-uniform index into the constant
  // address space reads it through the scalar cache, and those loads count
  // in lgkmcnt, apart from the page loads' vmcnt.  The ids of the next step
  // to be loaded are read at the end of the step before (the barrier at the
  // top of each step waits for them), so the scalar work of issuing a step
  // is a short chain without lane reads.  Entries past the partition's pages
  // are read at its last page (and none of their bytes is loaded).  An id
  // outside the pool reads the pool's last page and marks the block bad:
  // every wave keeps the largest id of the walk, as an unsigned number (so a
  // negative id is larger than any page), over every page of every step, so
  // the flag is the same in all of them.
  using const_i32 = const __attribute__((address_space(4))) int32_t;
  const_i32* const ctable = reinterpret_cast<const_i32*>(reinterpret_cast<uintptr_t>(table + pg0));
  int nid[PPS];  // ids of the pages of the next step to load
  uint32_t id_max = 0;
  const uint32_t id_last = static_cast<uint32_t>(p.num_blocks) - 1u;  // num_blocks >= 1
  auto read_ids = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < PPS; ++q) nid[q] = ctable[min(st * PPS + q, npg - 1)];
  };
  // Pages read by one workgroup only (a sequence of one row block) stream
  // past the caches; the row blocks of a longer chunk share theirs through
  // L2 / MALL.
  const bool stream_pages = b.nrb == 1;

  // Step st's K and V go straight from the cache into stage `stage`.  Load
  // u of wave w fills 64 consecutive 16-byte LDS slots, 64 / CCH whole rows
  // of one page; each lane fetches the chunk its slot holds (bf16 and E4M3 K
  // at D = 128: the swizzled position; other E4M3: as stored), at a byte
  // offset inside the page
  // that does not change along the walk.  The page is reached through a
  // buffer descriptor whose record count ends at the partition's last token,
  // so the rows past it read as zeros and no unread cache bytes (possibly
  // NaN) reach the PV product.
  uint32_t koff[PER_T], voff[PER_T];
#pragma unroll
  for (int u = 0; u < PER_T; ++u) {
    const int slot = (u * kMqWaves + wave) * 64 + lane;
    const int row = slot / CCH;
    const int pos = slot % CCH;
    // V, as stored (E4M3 codes) or as read (bf16): chunk-major per 1 KiB,
    // slot `slot` holding chunk lane / R of token (slot / 64) R + lane % R.
    constexpr int R = 1024 / CROWB;
    const int vrow = (slot / 64) * R + lane % R;
    voff[u] = (vrow % BS) * CROWB + (lane / R) * 16;
    if constexpr (kKRaw) {
      // K codes: 16-byte chunk ch of token `row` at position ch ^ kswz8(row),
      // so the 16 tokens of an 8-byte operand read hit distinct banks.
      koff[u] = (row % BS) * CROWB + ((pos ^ kswz8(row)) << 4);
    } else if constexpr (kFp8) {
      koff[u] = (row % BS) * CROWB + pos * 16;
    } else {
      koff[u] = (row % BS) * CROWB + ((pos ^ kswz<ROWB>(row)) << 4);
    }
  }
  constexpr int kLoadsPerStep = 2 * PER_T;  // per wave that loads (all, but for E4M3 at D = 64)
  // Bytes between consecutive physical pages: below 2^32 (the host bounds
  // the kv heads by 65535), so a page's offset is one 32 x 32-bit product.
  const uint32_t page_bytes = (uint32_t)p.block_stride * (uint32_t)sizeof(TC);
  const uint64_t kbase = reinterpret_cast<uint64_t>(kc);
  const uint64_t vbase = reinterpret_cast<uint64_t>(vc);
  const uint32_t ring_lds = lds_address(ring);
  // Loads step st's pages (ids in nid) into stage `stage`.  Load u of wave w
  // fills LDS slots (u kMqWaves + w) 64 .. +63, which hold page
  // (u kMqWaves + w) 64 / (CCH BS) of the step: the same page for every wave
  // when a page takes at least one load per wave, else a page that also
  // depends on the wave (wave_page for u = 0).
  const int wave_page = wave * 64 / (CCH * BS);
  // A cache of less than 4 GiB is one descriptor per cache for the whole
  // walk, its record count the bytes from this kv head's first page to the
  // cache's end: a whole page is reached through the load's scalar offset
  // (which the range check counts too).  Pages of a partition's last step,
  // whose rows past the partition must read as zeros, and larger caches take
  // a descriptor per page.
  const uint64_t pool_bytes = static_cast<uint64_t>(static_cast<uint32_t>(p.num_blocks)) * page_bytes;
  const bool small_pool = pool_bytes < (1ull << 32);
  const uint32_t pool_records = static_cast<uint32_t>(pool_bytes) - static_cast<uint32_t>(kvh * BS * CROWB);
  const i32x4_t kpool = raw_buffer(kc, pool_records);
  const i32x4_t vpool = raw_buffer(vc, pool_records);
  auto dma_step = [&](int st, int stage) __attribute__((always_inline)) {
    uint32_t id[PPS];
#pragma unroll
    for (int q = 0; q < PPS; ++q) {
      const uint32_t raw = static_cast<uint32_t>(nid[q]);
      id_max = max(id_max, raw);
      id[q] = min(raw, id_last);
    }
    // Tokens of the partition from this step on: every page of the step is
    // whole unless this is its last step.
    const int rem = tok1 - tok0 - st * STEP;
    if (small_pool && rem >= STEP) {
      uint32_t soff[PER_T], kdst[PER_T];
#pragma unroll
      for (int u = 0; u < PER_T; ++u) {
        const int slot0 = (u * kMqWaves + wave) * 64;
        if (slot0 >= CHUNKS) continue;
        uint32_t pid;
        if constexpr (CCH * BS >= kMqWaves * 64) {
          pid = id[u * kMqWaves * 64 / (CCH * BS)];
        } else {
          const int q = u * (kMqWaves * 64 / (CCH * BS)) + wave_page;
          pid = id[0];
#pragma unroll
          for (int r = 1; r < PPS; ++r)
            if (q == r) pid = id[r];
        }
        soff[u] = pid * page_bytes;
        kdst[u] = ring_lds + stage * 2 * RTILEB + slot0 * 16;
      }
      if (stream_pages) {
#pragma unroll
        for (int u = 0; u < PER_T; ++u) {
          if ((u * kMqWaves + wave) * 64 >= CHUNKS) continue;
          buffer_load_lds16<true>(koff[u], kpool, soff[u], kdst[u]);
          buffer_load_lds16<true>(voff[u], vpool, soff[u], kdst[u] + RTILEB);
        }
      } else {
#pragma unroll
        for (int u = 0; u < PER_T; ++u) {
          if ((u * kMqWaves + wave) * 64 >= CHUNKS) continue;
          buffer_load_lds16<false>(koff[u], kpool, soff[u], kdst[u]);
          buffer_load_lds16<false>(voff[u], vpool, soff[u], kdst[u] + RTILEB);
        }
      }
      return;
    }
    i32x4_t kr[PER_T], vr[PER_T];
    uint32_t kdst[PER_T];
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      const int slot0 = (u * kMqWaves + wave) * 64;  // wave-uniform
      if (slot0 >= CHUNKS) continue;
      int q;  // page of the step
      uint32_t pid;
      if constexpr (CCH * BS >= kMqWaves * 64) {
        q = u * kMqWaves * 64 / (CCH * BS);
        pid = id[q];
      } else {
        q = u * (kMqWaves * 64 / (CCH * BS)) + wave_page;
        pid = id[0];
#pragma unroll
        for (int r = 1; r < PPS; ++r)
          if (q == r) pid = id[r];
      }
      const uint64_t page = static_cast<uint64_t>(pid) * page_bytes;
      uint32_t bytes = BS * CROWB;
      if (rem < STEP) bytes = static_cast<uint32_t>(min(max(rem - q * BS, 0), BS)) * CROWB;
      kr[u] = raw_buffer(reinterpret_cast<const void*>(kbase + page), bytes);
      vr[u] = raw_buffer(reinterpret_cast<const void*>(vbase + page), bytes);
      kdst[u] = ring_lds + stage * 2 * RTILEB + slot0 * 16;
    }
    if (stream_pages) {
#pragma unroll
      for (int u = 0; u < PER_T; ++u) {
        if ((u * kMqWaves + wave) * 64 >= CHUNKS) continue;
        buffer_load_lds16<true>(koff[u], kr[u], kdst[u]);
        buffer_load_lds16<true>(voff[u], vr[u], kdst[u] + RTILEB);
      }
    } else {
#pragma unroll
      for (int u = 0; u < PER_T; ++u) {
        if ((u * kMqWaves + wave) * 64 >= CHUNKS) continue;
        buffer_load_lds16<false>(koff[u], kr[u], kdst[u]);
        buffer_load_lds16<false>(voff[u], vr[u], kdst[u] + RTILEB);
      }
    }
  };

  // E4M3: widen stage `stage` (16 codes per chunk, chunk c = token c / CCH,
  // codes at 16 (c % CCH)) into the bf16 tile, two 16-byte chunks per chunk
  // (exact; zero codes, the rows past the partition end, become +0).
  auto widen_step = [&](int stage) __attribute__((always_inline)) {
    const unsigned char* kq = ring + stage * 2 * RTILEB;
    const unsigned char* vq = kq + RTILEB;
    unsigned char* kt = wide;
    unsigned char* vt = wide_v;
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      const int c = tid + u * kMqWaves * 64;
      if (c >= CHUNKS) continue;
      if constexpr (!kKRaw) {
        const int tok = c / CCH;
        const int ch = c % CCH;
        const uint4 kw = *reinterpret_cast<const uint4*>(kq + c * 16);
        *reinterpret_cast<uint4*>(kt + tok * ROWB + (((2 * ch) ^ kswz<ROWB>(tok)) << 4)) = fp8x8_to_bf16x8(kw.x, kw.y);
        *reinterpret_cast<uint4*>(kt + tok * ROWB + (((2 * ch + 1) ^ kswz<ROWB>(tok)) << 4)) = fp8x8_to_bf16x8(kw.z, kw.w);
      }
      // V: consecutive threads take RW consecutive tokens of one code chunk,
      // then of the next, so that both the code reads and the widened
      // chunk-major stores of each 8 lanes fill distinct banks.
      constexpr int RW = 1024 / ROWB;   // widened tokens per KiB
      constexpr int RC = 1024 / CROWB;  // code tokens per KiB
      const int tok = c / (RW * CCH) * RW + c % RW;
      const int ch = c / RW % CCH;
      const uint4 vw = *reinterpret_cast<const uint4*>(vq + (tok / RC) * 1024 + (ch * RC + tok % RC) * 16);
      *reinterpret_cast<uint4*>(vt + vslot_cm<ROWB>(tok, 2 * ch)) = fp8x8_to_bf16x8(vw.x, vw.y);
      *reinterpret_cast<uint4*>(vt + vslot_cm<ROWB>(tok, 2 * ch + 1)) = fp8x8_to_bf16x8(vw.z, vw.w);
    }
  };

  // A step wholly below block_full_end needs no mask: every row of the
  // block sees all of its tokens.  Such steps also take the row max of the
  // raw scores and fold the scale into the exponent, which needs a positive
  // scale.
  const int block_first_qi = b.rb * b.rpb / G;
  const int block_full_end = min(tok1, b.ctx - b.qlen + block_first_qi + 1);

  // kt: the step's K (bf16 tile, or for kKRaw the stage's raw codes); vt:
  // its V tile in the transposed-read layout.
  // The K operand of 16-token tile tt and contraction step c (for kKRaw the
  // raw codes, widened at the product).
  using KRead = std::conditional_t<kKRaw, uint2, uint4>;
  auto read_k = [&](const unsigned char* kt, int tt, int c) __attribute__((always_inline)) {
    const int tok = 16 * tt + l16;
    if constexpr (kKRaw)
      // Codes of columns 32 c + 8 g4 .. +7: half g4 % 2 of chunk 2 c + g4 / 2.
      return *reinterpret_cast<const uint2*>(kt + tok * CROWB + (((2 * c + (g4 >> 1)) ^ kswz8(tok)) << 4) +
                                             (g4 & 1) * 8);
    else
      return *reinterpret_cast<const uint4*>(kt + tok * ROWB + (((4 * c + g4) ^ kswz<ROWB>(tok)) << 4));
  };
  // The first token tile's K operands are read right after the step's
  // barrier, before the page loads are issued, so that their LDS round trip
  // overlaps that scalar work (the E4M3 kernels at D = 64 read K from the
  // widened tile, after the widening).  Measured against no such reads: the
  // chunk-only prefill batch 158 -> 147 us (bf16) and 198 -> 184 us (E4M3),
  // the 70B verification shape 87.4 -> 81.8 us (E4M3) and 101.8 -> 100.4 us
  // (bf16); two of the four operands gave about half of that.
  constexpr int KPRE = kFp8 && !kKRaw ? 0 : NC;
  auto compute_step = [&](int st, const unsigned char* kt, const unsigned char* vt, auto full_tag,
                          const KRead* kpre) __attribute__((always_inline)) {
    constexpr bool kFull = decltype(full_tag)::value;
    const int t_base = tok0 + st * STEP;
    // S^T for the step's 16-token tiles; each K operand read feeds the NCT
    // row tiles.
    f32x4_t sc[NCT][NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) sc[ct][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const KRead kr = tt == 0 && c < KPRE ? kpre[c] : read_k(kt, tt, c);
        uint4 ka;
        if constexpr (kKRaw)
          ka = fp8x8_to_bf16x8(kr.x, kr.y);
        else
          ka = kr;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          sc[ct][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka), qb[ct][c],
                                                               sc[ct][tt], 0, 0, 0);
      }
    }
    // Causal mask and online softmax per tile: lane holds tokens 16 tt + 4 g4 + j.
    // P^T of tile ct as the B operand, two 16-token tiles per product: k slot
    // j of lane group g4 is token 32 h + 4 g4 + j (j < 4) or 32 h + 16 + 4 g4
    // + j - 4.
    // Each lane's maxima first, then the column maxima of all tiles (both
    // tiles' cross-lane steps together).
    uint4 pbits[NCT][NTT / 2];
    float sv[NCT][NTT][4];
    float mxs[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      if constexpr (kFull) {
        float raw = sc[ct][0][0];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
          for (int j = 0; j < 4; ++j) raw = fmaxf(raw, sc[ct][tt][j]);
        mxs[ct] = raw;
      } else {
        float mx = m_run[ct];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int t = t_base + 16 * tt + 4 * g4 + j;
            const bool valid = t < tok1 && t <= last_seen[ct];
            sv[ct][tt][j] = valid ? sc[ct][tt][j] * p.scale_log2e : -__builtin_inff();
            mx = fmaxf(mx, sv[ct][tt][j]);
          }
        mxs[ct] = mx;
      }
    }
    if constexpr (NCT == 2)
      column_max2(mxs[0], mxs[1]);
    else
      mxs[0] = column_max(mxs[0]);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float mx = kFull ? max_of(m_run[ct], mxs[ct] * p.scale_log2e) : mxs[ct];
      if (__any(mx > m_run[ct] + kRescaleLog2)) {
        const float alpha = fast_exp2(m_run[ct] - mx);
        m_run[ct] = mx;
        l_run[ct] *= alpha;
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[ct][m] *= alpha;
      }
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // Masked steps take the same product as unmasked ones for the
          // tokens they keep, so which loop runs a step never changes a bit.
          const float e = fast_exp2(fmaf(sc[ct][tt][j], p.scale_log2e, -m_run[ct]));
          if constexpr (kFull)
            sv[ct][tt][j] = e;
          else
            sv[ct][tt][j] = sv[ct][tt][j] == -__builtin_inff() ? 0.f : e;
        }
      // The running sum adds the weights as rounded to bf16 for the product.
#pragma unroll
      for (int h = 0; h < NTT / 2; ++h) {
        uint4& pb = pbits[ct][h];
        pb.x = pack_bf16x2(sv[ct][2 * h][0], sv[ct][2 * h][1]);
        pb.y = pack_bf16x2(sv[ct][2 * h][2], sv[ct][2 * h][3]);
        pb.z = pack_bf16x2(sv[ct][2 * h + 1][0], sv[ct][2 * h + 1][1]);
        pb.w = pack_bf16x2(sv[ct][2 * h + 1][2], sv[ct][2 * h + 1][3]);
        l_run[ct] = bf16x2_acc(pb.w, bf16x2_acc(pb.z, bf16x2_acc(pb.y, bf16x2_acc(pb.x, l_run[ct]))));
      }
    }
    // O^T += V^T P^T; each V^T operand read feeds the NCT row tiles.
#pragma unroll
    for (int h = 0; h < NTT / 2; ++h) {
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const s16x4_t lo = vt4_cm<ROWB>(vt, l16, 32 * h + 4 * g4, 16 * m);
        const s16x4_t hi = vt4_cm<ROWB>(vt, l16, 32 * h + 16 + 4 * g4, 16 * m);
        const s16x8_t va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          acc[ct][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, va),
                                                               __builtin_bit_cast(bf16x8_t, pbits[ct][h]),
                                                               acc[ct][m], 0, 0, 0);
      }
    }
  };

  // Steps.  The unmasked steps come first and run as a loop of their own;
  // every wave passes the same barriers, so the split point is the
  // workgroup's, set by its first row.
  // (A whole number of ring rounds, so that both loops start at stage 0; the
  // full steps past it take the masked path, which handles them too.)
  const int nfull =
      p.scale_log2e > 0.f ? min(nsteps, max(0, (block_full_end - tok0) / STEP)) / NSTAGE * NSTAGE : 0;
  if (nsteps > 0) {
    read_ids(0);
    // Step st + NSTAGE - 1 is loaded while step st is computed.  At the top
    // of step st the wave waits until only the loads of the steps after st
    // are outstanding (all of them in the last steps); the barrier then
    // publishes step st's stage and frees the stage of step st - 1, which
    // the loads of step st + NSTAGE - 1 reuse (for E4M3 also the widened
    // tile, which a second barrier publishes).
    constexpr int kAhead = NSTAGE - 1;
    for (int st = 0; st < kAhead && st < nsteps; ++st) {
      dma_step(st, st);
      if (st + 1 < nsteps) read_ids(st + 1);
    }
    // Step st on ring stage S (a constant, so every LDS address of the step
    // is a per-lane base plus an immediate offset).
    auto step = [&](int st, auto stage_c, auto full_tag) __attribute__((always_inline)) {
      constexpr int S = decltype(stage_c)::value;
      if (st + kAhead - 1 < nsteps)
        vm_wait<(kAhead - 1) * kLoadsPerStep>();
      else
        vm_wait<0>();
      block_barrier();
      const unsigned char* kt = ring + S * 2 * RTILEB;
      const unsigned char* vt = kt + RTILEB;
      KRead kpre[KPRE > 0 ? KPRE : 1];
      if (wave_rows) {
#pragma unroll
        for (int c = 0; c < KPRE; ++c) kpre[c] = read_k(kt, 0, c);
      }
      if (st + kAhead < nsteps) dma_step(st + kAhead, (S + NSTAGE - 1) % NSTAGE);
      if constexpr (kFp8) {
        widen_step(S);
        block_barrier();
        if constexpr (!kKRaw) kt = wide;
        vt = wide_v;
      }
      if (wave_rows) compute_step(st, kt, vt, full_tag, kpre);
      if (st + kAhead + 1 < nsteps) read_ids(st + kAhead + 1);
    };
    // Steps st0 .. st1 - 1, st0 a multiple of NSTAGE: whole ring rounds.
    auto run_steps = [&](int st0, int st1, auto full_tag) {
      static_assert(NSTAGE == 2 || NSTAGE == 3, "ring rounds of two or three stages");
      for (int st = st0; st < st1;) {
        step(st, std::integral_constant<int, 0>{}, full_tag);
        if (++st == st1) break;
        step(st, std::integral_constant<int, 1>{}, full_tag);
        ++st;
        if constexpr (NSTAGE == 3) {
          if (st == st1) break;
          step(st, std::integral_constant<int, 2>{}, full_tag);
          ++st;
        }
      }
    };
    run_steps(0, nfull, std::true_type{});
    run_steps(nfull, nsteps, std::false_type{});
  }
  const bool bad = b.bad || id_max > id_last;

#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    // The four lanes of a row each hold a share of its running sum.
    float l = l_run[ct];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (!row_ok[ct]) continue;
    const int64_t orow = qrow[ct] * p.num_heads + head[ct];
    if (b.nparts == 1) {
      uint16_t* o = static_cast<uint16_t*>(p.out) + orow * D;
      const float inv = l == 0.f ? 0.f : p.v_scale / l;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = bad ? __builtin_nanf("") : acc[ct][m][j] * inv;
        uint2 w;
        w.x = f32_to_bf16_bits(v[0]) | (uint32_t)f32_to_bf16_bits(v[1]) << 16;
        w.y = f32_to_bf16_bits(v[2]) | (uint32_t)f32_to_bf16_bits(v[3]) << 16;
        *reinterpret_cast<uint2*>(o + 16 * m + 4 * g4) = w;
      }
    } else {
      const int64_t slot = orow * p.max_parts + part;
      float* a = p.ws_acc + slot * D;
#pragma unroll
      for (int m = 0; m < NM; ++m)
        *reinterpret_cast<float4*>(a + 16 * m + 4 * g4) =
            make_float4(acc[ct][m][0], acc[ct][m][1], acc[ct][m][2], acc[ct][m][3]);
      if (g4 == 0) {
        p.ws_ml[slot * 2] = bad ? 0.f : m_run[ct];
        p.ws_ml[slot * 2 + 1] = bad ? __builtin_nanf("") : l;
      }
    }
  }
}

// Verification rows over an E4M3 cache (a sequence of at most 32 rows) in
// the decode kernel's layout instead of the LDS ring: each wave streams its own pages of
// the partition (page pg0 + wave + 4 k) with one page in flight, K straight
// from the cache into the A operand and V through a per-wave LDS page read
// back transposed, and computes all of the sequence's rows as NCT 16-column
// tiles of S^T = K Q^T and O^T += V^T P^T (the K and V^T operands are shared
// by the tiles).  No barrier inside the walk: every wave's dependency chain
// overlaps the others' loads, where the ring's per-step barriers (two for
// E4M3, around the widening) expose it.
// Column l16 of tile ct is row 16 ct + l16 (query r / G, head r % G) with its
// own causal limit; the waves' partial states are merged through LDS, one tile
// at a time, into the row (one partition) or its partition slot, which the
// reduce kernel merges.  Needs the partition's pages to fit one page id per
// lane and wave (partition_tokens <= 256 pages).
template <typename TC, int D, int BS, int G, int NCT>
__global__ __launch_bounds__(kMqWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void multi_query_stream_kernel(MultiQueryParams p) {
  constexpr bool kFp8 = sizeof(TC) == 1;
  constexpr int NT = BS / 16;       // 16-token tiles per page
  constexpr int NC = D / 32;        // 32-wide steps of the QK contraction
  constexpr int NM = D / 16;        // 16-wide output tiles along head_dim
  constexpr int ROWB = D * 2;       // bytes of one bf16 token row (LDS page)
  constexpr int CROWB = D * (int)sizeof(TC);  // bytes of one cache token row
  constexpr int CNCH = CROWB / 16;  // 16-byte cache chunks per row
  constexpr int RPL = 64 / CNCH;    // rows per row-contiguous wave load of V
  constexpr int NV = BS / RPL;      // V loads per lane per page
  constexpr int NKL = kFp8 ? D / 64 : NC;  // K loads per 16-token tile
  constexpr int PAGEB = BS * ROWB;  // bytes of one bf16 page in LDS
  constexpr int EPI = (kMqWaves * 16 * D + 2 * kMqWaves * 16) * 4;
  constexpr int SMEM = kMqWaves * PAGEB > EPI ? kMqWaves * PAGEB : EPI;
  static_assert(NCT >= 1 && NCT * 16 <= kRowsPerBlock && BS % RPL == 0, "tile shape");

  const int kvh = blockIdx.x % p.num_kv_heads;
  const int item = blockIdx.x / p.num_kv_heads;
  int2 w;
  if (p.find_items) {
    if (!find_item<G>(p, item, &w)) return;  // uniform over the workgroup
  } else {
    if (item >= *p.work_count) return;  // uniform over the workgroup
    w = p.work[item];
  }
  const int s = w.x;
  const int part = w.y & 0xffff;
  const MqBlock b = mq_block<G>(p, s, row_block_of(w.y));
  if (b.skip || part >= b.nparts || b.nrb != 1 || b.rows > p.stream_rows) return;  // the ring kernel's

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  const int pt = p.partition_tokens;
  const int tok0 = b.nparts > 1 ? part * pt : 0;
  const int tok1 = b.bad ? tok0 : (b.nparts > 1 ? min(b.kv_end, tok0 + pt) : b.kv_end);
  const int pg0 = tok0 / BS;
  const int npg = tok1 > tok0 ? (tok1 - tok0 + BS - 1) / BS : 0;
  const int nk = npg > wave ? (npg - wave + kMqWaves - 1) / kMqWaves : 0;  // <= 64 (host bound)
  // Pages every row sees in full: no mask.
  const int full_end = min(tok1, b.ctx - b.qlen + 1);

  // Physical id of this wave's page k in lane k (ids outside the pool become
  // 0 and make the wave's results NaN).
  int my_id = 0;
  bool id_bad = false;
  if (lane < nk) {
    my_id = p.block_tables[(int64_t)s * p.max_blocks_per_seq + pg0 + wave + kMqWaves * lane];
    id_bad = my_id < 0 || my_id >= p.num_blocks;
    if (id_bad) my_id = 0;
  }
  const bool bad = b.bad || __any(id_bad);

  // B operands (Q^T) of the tiles: for bf16 caches lane holds row l16's
  // columns 32c + 8 g4 .. +7; for E4M3 caches, whose 16-byte K loads carry 16
  // columns, step c = 2kk + h holds columns 64kk + 16 g4 + 8h .. +7 (the K
  // operand takes the same order).  Zero for rows past the sequence's.
  bf16x8_t qb[NCT][NC];
  int lim[NCT];  // column l16 of tile ct sees tokens < lim[ct]
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int r = 16 * ct + l16;
    const bool row_ok = r < b.rows;
    const int qi = row_ok ? r / G : 0;
    lim[ct] = row_ok ? min(tok1, b.ctx - b.qlen + qi + 1) : 0;
    const uint16_t* qp =
        static_cast<const uint16_t*>(p.q) + ((int64_t)(b.t0 + qi) * p.num_heads + kvh * G + (row_ok ? r % G : 0)) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int col0 = kFp8 ? 64 * (c >> 1) + 16 * g4 + 8 * (c & 1) : 32 * c + 8 * g4;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (row_ok) v = *reinterpret_cast<const uint4*>(qp + col0);
      qb[ct][c] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  f32x4_t acc[NCT][NM];  // O^T[d = 16 m + 4 g4 + j][row 16 ct + l16]
  float m_run[NCT], l_run[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[ct][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[ct] = -FLT_MAX;
    l_run[ct] = 0.f;
  }

  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  unsigned char* vbuf = smem + wave * PAGEB;

  const TC* kc = static_cast<const TC*>(p.k_cache) + (int64_t)kvh * BS * D;
  const TC* vc = static_cast<const TC*>(p.v_cache) + (int64_t)kvh * BS * D;
  const int k_off = l16 * D + (kFp8 ? 16 : 8) * g4;  // A operand: token l16
  const int v_row = lane / CNCH;                     // row-contiguous V load
  const int v_ch = lane % CNCH;
  const int v_off = v_row * D + v_ch * (16 / (int)sizeof(TC));

  auto load_k = [&](int k, uint4 (&kr)[NT][NKL]) {
    const int64_t phys = __builtin_amdgcn_readlane(my_id, k);
    const TC* kp = kc + phys * p.block_stride + k_off;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int c = 0; c < NKL; ++c) kr[tt][c] = load_page16<true>(kp + tt * 16 * D + (kFp8 ? 64 : 32) * c);
  };
  auto load_v = [&](int k, uint4 (&vr)[NV]) {
    const int64_t phys = __builtin_amdgcn_readlane(my_id, k);
    const TC* vp = vc + phys * p.block_stride + v_off;
#pragma unroll
    for (int n = 0; n < NV; ++n) vr[n] = load_page16<true>(vp + n * RPL * D);
  };
  // V page into LDS in the transposed-read layout; rows past the partition
  // end become zeros, so unread cache bytes (possibly NaN) never reach PV.
  auto stage_v = [&](int k, const uint4 (&vr)[NV]) {
    const int t0 = (pg0 + wave + k * kMqWaves) * BS;
    const bool whole = t0 + BS <= tok1;
    wave_lds_fence();
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      const int row = n * RPL + v_row;
      const bool keep = whole || t0 + row < tok1;
      if constexpr (kFp8) {
        uint4 lo = fp8x8_to_bf16x8(vr[n].x, vr[n].y);
        uint4 hi = fp8x8_to_bf16x8(vr[n].z, vr[n].w);
        if (!keep) lo = hi = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(vbuf + row * ROWB + (((2 * v_ch) ^ swz<ROWB>(row)) << 4)) = lo;
        *reinterpret_cast<uint4*>(vbuf + row * ROWB + (((2 * v_ch + 1) ^ swz<ROWB>(row)) << 4)) = hi;
      } else {
        uint4 v = vr[n];
        if (!keep) v = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(vbuf + row * ROWB + ((v_ch ^ swz<ROWB>(row)) << 4)) = v;
      }
    }
    wave_lds_fence();
  };

  auto scores = [&](const uint4 (&kr)[NT][NKL], f32x4_t (&st)[NCT][NT]) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) st[ct][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        uint4 ka;
        if constexpr (kFp8) {
          const uint4& kw = kr[tt][c >> 1];
          ka = (c & 1) ? fp8x8_to_bf16x8(kw.z, kw.w) : fp8x8_to_bf16x8(kw.x, kw.y);
        } else {
          ka = kr[tt][c];
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          st[ct][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka), qb[ct][c],
                                                               st[ct][tt], 0, 0, 0);
      }
  };

  auto softmax_pv = [&](int k, const f32x4_t (&st)[NCT][NT]) {
    const int t0 = (pg0 + wave + k * kMqWaves) * BS;
    const bool full = t0 + BS <= full_end;
    // P^T of each tile (token 16 tt + 4 g4 + j of row l16 in this lane).
    uint32_t pw[NCT][2 * NT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float sv[NT][4];
      float mx = m_run[ct];
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool valid = full || t0 + 16 * tt + 4 * g4 + j < lim[ct];
          sv[tt][j] = valid ? st[ct][tt][j] * p.scale_log2e : -__builtin_inff();
          mx = fmaxf(mx, sv[tt][j]);
        }
      mx = column_max(mx);
      // Lazy rescaling (reference moves only when exceeded by more than
      // 2^kRescaleLog2); a wave-uniform branch per tile.
      if (__any(mx > m_run[ct] + kRescaleLog2)) {
        const float alpha = fast_exp2(m_run[ct] - mx);
        m_run[ct] = mx;
        l_run[ct] *= alpha;
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[ct][m] *= alpha;
      }
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j) sv[tt][j] = fast_exp2(sv[tt][j] - m_run[ct]);
      // The running sum adds the weights as rounded to bf16 for the product.
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        pw[ct][2 * tt] = pack_bf16x2(sv[tt][0], sv[tt][1]);
        pw[ct][2 * tt + 1] = pack_bf16x2(sv[tt][2], sv[tt][3]);
        l_run[ct] = bf16x2_acc(pw[ct][2 * tt + 1], bf16x2_acc(pw[ct][2 * tt], l_run[ct]));
      }
    }
    // O^T += V^T P^T; each V^T read feeds every tile.
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if constexpr (BS == 32) {
        // k slot j of lane group g4: token 4 g4 + j (j < 4) or 16 + 4 g4 + j - 4.
        const s16x4_t lo = vt4<ROWB>(vbuf, l16, 4 * g4, 16 * m);
        const s16x4_t hi = vt4<ROWB>(vbuf, l16, 16 + 4 * g4, 16 * m);
        const s16x8_t va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const uint4 pbits = make_uint4(pw[ct][0], pw[ct][1], pw[ct][2], pw[ct][3]);
          acc[ct][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, va),
                                                               __builtin_bit_cast(bf16x8_t, pbits), acc[ct][m], 0,
                                                               0, 0);
        }
      } else {
        const s16x4_t va = vt4<ROWB>(vbuf, l16, 4 * g4, 16 * m);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const uint2 pbits = make_uint2(pw[ct][0], pw[ct][1]);
          acc[ct][m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, __builtin_bit_cast(s16x4_t, pbits), acc[ct][m],
                                                                 0, 0, 0);
        }
      }
    }
  };

  // One K and one V register buffer per wave, as in the decode kernel: the
  // next page's V is requested once this page's V sits in LDS, the next K
  // once the QK products have consumed this page's K.
  if (!bad && nk > 0) {
    uint4 kr[NT][NKL], vr[NV];
    load_k(0, kr);
    load_v(0, vr);
    for (int k = 0; k < nk; ++k) {
      stage_v(k, vr);
      if (k + 1 < nk) load_v(k + 1, vr);
      f32x4_t st[NCT][NT];
      scores(kr, st);
      if (k + 1 < nk) load_k(k + 1, kr);
      softmax_pv(k, st);
    }
  }

  // Merge the waves' states tile by tile through LDS.
  float* sm_acc = reinterpret_cast<float*>(smem);  // [kMqWaves][16][D]
  float* sm_m = sm_acc + kMqWaves * 16 * D;          // [kMqWaves][16]
  float* sm_l = sm_m + kMqWaves * 16;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    if (16 * ct >= b.rows) break;  // uniform over the workgroup
    float l = l_run[ct];
    l += __shfl_xor(l, 16);  // the four lanes of a column each hold a share
    l += __shfl_xor(l, 32);
    __syncthreads();  // the page buffers (first tile) or the previous tile are done with
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) sm_acc[(wave * 16 + l16) * D + 16 * m + 4 * g4 + j] = acc[ct][m][j];
    if (g4 == 0) {
      sm_m[wave * 16 + l16] = bad ? 0.f : m_run[ct];
      sm_l[wave * 16 + l16] = bad ? __builtin_nanf("") : l;
    }
    __syncthreads();
    for (int idx = tid; idx < 16 * D; idx += kMqWaves * 64) {
      const int c = idx / D;
      const int d = idx % D;
      const int r = 16 * ct + c;
      if (r >= b.rows) continue;
      float mm = -FLT_MAX;
#pragma unroll
      for (int wv = 0; wv < kMqWaves; ++wv) mm = fmaxf(mm, sm_m[wv * 16 + c]);
      float ll = 0.f, aa = 0.f;
#pragma unroll
      for (int wv = 0; wv < kMqWaves; ++wv) {
        const float wt = fast_exp2(sm_m[wv * 16 + c] - mm);
        ll += sm_l[wv * 16 + c] * wt;
        aa += sm_acc[(wv * 16 + c) * D + d] * wt;
      }
      const int64_t orow = (int64_t)(b.t0 + r / G) * p.num_heads + kvh * G + r % G;
      if (b.nparts == 1) {
        const float o = ll == 0.f ? 0.f : aa * (p.v_scale / ll);
        Elem<uint16_t>::store(static_cast<uint16_t*>(p.out) + orow * D + d, o);
      } else {
        const int64_t slot = orow * p.max_parts + part;
        p.ws_acc[slot * D + d] = aa;
        if (d == 0) {
          p.ws_ml[slot * 2] = mm;
          p.ws_ml[slot * 2 + 1] = ll;
        }
      }
    }
  }
}

// The work list: one item per (sequence, row block) of every sequence with
// more than one query, or per (sequence, partition) for a sequence whose rows
// fit one block.  Two classes: first every item but the last partition of a
// cut sequence, in sequence order (a sequence's last row blocks, the ones
// that see the most tokens, first), then those last partitions, the only
// ones shorter than the partition length: here in sequence order, in the
// workgroups' own lookup (batches of at most 64 sequences) longest first.
// Workgroups are placed on the CUs in list order, so the short items spread
// over the CUs and the shortest land on the CUs that already hold the most
// work, instead of some CUs holding only full-length items (an order of
// items never changes the bits).  One workgroup scans the sequences in chunks
// of its size, once per class; items past the list's capacity (only possible
// when query ranges overlap) are dropped.
template <int G>
__global__ __launch_bounds__(256) void multi_query_schedule_kernel(MultiQueryParams p) {
  __shared__ int sums[256];
  __shared__ int base;
  const int tid = threadIdx.x;
  if (tid == 0) base = 0;
  __syncthreads();
  for (int cls = 0; cls < 2; ++cls) {
    for (int s0 = 0; s0 < p.num_seqs; s0 += 256) {
      const int s = s0 + tid;
      int n = 0;
      bool single = false;
      if (s < p.num_seqs) {
        const MqBlock b = mq_block<G>(p, s, 0);
        if (!b.skip) {
          single = b.nrb == 1;
          n = single ? b.nparts : b.nrb;
        }
      }
      const int last = single && n > 1 ? 1 : 0;  // the cut sequence's last partition
      const int m = cls == 0 ? n - last : last;   // this class's items of sequence s
      sums[tid] = m;
      __syncthreads();
      for (int off = 1; off < 256; off <<= 1) {  // inclusive scan
        const int v = tid >= off ? sums[tid - off] : 0;
        __syncthreads();
        sums[tid] += v;
        __syncthreads();
      }
      const int start = base + sums[tid] - m;
      for (int i = 0; i < m && start + i < p.work_capacity; ++i) {
        const int k = cls == 0 ? i : n - 1;
        p.work[start + i] = make_int2(s, single ? k : pack_row_block(k));
      }
      __syncthreads();  // every thread has read base
      if (tid == 255) base += sums[255];
      __syncthreads();
    }
  }
  if (tid == 0) *p.work_count = min(base, p.work_capacity);
}

// Merges the partitions of sequences whose rows fit one block (the only ones
// cut): one workgroup per (sequence, kv head), four threads per row, each
// owning D / 4 output columns, a loop over the partitions.  Launched for
// batches with longer chunks, on which most workgroups find nothing to merge
// and exit at once: small workgroups keep that cheap.
template <int D, int G>
__global__ __launch_bounds__(kMqWaves * 64) void multi_query_reduce_kernel(MultiQueryParams p) {
  constexpr int DQ = D / 4;
  const int kvh = blockIdx.x % p.num_kv_heads;
  const int s = blockIdx.x / p.num_kv_heads;
  const MqBlock b = mq_block<G>(p, s, 0);
  if (b.skip || b.nparts <= 1) return;  // written by the partition kernel
  const int r = b.rb * b.rpb + threadIdx.x / 4;
  if (r >= b.rows) return;
  const int64_t orow = (int64_t)(b.t0 + r / G) * p.num_heads + kvh * G + r % G;
  const float2* ml = reinterpret_cast<const float2*>(p.ws_ml) + orow * p.max_parts;
  float mm = -FLT_MAX;
  for (int q = 0; q < b.nparts; ++q) mm = fmaxf(mm, ml[q].x);
  float ll = 0.f;
  float aa[DQ];
#pragma unroll
  for (int e = 0; e < DQ; ++e) aa[e] = 0.f;
  const int d0 = (threadIdx.x % 4) * DQ;
  for (int q = 0; q < b.nparts; ++q) {
    const float2 v = ml[q];
    const float w = fast_exp2(v.x - mm);
    ll += v.y * w;
    const float4* a = reinterpret_cast<const float4*>(p.ws_acc + (orow * p.max_parts + q) * D + d0);
#pragma unroll
    for (int e = 0; e < DQ / 4; ++e) {
      const float4 f = a[e];
      aa[4 * e] += f.x * w;
      aa[4 * e + 1] += f.y * w;
      aa[4 * e + 2] += f.z * w;
      aa[4 * e + 3] += f.w * w;
    }
  }
  const float inv = ll == 0.f ? 0.f : p.v_scale / ll;
  uint16_t* o = static_cast<uint16_t*>(p.out) + orow * D + d0;
#pragma unroll
  for (int e = 0; e < DQ / 2; ++e) {
    const uint32_t w = f32_to_bf16_bits(aa[2 * e] * inv) | (uint32_t)f32_to_bf16_bits(aa[2 * e + 1] * inv) << 16;
    *reinterpret_cast<uint32_t*>(o + 2 * e) = w;
  }
}

// The same merge for batches in which every sequence's rows fit one block
// (speculative verification), where most sequences are cut: one workgroup of
// 16 waves per (sequence, kv head), four rows per wave, 16 lanes per row, each
// lane owning D / 16 consecutive output columns.  Up to kMqFewParts
// partitions every load of the wave goes out at once and the weights reach
// the column owners by shuffles within the row's 16 lanes; more take a loop.
// Both kernels add the partitions in the same order with the same products,
// so they give the same bits.
constexpr int kMqFewParts = 8;
constexpr int kMqReduceWaves = kRowsPerBlock / 4;

template <int D, int G>
__global__ __launch_bounds__(kMqReduceWaves * 64) void multi_query_reduce_rows_kernel(MultiQueryParams p) {
  constexpr int C = D / 16;  // output columns per lane
  const int kvh = blockIdx.x % p.num_kv_heads;
  const int s = blockIdx.x / p.num_kv_heads;
  const MqBlock b = mq_block<G>(p, s, 0);
  if (b.skip || b.nparts <= 1) return;  // written by the partition kernel
  const int lane = threadIdx.x & 63;
  const int j = lane & 15;                                   // lane within the row
  const int r = (threadIdx.x >> 6) * 4 + (lane >> 4);        // the row
  if (r >= b.rows) return;  // a row's 16 lanes leave together; shuffles stay within a row
  const int64_t orow = (int64_t)(b.t0 + r / G) * p.num_heads + kvh * G + r % G;
  const float2* ml = reinterpret_cast<const float2*>(p.ws_ml) + orow * p.max_parts;
  const float* acc = p.ws_acc + orow * p.max_parts * D + j * C;
  const int n = b.nparts;
  float aa[C];
#pragma unroll
  for (int c = 0; c < C; ++c) aa[c] = 0.f;
  float ll = 0.f;
  if (n <= kMqFewParts) {
    const float2 v = j < n ? ml[j] : make_float2(-FLT_MAX, 0.f);
    float4 a[kMqFewParts][C / 4];
#pragma unroll
    for (int q = 0; q < kMqFewParts; ++q)
#pragma unroll
      for (int c = 0; c < C / 4; ++c)
        a[q][c] = q < n ? *reinterpret_cast<const float4*>(acc + (int64_t)q * D + 4 * c)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    float mm = v.x;
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) mm = fmaxf(mm, __shfl_xor(mm, off, 16));
    const float w = j < n ? fast_exp2(v.x - mm) : 0.f;
#pragma unroll
    for (int q = 0; q < kMqFewParts; ++q) {
      const float wq = __shfl(w, q, 16);
      const float lq = __shfl(v.y, q, 16);
      if (q < n) {
        ll += lq * wq;
#pragma unroll
        for (int c = 0; c < C / 4; ++c) {
          aa[4 * c] += a[q][c].x * wq;
          aa[4 * c + 1] += a[q][c].y * wq;
          aa[4 * c + 2] += a[q][c].z * wq;
          aa[4 * c + 3] += a[q][c].w * wq;
        }
      }
    }
  } else {
    float mm = -FLT_MAX;
    for (int q = 0; q < n; ++q) mm = fmaxf(mm, ml[q].x);
    for (int q = 0; q < n; ++q) {
      const float2 v = ml[q];
      const float w = fast_exp2(v.x - mm);
      ll += v.y * w;
#pragma unroll
      for (int c = 0; c < C / 4; ++c) {
        const float4 f = *reinterpret_cast<const float4*>(acc + (int64_t)q * D + 4 * c);
        aa[4 * c] += f.x * w;
        aa[4 * c + 1] += f.y * w;
        aa[4 * c + 2] += f.z * w;
        aa[4 * c + 3] += f.w * w;
      }
    }
  }
  const float inv = ll == 0.f ? 0.f : p.v_scale / ll;
  uint32_t* o = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.out) + orow * D + j * C);
#pragma unroll
  for (int c = 0; c < C / 2; ++c)
    o[c] = f32_to_bf16_bits(aa[2 * c] * inv) | (uint32_t)f32_to_bf16_bits(aa[2 * c + 1] * inv) << 16;
}

template <typename TC, int D, int BS, int G>
hipError_t launch_t(const MultiQueryLaunch& a, MultiQueryParams p) {
  // When the query ranges cover every row of q, the shortest sequence has at
  // least num_query_tokens - (num_seqs - 1) * max_query_len queries.  Shapes
  // that bound excludes launch nothing for them: a batch whose sequences all
  // have more than 64 rows cuts no context (only single-block sequences are
  // cut) and launches no merge kernel, one whose sequences all have more than
  // the streaming kernel's rows launches no streaming kernel (an empty grid
  // of 4.7 us after the ring kernel on the 70B verification shape over an
  // E4M3 cache).  Ranges that leave rows to no sequence can break the bound;
  // the kernels then serve the short sequences on the ring, uncut, which
  // computes the same rows (their rounding may differ).
  const int64_t min_rows =
      ((int64_t)a.num_query_tokens - (int64_t)(a.num_seqs - 1) * a.max_query_len) * G;
  p.whole_contexts = a.max_parts <= 1 || min_rows > kRowsPerBlock;
  // E4M3 caches at head_dim 64, or without grouping: sequences whose rows fit
  // two 16-row tiles stream on the decode layout (multi_query_stream_kernel),
  // when a partition holds at most 256 pages (one page id per lane and wave).
  // The choice depends on the shape, the sequence and the partition length
  // alone (with ranges that cover every row), so with a fixed partition
  // length a sequence's rows are the same bits in any batch.  Measured over
  // E4M3, 32 sequences of 1024-8192 tokens, default partitions, streaming
  // against the ring: head_dim 64 at G = 8, 4 queries 46.7 against 49.6 us
  // (block size 32: 43.9 / 48.3), G = 4 with 2 queries 37.6 / 43.3; G = 1
  // (40 heads) with 2-4 queries 283-289 / 292-297 (with 32 rows 373 / 345).
  // At head_dim 128 with G >= 2 the 64-token E4M3 ring, with its K codes
  // read in place, wins: G = 8 with 1-4 queries 68.8-71.3 / 63.2-65.1 (block
  // size 32: 96.4 / 70.8), G = 4 and 2 with 8-32 rows 70.6-80.5 / 64.5-71.2.
  // bf16 stays on the ring at every query length (117-144 us against 104-120
  // when last measured).
  constexpr int kStreamRows = sizeof(TC) == 1 && (D == 64 || G == 1) ? 32 : 0;
  p.stream_rows = a.partition_tokens <= 256 * BS && min_rows <= kStreamRows ? kStreamRows : 0;
  const int rows = a.max_query_len * G;  // rows of the longest sequence
  // Up to 64 sequences each workgroup finds its own work item (one wave's
  // scan, no schedule launch: 70B verification shape, bf16, 107.6 -> 104.5
  // us; E4M3 unchanged); larger batches get the list from the schedule
  // kernel.  Same items either way.
  p.find_items = a.num_seqs <= 64;
  hipError_t e = hipSuccess;
  if (!p.find_items) {
    hipLaunchKernelGGL((multi_query_schedule_kernel<G>), dim3(1), dim3(256), 0, a.stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)((int64_t)a.work_capacity * a.num_kv_heads));
  // The ring kernel takes the other sequences, and runs when the batch can
  // hold any.  When every sequence's rows fit one block (each page is read by
  // one workgroup) a two-stage ring (D = 128: 32 KiB of LDS for bf16, 16 + 16
  // KiB for E4M3 with its widened tile) lets four workgroups share a CU;
  // longer chunks, whose row blocks re-read pages from L2, take three stages
  // (48 KiB; E4M3 24 + 16 KiB).  Measured on the 70B-shaped verification
  // batch (bf16): 115 us against 126 us; on the chunked-prefill batch: 690 us
  // against 651 us.
  // Sequences of more than 128 rows run in 128-row blocks on the two-tile
  // kernel, launched first (the longest workgroups); the one-tile kernel
  // takes the rest.
  //
  // Beside the decode kernels (which need many waves in flight to keep HBM
  // busy) the two-tile kernel asks for 64 KiB of LDS per workgroup instead of
  // its 48, so at most two of its workgroups share a CU and the decode
  // waves take the rest.  Measured on the chunked-prefill batch (2048- and
  // 1024-token chunks beside 64 decodes, LLaMA-13B shape): 592 us against
  // 681 us at three per CU; the chunks alone run at the same speed either way
  // (194 us).
  // With a sequence of 128-row blocks in the batch the two-tile kernel is the
  // only ring launch: it also takes the 64-row blocks (two of its waves hold
  // their rows), so no second grid of workgroups that look up their item and
  // exit (chunk-only prefill batch, back-to-back calls: 164.6 -> 160.2 us,
  // E4M3 236.7 -> 232.0 us).
  p.one_ring = rows > 2 * kRowsPerBlock;
  if (p.one_ring) {
    constexpr int kRingBytes = ring_lds_bytes<TC, D, 3>();
    const int pad = a.beside_decode && kRingBytes < 65536 ? 65536 - kRingBytes : 0;
    hipLaunchKernelGGL((multi_query_kernel<TC, D, BS, G, 3, 2>), grid, dim3(kMqWaves * 64), pad, a.stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!p.one_ring && rows > p.stream_rows) {
    // Verification rows over an E4M3 cache take 64-token steps: the step's
    // fixed costs (barriers, issuing the page loads, the waits) are shared by
    // twice the tokens, in a 48 KiB ring.  Measured on the 70B verification
    // shape (6 queries): 32 sequences 89.9 against 95.4 us, 8 sequences 40.1
    // against 41.2, 64 sequences 169.9 against 173.6.
    if constexpr (sizeof(TC) == 1) {
      if (a.max_row_blocks == 1)
        hipLaunchKernelGGL((multi_query_kernel<TC, D, BS, G, 2, 1, 2 * kStepTokens>), grid, dim3(kMqWaves * 64), 0,
                           a.stream, p);
      else
        hipLaunchKernelGGL((multi_query_kernel<TC, D, BS, G, 3, 1>), grid, dim3(kMqWaves * 64), 0, a.stream, p);
    } else if (a.max_row_blocks == 1)
      hipLaunchKernelGGL((multi_query_kernel<TC, D, BS, G, 2, 1>), grid, dim3(kMqWaves * 64), 0, a.stream, p);
    else
      hipLaunchKernelGGL((multi_query_kernel<TC, D, BS, G, 3, 1>), grid, dim3(kMqWaves * 64), 0, a.stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // After the ring kernel: on a chunked-prefill batch, which has no such
  // sequence, its workgroups only look up their item and exit, and launched
  // first they would wait for CU slots ahead of the ring kernel (50 us).
  if constexpr (kStreamRows > 0) {
    if (p.stream_rows > 0) {
      if (rows <= 16)
        hipLaunchKernelGGL((multi_query_stream_kernel<TC, D, BS, G, 1>), grid, dim3(kMqWaves * 64), 0, a.stream, p);
      else
        hipLaunchKernelGGL((multi_query_stream_kernel<TC, D, BS, G, 2>), grid, dim3(kMqWaves * 64), 0, a.stream, p);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (p.whole_contexts) return hipSuccess;  // nothing to merge
  // Verification batches (every sequence one block) merge on the 16-wave
  // kernel, whose loads go out in one round trip (70B verification shape:
  // 4.7 us against 8.3); other batches, where most workgroups exit at once,
  // on the small one (chunked prefill: 4.9 us against 13.7).
  if (a.max_row_blocks == 1)
    hipLaunchKernelGGL((multi_query_reduce_rows_kernel<D, G>), dim3((unsigned)a.num_seqs * a.num_kv_heads),
                       dim3(kMqReduceWaves * 64), 0, a.stream, p);
  else
    hipLaunchKernelGGL((multi_query_reduce_kernel<D, G>), dim3((unsigned)a.num_seqs * a.num_kv_heads),
                       dim3(kMqWaves * 64), 0, a.stream, p);
  return hipGetLastError();
}

template <typename TC, int D, int BS>
hipError_t by_group(const MultiQueryLaunch& a, const MultiQueryParams& p) {
  switch (a.num_heads / a.num_kv_heads) {
    case 1: return launch_t<TC, D, BS, 1>(a, p);
    case 2: return launch_t<TC, D, BS, 2>(a, p);
    case 4: return launch_t<TC, D, BS, 4>(a, p);
    case 8: return launch_t<TC, D, BS, 8>(a, p);
    default: return hipErrorInvalidValue;
  }
}

template <typename TC, int D>
hipError_t by_block(const MultiQueryLaunch& a, const MultiQueryParams& p) {
  return a.block_size == 16 ? by_group<TC, D, 16>(a, p) : by_group<TC, D, 32>(a, p);
}

template <typename TC>
hipError_t by_dim(const MultiQueryLaunch& a, const MultiQueryParams& p) {
  return a.head_dim == 64 ? by_block<TC, 64>(a, p) : by_block<TC, 128>(a, p);
}

}  // namespace

int multi_query_rows_per_block() { return kRowsPerBlock; }

int default_multi_query_partition_tokens(int block_size, int num_seqs, int num_kv_heads, int max_context_len) {
  // Each 32-token step of a workgroup costs about a microsecond of latency,
  // so short partitions win while the grid is small and long ones (fewer
  // partial results to merge) once it fills the chip: the smallest of 512,
  // 1024 and 2048 tokens that keeps (sequence, kv head, partition) items
  // within 1024, four per CU.  Measured on 6-query verification (70B GQA
  // shape, contexts up to 8K): 2-8 sequences 41-56 us at 512 against 72-77
  // at 2048; 16 sequences 75 us at 1024 against 94; 32 sequences 115 us at
  // 2048 against 136 at 1024.
  constexpr int64_t kTargetItems = 1024;
  int t = 512;
  while (t < 2048 && (int64_t)num_seqs * num_kv_heads * (((int64_t)max_context_len + t - 1) / t) > kTargetItems)
    t *= 2;
  return t - t % block_size;
}

hipError_t launch_multi_query(const MultiQueryLaunch& a) {
  MultiQueryParams p;
  p.out = a.out;
  p.q = a.q;
  p.k_cache = a.k_cache;
  p.v_cache = a.v_cache;
  p.block_tables = a.block_tables;
  p.context_lens = a.context_lens;
  p.query_start = a.query_start;
  p.ws_ml = a.ws_ml;
  p.ws_acc = a.ws_acc;
  p.block_stride = (int64_t)a.num_kv_heads * a.block_size * a.head_dim;
  p.max_blocks_per_seq = a.max_blocks_per_seq;
  p.num_seqs = a.num_seqs;
  p.num_query_tokens = a.num_query_tokens;
  p.num_heads = a.num_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.num_blocks = a.num_blocks;
  p.max_context_len = a.max_context_len;
  p.max_query_len = a.max_query_len;
  p.partition_tokens = a.partition_tokens;
  p.max_parts = a.max_parts;
  p.max_row_blocks = a.max_row_blocks;
  p.work = reinterpret_cast<int2*>(a.work);
  p.work_count = a.work_count;
  p.work_capacity = a.work_capacity;
  p.decode_rows_elsewhere = a.decode_rows_elsewhere ? 1 : 0;
  p.stream_rows = 0;  // set per shape by launch_t
  p.one_ring = 0;
  const bool fp8 = a.cache_dtype == kDtypeFp8;
  p.scale_log2e = a.scale * kLog2e * (fp8 ? a.k_scale : 1.f);
  p.v_scale = fp8 ? a.v_scale : 1.f;
  return fp8 ? by_dim<uint8_t>(a, p) : by_dim<uint16_t>(a, p);
}

}  // namespace pa
