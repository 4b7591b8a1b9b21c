// Paged single-token decode attention, split over long contexts.
//
// Semantics: 「Nano-vLLM深度解读（下）」 §4 and 「同一个 Qwen3，两种写法」 §3.4
// (flash_attn_with_kvcache with cache_seqlens and block_table): the single query of
// sequence b attends to its context_lens[b] cached positions, read through its block
// table; Q head h uses KV head h / G (G = Hq/Hkv, the repeat_kv grouping).
//
// Work decomposition (MI355X):
//   grid (split, kv_head, seq), one wave (64 lanes) per workgroup.  A split is
//   `split_tokens` consecutive logical positions of one (sequence, KV head); splits
//   past a sequence's length exit at once.  All G query heads of the group are served
//   by one pass over the K/V bytes.  The wave walks its split in rounds of 16 positions
//   (a round never crosses a block, so its block-table entry is one scalar load).
//   K and V rows of a round are copied HBM -> LDS with global_load_lds (16 bytes per
//   lane; each instruction moves whole 256-byte head rows) into a private 4-stage
//   ring: three rounds are in flight while the wave works on the fourth, and no VGPR
//   is held by a load in flight.  Inside a stage, 16-byte chunk c of row t sits at
//   position c ^ (t mod chunks_per_row) so that reads down a column of rows spread over
//   the LDS banks.  Positions past the end of the split re-read its last row (written
//   and finite) and get weight 0, so the copies need no lane-divergent branches.
//
//   bf16 (MFMA): with GQA, q.K^T of a round is a [G x D] x [D x 16] product and P.V a
//   [G x 16] x [16 x D] one, so both run on the matrix cores with the G heads in the
//   N = 16 columns:  S^T = K Q^T  (v_mfma_f32_16x16x32_bf16, K read straight from
//   the ring) and  O^T += V^T P^T  (v_mfma_f32_16x16x16_bf16, V^T read from the ring
//   with the transposing ds_read_b64_tr_b16, P^T taken from S^T's accumulator
//   registers, whose layout is exactly the B operand's).  Each lane then owns one head
//   column: the running max is a 4-lane exchange (permlane16/32 swaps) and is raised
//   lazily (rescale only when a score exceeds it by more than 2^8, so every weight
//   stays <= 256); the row sum stays in the lane until the end.
//   fp32 (VALU): 8 lanes own one row; each 8-lane group takes 2 positions per round;
//   q.k is summed over the group with DPP; the same lazy running max.
//
//   A sequence with one split writes `out` directly; otherwise (max, sum, weighted
//   values) go to the workspace and decode_reduce_kernel merges the splits.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace nkv {

constexpr int kRound = 16;            // positions per round
#ifndef NKV_DECODE_STAGES
#define NKV_DECODE_STAGES 4
#endif
constexpr int kStages = NKV_DECODE_STAGES;  // LDS ring depth
constexpr float kLazyRescale = 8.0f;  // log2 headroom before rescaling

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;

template <class S, int D>
struct DecGeom {
  static constexpr int EPV = 16 / S::bytes;         // elements per 16-byte chunk
  static constexpr int ROW_BYTES = D * S::bytes;    // one head's row
  static constexpr int CPR = ROW_BYTES / 16;        // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;              // rows per copy instruction
  static constexpr int LPR = kRound / RPI;          // copy instructions per round, K or V
  static constexpr int ROUND_BYTES = kRound * ROW_BYTES;
  static constexpr int STAGE_BYTES = 2 * ROUND_BYTES;  // K then V
  static constexpr int LOADS_PER_ROUND = 2 * LPR;
  // copies allowed in flight while consuming a stage (the counter is 6 bits wide;
  // waiting for fewer than the ring holds is still correct, only less overlapped)
  static constexpr int IN_FLIGHT_LOADS =
      (kStages - 1) * LOADS_PER_ROUND < 63 ? (kStages - 1) * LOADS_PER_ROUND : 63;
  static_assert(CPR <= 64 && 64 % CPR == 0 && (CPR & (CPR - 1)) == 0, "unsupported head_dim");
  // byte offset, inside a stage half, of 16-byte chunk c of row t
  __device__ static constexpr int slot(int t, int c) { return (t * CPR + (c ^ (t & (CPR - 1)))) * 16; }
};

// Block ids of the split's logical blocks, fetched once at the start (a dependent
// load per round would stall the wave for a full memory latency before every copy):
// lane i of register k holds the id of the split's block 64*k + i.
constexpr int kBlkRegs = 4;                 // up to 256 blocks per split
constexpr int kMaxSplitBlocks = 64 * kBlkRegs;

struct SplitBlocks {
  int32_t reg[kBlkRegs];
  int first;
  __device__ void load(const int32_t* trow, int begin, int end, int log2_bs) {
    first = begin >> log2_bs;
    const int n = ((end - 1) >> log2_bs) - first + 1;
#pragma unroll
    for (int k = 0; k < kBlkRegs; ++k) {
      const int i = 64 * k + int(threadIdx.x);
      reg[k] = i < n ? trow[first + i] : 0;
    }
  }
  // id of the block holding logical position `pos` (wave-uniform)
  __device__ int32_t at(int pos, int log2_bs) const {
    const int i = (pos >> log2_bs) - first;
    int32_t v = __builtin_amdgcn_readlane(reg[0], i & 63);
#pragma unroll
    for (int k = 1; k < kBlkRegs; ++k)
      if ((i >> 6) == k) v = __builtin_amdgcn_readlane(reg[k], i & 63);
    return v;
  }
};

// Copies of round r (positions begin + 16r ...) into ring stage r % kStages.
template <class S, int D>
struct Ring {
  using Geo = DecGeom<S, D>;
  const typename S::elem* kbase;
  const typename S::elem* vbase;
  SplitBlocks blocks;
  int64_t row_elems;
  int begin, end, log2_bs, bs_mask;
  int lrow[Geo::LPR];    // row (0..15) this lane copies in instruction j
  int lelem[Geo::LPR];   // element offset of its chunk inside the row

  __device__ void init(int lane) {
#pragma unroll
    for (int j = 0; j < Geo::LPR; ++j) {
      const int s = j * 64 + lane;                 // LDS slot written by this lane
      const int t = s / Geo::CPR;
      const int c = (s % Geo::CPR) ^ (t & (Geo::CPR - 1));
      lrow[j] = t;
      lelem[j] = c * Geo::EPV;
    }
  }

  __device__ void issue(uint8_t* ring, int r) const {
    const int base = begin + r * kRound;
    const int64_t blk0 = int64_t(blocks.at(base, log2_bs)) << log2_bs;
    uint8_t* sk = ring + (r % kStages) * Geo::STAGE_BYTES;
    uint8_t* sv = sk + Geo::ROUND_BYTES;
#pragma unroll
    for (int j = 0; j < Geo::LPR; ++j) {
      const int t = min(base + lrow[j], end - 1);
      const int64_t off = (blk0 + (t & bs_mask)) * row_elems + lelem[j];
      load_lds16(kbase + off, sk + j * 1024);
      load_lds16(vbase + off, sv + j * 1024);
    }
  }
};

template <class S>
__device__ __forceinline__ void store_elem(typename S::elem* p, float x) {
  if constexpr (S::bytes == 2) {
    *p = __builtin_bit_cast(uint16_t, (__bf16)x);  // round to nearest even
  } else {
    *p = x;
  }
}

// ---- bf16: stream-K over (sequence, KV head, round), MFMA -------------------------------
//
// The whole batch is one sequence of "rounds" (16 positions of one KV head): pair
// p = b*Hkv + g owns ceil(L_b/16) consecutive rounds.  Every workgroup takes an equal
// contiguous range of rounds, crossing pair boundaries, so the load is balanced for
// any length mix.  A pair that lies wholly inside one range is finished in place;
// the pieces of a pair cut by range boundaries (at most one at each end of a range)
// are written as partials (max, sum, weighted values) and merged by
// decode_fixup_kernel.  The assignment depends only on the lengths, so results are
// reproducible and independent of the physical block layout.  The K/V copies carry the
// nontemporal hint: a step reads each cached row once, and with the hint a step of 64
// sequences with 512-4096 cached tokens (8 KV heads, 595 MB) went from 115 to 105 us.

#ifndef NKV_SK_STAGES
#define NKV_SK_STAGES 4
#endif
#ifndef NKV_SK_MAX_SEQS
#define NKV_SK_MAX_SEQS 512
#endif
constexpr int kSkStages = NKV_SK_STAGES;  // ring depth (stages - 1 rounds in flight)
constexpr int kSkWindow = 64;         // rounds described per lookahead window
constexpr int kMaxChunkSeqs = NKV_SK_MAX_SEQS;  // sequences per launch (prefix sums in LDS)

template <int D, int G>
struct SkGeom {
  using Row = DecGeom<BF16, D>;
  static constexpr int QROW = D * 2;                       // bytes of one q head
  static constexpr int QCH = QROW / 16;                    // 16-byte chunks per q head
  static constexpr int QI = (G * QROW + 1023) / 1024;      // q copy instructions per round
  static constexpr int QSLOT = QI * 1024;
  static constexpr int STAGE = 2 * Row::ROUND_BYTES + QSLOT;  // K, V, q
  static constexpr int KV_LOADS = 2 * Row::LPR;             // K and V copies of every round
  // q is copied only with the first round of a piece of a pair, so a round has KV_LOADS
  // or KV_LOADS + QI copies; waiting as if every round had KV_LOADS is exact or stricter
  static constexpr int IN_FLIGHT =
      (kSkStages - 1) * KV_LOADS < 63 ? (kSkStages - 1) * KV_LOADS : 63;
};

// How the R rounds of a launch are cut into pieces.  The first Rs rounds are split
// evenly over We persistent workgroups (stream-K); when every workgroup has enough
// rounds and the batch has at least as many (sequence, KV head) pairs as workgroups,
// the last ~15% are cut into U units of L rounds that workgroups claim from a counter
// once their own range is done, so that faster CUs take more of the tail.  With fewer
// pairs than workgroups every pair is already cut into several pieces, and units would
// cut the last pairs into many more (a 40960-token pair into ~160), each a partial for
// the merge.
// Piece p: p < We is workgroup p's range, p >= We is unit p - We.  The cuts depend
// only on R and the grid, never on timing, so the merge order of partials is fixed.
#ifndef NKV_SK_DYN_NUM
#define NKV_SK_DYN_NUM 3              // twentieths of the rounds handed out as units
#endif
#ifndef NKV_SK_UNIT_MIN
#define NKV_SK_UNIT_MIN 16
#endif
#ifndef NKV_SK_DYN_MIN_PER_WG
#define NKV_SK_DYN_MIN_PER_WG 32
#endif
constexpr int kSkDynMinPerWg = NKV_SK_DYN_MIN_PER_WG;   // rounds per workgroup below which no units
constexpr int kSkDynNum = NKV_SK_DYN_NUM, kSkDynDen = 20;
constexpr int kSkUnitMin = NKV_SK_UNIT_MIN;   // rounds per unit, at least
constexpr int kSkMaxUnits = 4096;     // units per launch, at most (workspace slots)

struct SkSplit {
  int64_t R, Rs;
  int We, L, U;
  __device__ int64_t start(int p) const {
    return p < We ? int64_t(p) * Rs / We : Rs + int64_t(p - We) * L;
  }
  __device__ int64_t end(int p) const {
    const int64_t e = start(p + 1);
    return e < R ? e : R;
  }
  __device__ int piece(int64_t t) const {    // piece that holds round t
    return t < Rs ? int(((t + 1) * We - 1) / Rs) : We + int((t - Rs) / L);
  }
};

__device__ __forceinline__ SkSplit make_split(int64_t R, int W, int64_t pairs) {
  SkSplit sp;
  sp.R = R;
  sp.We = R < W ? int(R) : W;               // every static range non-empty
  const int64_t Rd = R >= int64_t(kSkDynMinPerWg) * sp.We && pairs >= sp.We ? R * kSkDynNum / kSkDynDen : 0;
  const int64_t L = Rd > 0 ? (Rd + kSkMaxUnits - 1) / kSkMaxUnits : kSkUnitMin;
  sp.L = int(L > kSkUnitMin ? L : kSkUnitMin);
  sp.U = int((Rd + sp.L - 1) / sp.L);
  sp.Rs = R - Rd;
  return sp;
}

// Descriptor of round t (per lane of a window): which pair, where, how long.
struct SkWin {
  int b;      // sequence
  int g;      // KV head
  int local;  // round inside the pair
  int nr;     // rounds of the pair
};

template <int D, int G>
__global__ void __launch_bounds__(64)
decode_streamk_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
                      const uint16_t* __restrict__ v_cache,
                      const int32_t* __restrict__ context_lens,
                      const int32_t* __restrict__ block_table, int32_t max_blocks,
                      int32_t num_seqs, int32_t num_kv_heads, int32_t log2_bs,
                      float scale_log2e, uint16_t* __restrict__ out,
                      float* __restrict__ ws_part, float* __restrict__ ws_ml,
                      int32_t* __restrict__ ws_prefix, int32_t* __restrict__ ws_claim) {
  using Geo = SkGeom<D, G>;
  using Row = typename Geo::Row;
  constexpr int KS = D / 32;   // k-steps of S^T = K Q^T
  constexpr int DT = D / 16;   // 16-dim tiles of O^T
  static_assert(G <= 16, "the GQA group must fit the 16 MFMA columns");
  __shared__ __attribute__((aligned(16))) uint8_t ring[kSkStages * Geo::STAGE];
  __shared__ int32_t s_prefix[kMaxChunkSeqs + 1];             // rounds before sequence b
  __shared__ int32_t s_phys[2][kSkWindow];                     // block id of each round
  __shared__ int32_t s_len[2][kSkWindow];                      // context length of its sequence

  const int lane = threadIdx.x;
  const int W = gridDim.x;
  const int w = blockIdx.x;
  const int hkv = num_kv_heads;
  const int hq = G * hkv;
  const int bs_mask = (1 << log2_bs) - 1;

  // ---- rounds per sequence, exclusive prefix sums (each lane a contiguous run) ----
  {
    const int per = (num_seqs + 63) / 64;
    const int b0 = lane * per;
    int sum = 0;
    for (int i = 0; i < per; ++i)
      if (b0 + i < num_seqs) sum += (context_lens[b0 + i] + kRound - 1) / kRound;
    int incl = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    int run = incl - sum;
    for (int i = 0; i < per; ++i)
      if (b0 + i < num_seqs) {
        s_prefix[b0 + i] = run;
        run += (context_lens[b0 + i] + kRound - 1) / kRound;
      }
    if (lane == 63) s_prefix[num_seqs] = incl;
    __syncthreads();
  }
  if (w == 0)
    for (int i = lane; i <= num_seqs; i += 64) ws_prefix[i] = s_prefix[i];
  // Workers actually used: never more than there are rounds, so that every range is
  // non-empty (the grid is sized from an upper bound on the lengths).
  const int64_t R = int64_t(hkv) * s_prefix[num_seqs];
  const SkSplit sp = make_split(R, W, int64_t(hkv) * num_seqs);
  if (w >= sp.We) return;
  // The unit counter starts at zero: zeroed here, long before any workgroup finishes
  // its own range and claims, and again by the fixup kernel after every launch.
  if (w == 0 && lane == 0 && sp.U > 0) atomicExch(ws_claim, 0);
  int64_t t0 = sp.start(w), t1 = sp.end(w);  // the range being processed
  int piece = w;                              // its partial slots

  // ---- lookahead windows: lane i describes round wbase + i ----
  auto fill = [&](int64_t wbase, int slot, SkWin& wn) {
    const int64_t t = wbase + lane < t1 ? wbase + lane : t1 - 1;
    int lo = 0, hi = num_seqs - 1;            // last b with hkv * prefix[b] <= t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (int64_t(hkv) * s_prefix[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int nr = s_prefix[lo + 1] - s_prefix[lo];
    const int r = int(t - int64_t(hkv) * s_prefix[lo]);
    const int g = r / nr;
    const int local = r - g * nr;
    wn.b = lo;
    wn.g = g;
    wn.local = local;
    wn.nr = nr;
    load_lds4(block_table + int64_t(lo) * max_blocks + ((local * kRound) >> log2_bs), &s_phys[slot][0]);
    load_lds4(context_lens + lo, &s_len[slot][0]);
  };
  SkWin wa, wb;
  int64_t wbase = t0;        // window slot `wcur` covers [wbase, wbase + 64)
  int wcur = 0;

  struct Desc {
    int b, g, local, nr, len, phys;
  };
  auto desc = [&](int64_t t) -> Desc {
    const int idx = int(t - wbase);
    Desc d;
    if (idx < kSkWindow) {
      d.b = __builtin_amdgcn_readlane(wa.b, idx);
      d.g = __builtin_amdgcn_readlane(wa.g, idx);
      d.local = __builtin_amdgcn_readlane(wa.local, idx);
      d.nr = __builtin_amdgcn_readlane(wa.nr, idx);
      d.len = __builtin_amdgcn_readfirstlane(s_len[wcur][idx]);
      d.phys = __builtin_amdgcn_readfirstlane(s_phys[wcur][idx]);
    } else {
      d.b = __builtin_amdgcn_readlane(wb.b, idx - kSkWindow);
      d.g = __builtin_amdgcn_readlane(wb.g, idx - kSkWindow);
      d.local = __builtin_amdgcn_readlane(wb.local, idx - kSkWindow);
      d.nr = __builtin_amdgcn_readlane(wb.nr, idx - kSkWindow);
      d.len = __builtin_amdgcn_readfirstlane(s_len[wcur ^ 1][idx - kSkWindow]);
      d.phys = __builtin_amdgcn_readfirstlane(s_phys[wcur ^ 1][idx - kSkWindow]);
    }
    return d;
  };

  // ---- copies of one round: K and V rows into the stage, plus the pair's q ----
  // Lane offsets in bytes are fixed for the whole launch: row lrow[j] of the round, the
  // swizzled 16-byte chunk of that row; the round itself is a wave-uniform base address.
  const int row_bytes = hkv * D * 2;                  // one pool row (all KV heads)
  int lrow[Row::LPR], lelem[Row::LPR];
  uint32_t voff[Row::LPR];
#pragma unroll
  for (int j = 0; j < Row::LPR; ++j) {
    const int s = j * 64 + lane;
    lrow[j] = s / Row::CPR;
    lelem[j] = ((s % Row::CPR) ^ (lrow[j] & (Row::CPR - 1))) * Row::EPV;
    voff[j] = uint32_t(lrow[j] * row_bytes + lelem[j] * 2);
  }
  uint32_t qoff[Geo::QI];
#pragma unroll
  for (int j = 0; j < Geo::QI; ++j) {
    const int ch = j * 64 + lane;
    const int head = min(ch / Geo::QCH, G - 1);
    qoff[j] = uint32_t((head * D + (ch % Geo::QCH) * 8) * 2);
  }
  auto issue = [&](int64_t t, const Desc& d) {
    uint8_t* sk = ring + int((t - t0) % kSkStages) * Geo::STAGE;
    uint8_t* sv = sk + Row::ROUND_BYTES;
    uint8_t* sq = sv + Row::ROUND_BYTES;
    const int base = d.local * kRound;
    // the 16 positions of a round lie in one block (block_size >= 16, rounds aligned)
    const int64_t off = ((int64_t(d.phys) << log2_bs) + (base & bs_mask)) * row_bytes +
                        int64_t(d.g) * (D * 2);
    const uint8_t* kb = reinterpret_cast<const uint8_t*>(k_cache) + off;
    const uint8_t* vb = reinterpret_cast<const uint8_t*>(v_cache) + off;
    if (base + kRound <= d.len) {
#pragma unroll
      for (int j = 0; j < Row::LPR; ++j) {
        load_lds16_s_nt(kb, voff[j], sk + j * 1024);
        load_lds16_s_nt(vb, voff[j], sv + j * 1024);
      }
    } else {             // the sequence ends inside this round: rows past it repeat the last
      const int last = d.len - 1 - base;
#pragma unroll
      for (int j = 0; j < Row::LPR; ++j) {
        const uint32_t o = uint32_t(min(lrow[j], last) * row_bytes + lelem[j] * 2);
        load_lds16_s_nt(kb, o, sk + j * 1024);
        load_lds16_s_nt(vb, o, sv + j * 1024);
      }
    }
    if (d.local == 0 || t == t0) {   // q is read only where a pair's piece starts
      const uint8_t* qbase = reinterpret_cast<const uint8_t*>(q) + (int64_t(d.b) * hq + d.g * G) * (D * 2);
#pragma unroll
      for (int j = 0; j < Geo::QI; ++j) load_lds16_s(qbase, qoff[j], sq + j * 1024);
    }
  };
  Desc dd[kSkStages];    // descriptors of the rounds in the ring, oldest first


  // ---- per-lane LDS offsets: K rows (A operand), V^T (transposing reads) ----
  const int col = lane & 15;        // MFMA column = head inside the group
  const int quad = lane >> 4;
  int k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = Row::slot(col, ks * 4 + quad);
  int v_off[DT];
  {
    const int t = 4 * quad + (col >> 2);
    const int d0 = 4 * (col & 3);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int dim = dt * 16 + d0;
      v_off[dt] = Row::slot(t, dim >> 3) + (dim & 7) * 2;
    }
  }

  f32x4_t o[DT];
  bf16x8_t qb[KS];
  float m = -INFINITY, l_part = 0.f;
  int seg_local0 = 0;
  bool seg_first = true;

  // ---- one range [t0, t1): windows, ring prologue, rounds ----
  auto run_range = [&]() {
  wbase = t0;
  wcur = 0;
  fill(wbase, 0, wa);
  fill(wbase + kSkWindow, 1, wb);
  wait_vmcnt<0>();  // the first windows are read right away; later fills land within
                    // two rounds, long before the issue cursor reaches them
#pragma unroll
  for (int i = 0; i < kSkStages - 1; ++i)
    if (t0 + i < t1) {
      dd[i] = desc(t0 + i);
      issue(t0 + i, dd[i]);
    }
  for (int64_t c = t0; c < t1; ++c) {
    if (c - wbase == kSkWindow) {           // slide the lookahead windows
      wbase += kSkWindow;
      wa = wb;
      wcur ^= 1;
      fill(wbase + kSkWindow, wcur ^ 1, wb);
    }
    if (c + kSkStages - 1 < t1) {
      dd[kSkStages - 1] = desc(c + kSkStages - 1);
      issue(c + kSkStages - 1, dd[kSkStages - 1]);
      wait_vmcnt<Geo::IN_FLIGHT>();         // round c has landed
    } else {
      wait_vmcnt<0>();
    }
    const Desc d = dd[0];
#pragma unroll
    for (int i = 0; i + 1 < kSkStages; ++i) dd[i] = dd[i + 1];
    const uint8_t* sk = ring + int((c - t0) % kSkStages) * Geo::STAGE;
    const uint8_t* sv = sk + Row::ROUND_BYTES;
    const uint8_t* sq = sv + Row::ROUND_BYTES;

    if (d.local == 0 || c == t0) {          // a new pair starts here
      m = -INFINITY;
      l_part = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qb[ks] = col < G ? *reinterpret_cast<const bf16x8_t*>(sq + col * Geo::QROW + (ks * 32 + 8 * quad) * 2)
                         : bf16x8_t{};
      seg_local0 = d.local;
      seg_first = c == t0;
    }

    // S^T[16 positions x 16 heads] = K Q^T
    f32x4_t st = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(sk + k_off[ks]);
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[ks], st, 0, 0, 0);
    }
    const int base = d.local * kRound;
    float sc[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool valid = base + 4 * quad + i < d.len;
      sc[i] = valid ? st[i] * scale_log2e : -INFINITY;
      mx = fmaxf(mx, sc[i]);
    }
    mx = xor32_max(xor16_max(mx));
    if (__any(mx > m + kLazyRescale)) {
      const float mn = fmaxf(m, mx);
      const float alpha = fast_exp2(m - mn);
      l_part *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
      m = mn;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sc[i] - m);
    // the row sum adds the bf16-rounded weights that P.V multiplies, so the
    // normalisation matches the weights actually applied
    const uint32_t p01 = pack_bf16x2(p[0], p[1]), p23 = pack_bf16x2(p[2], p[3]);
    l_part = dot2_bf16(p23, 0x3f803f80u, dot2_bf16(p01, 0x3f803f80u, l_part));
    const s16x4_t pb = __builtin_bit_cast(s16x4_t, (u32x2_t){p01, p23});
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const s16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(sv + v_off[dt]));
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, o[dt], 0, 0, 0);
    }

    if (d.local == d.nr - 1 || c == t1 - 1) {   // the piece of this pair ends here
      const float l = xor32_sum(xor16_sum(l_part));
      if (col < G) {
        const int64_t row = int64_t(d.b) * hq + d.g * G + col;
        if (seg_local0 == 0 && d.local == d.nr - 1) {     // whole pair: final output
          const float inv = 1.0f / l;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const u32x2_t wv = {pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv),
                                pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv)};
            *reinterpret_cast<u32x2_t*>(out + row * D + dt * 16 + 4 * quad) = wv;
          }
        } else {                                          // a piece: partial for the fixup
          const int64_t slot = (int64_t(piece) * 2 + (seg_first ? 0 : 1)) * G + col;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            *reinterpret_cast<f32x4_t*>(ws_part + slot * D + dt * 16 + 4 * quad) = o[dt];
          if (quad == 0) {
            ws_ml[slot * 2 + 0] = m;
            ws_ml[slot * 2 + 1] = l;
          }
        }
      }
    }
  }
  };

  run_range();                                 // this workgroup's own range
  // Then units of the tail, claimed one at a time.  The copy ring is drained at the end
  // of every range, so waiting for the claim costs no overlap.
  for (;;) {
    if (sp.U == 0) break;
    int u = 0;
    if (lane == 0) u = atomicAdd(ws_claim, 1);
    u = __builtin_amdgcn_readfirstlane(u);
    // unsigned: a counter value not yet reset (workspace contents on entry are
    // arbitrary) never names a piece; workgroup 0 resets it and then claims until done
    if (unsigned(u) >= unsigned(sp.U)) break;
    piece = sp.We + u;
    t0 = sp.start(piece);
    t1 = sp.end(piece);
    run_range();
  }
}

// Merge the pieces of every pair that a piece boundary cut.  Piece p holds the pair in
// slot 0 if p's range starts inside or at the start of the pair (the pair is p's first
// segment), else in slot 1 (the pair is p's last segment).
//
// One single-wave workgroup per (Q head, sequence); most of them find their pair whole and
// leave at once.  Lane l owns the 16-byte column chunk l % (D/4) of the partial rows of
// pieces l / (D/4), l / (D/4) + PG, ... of a chunk of kFixPieces pieces: all of a chunk's
// row and (m, l) loads are issued together, and the next chunk's before this one is
// summed, so even a pair cut into a hundred pieces costs about one memory round trip.
// Across chunks the sums are rescaled to the running maximum.  Every sum runs in a fixed
// order, so the result is deterministic.
constexpr int kFixPieces = 32;

template <int D, int G>
__global__ void __launch_bounds__(64)
decode_fixup_kernel(const int32_t* __restrict__ prefix, int32_t num_seqs, int32_t num_kv_heads,
                    int32_t W, const float* __restrict__ ws_part, const float* __restrict__ ws_ml,
                    int32_t* __restrict__ ws_claim, uint16_t* __restrict__ out) {
  constexpr int NCH = D / 4;                  // 16-byte chunks of a partial row
  constexpr int PG = 64 / NCH;                // pieces per pass
  constexpr int NP = kFixPieces / PG;        // passes per chunk
  static_assert(NCH <= 64 && 64 % NCH == 0 && kFixPieces % PG == 0, "unsupported head_dim");
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int g = h / G;
  const int col = h % G;
  const int lane = threadIdx.x;
  if (h == 0 && b == 0 && lane == 0) atomicExch(ws_claim, 0);   // for the next launch
  const int64_t R = int64_t(num_kv_heads) * prefix[num_seqs];
  const int nr = prefix[b + 1] - prefix[b];
  if (nr == 0 || R == 0) return;
  const SkSplit sp = make_split(R, W, int64_t(num_kv_heads) * num_seqs);   // the stream-K kernel's pieces
  const int64_t s = int64_t(num_kv_heads) * prefix[b] + int64_t(g) * nr;   // first round
  const int64_t e = s + nr;                                               // past the last
  const int w0 = sp.piece(s), w1 = sp.piece(e - 1);
  if (w0 == w1) return;                      // finished in place
  const int np = w1 - w0 + 1;
  auto slot_of = [&](int w) {
    const int k = sp.start(w) >= s ? 0 : 1;
    return (w * 2 + k) * G + col;
  };
  const int c = lane % NCH, pg = lane / NCH;
  float M = -INFINITY, den = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  // Issue every load of the chunk at c0.  Lane i < kFixPieces locates piece c0 + i once
  // (the split's divisions) and reads its (m, l); the row loads get slots by shuffles.
  auto load = [&](int c0, f32x4_t (&row)[NP], float& my_m, float& my_l) {
    const bool mine = lane < kFixPieces && c0 + lane < np;
    const int my_slot = mine ? slot_of(w0 + c0 + lane) : 0;
    my_m = mine ? ws_ml[int64_t(my_slot) * 2] : -INFINITY;
    my_l = mine ? ws_ml[int64_t(my_slot) * 2 + 1] : 0.f;
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int src = k * PG + pg;
      const int64_t sl = __shfl(my_slot, src);
      row[k] = c0 + src < np ? *reinterpret_cast<const f32x4_t*>(ws_part + sl * D + 4 * c)
                             : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  // Fold a loaded chunk into the running sums (pieces past np have m = -inf, weight 0).
  auto consume = [&](const f32x4_t (&row)[NP], float my_m, float my_l) {
    float mn = my_m;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mn = fmaxf(mn, __shfl_xor(mn, off));
    mn = fmaxf(mn, M);
    const float alpha = fast_exp2(M - mn);        // 0 on the first chunk (M = -inf)
    acc *= alpha;
    den *= alpha;
    M = mn;
    const float my_w = fast_exp2(my_m - M);
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int src = k * PG + pg;
      const float wt = __shfl(my_w, src);
      acc += wt * row[k];
      den = fmaf(wt, __shfl(my_l, src), den);     // every lane of a piece group alike
    }
  };
  // Two chunks in flight: the next chunk's loads go out before this one is folded in.
  f32x4_t ra[NP], rb[NP];
  float ma, la, mb, lb;
  load(0, ra, ma, la);
  for (int c0 = 0; c0 < np; c0 += 2 * kFixPieces) {
    const bool has_b = c0 + kFixPieces < np;
    if (has_b) load(c0 + kFixPieces, rb, mb, lb);
    consume(ra, ma, la);
    if (!has_b) break;
    if (c0 + 2 * kFixPieces < np) load(c0 + 2 * kFixPieces, ra, ma, la);
    consume(rb, mb, lb);
  }
  // sum the PG piece groups (lanes c, c + NCH, ...) in a fixed order
#pragma unroll
  for (int off = NCH; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] += __shfl_xor(acc[j], off);
    den += __shfl_xor(den, off);
  }
  if (lane < NCH) {
    const float inv = 1.0f / den;
    const int64_t orow = int64_t(b) * num_kv_heads * G + h;
    const u32x2_t w2 = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
    *reinterpret_cast<u32x2_t*>(out + orow * D + 4 * lane) = w2;
  }
}

// ---- fp32: VALU ---------------------------------------------------------------------------

__device__ __forceinline__ float group_sum_all(float x) {  // over the 8 groups of 8 lanes
  x += dpp<kDppRowRor8>(x);
  x = xor16_sum(x);
  return xor32_sum(x);
}

template <int D, int G>
__global__ void __launch_bounds__(64)
decode_split_f32_kernel(const float* __restrict__ q, const float* __restrict__ k_cache,
                        const float* __restrict__ v_cache, const int32_t* __restrict__ context_lens,
                        const int32_t* __restrict__ block_table, int32_t max_blocks,
                        int32_t num_kv_heads, int32_t log2_bs, float scale_log2e,
                        int32_t split_tokens, int32_t max_splits, float* __restrict__ out,
                        float* __restrict__ ws_ml, float* __restrict__ ws_acc) {
  using Geo = DecGeom<F32, D>;
  constexpr int EPV = Geo::EPV;               // 4 floats per chunk
  constexpr int NV = D / (8 * EPV);           // chunks per lane per row
  constexpr int DPL = NV * EPV;               // dims per lane
  constexpr int TPG = 2;                      // positions per 8-lane group per round
  __shared__ __attribute__((aligned(16))) uint8_t ring[kStages * Geo::STAGE_BYTES];

  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int ctx = context_lens[b];
  const int begin = split * split_tokens;
  if (begin >= ctx) return;
  const int end = min(ctx, begin + split_tokens);
  const int nsplit = (ctx + split_tokens - 1) / split_tokens;
  const int nr = (end - begin + kRound - 1) / kRound;

  const int lane = threadIdx.x;
  const int grp = lane >> 3;
  const int u = lane & 7;
  const int hq = G * num_kv_heads;

  Ring<F32, D> rg;
  rg.kbase = k_cache + int64_t(g) * D;
  rg.vbase = v_cache + int64_t(g) * D;
  rg.blocks.load(block_table + int64_t(b) * max_blocks, begin, end, log2_bs);
  rg.row_elems = int64_t(num_kv_heads) * D;
  rg.begin = begin;
  rg.end = end;
  rg.log2_bs = log2_bs;
  rg.bs_mask = (1 << log2_bs) - 1;
  rg.init(lane);

  // lane u owns chunks v*8+u (v < NV) of a row
  u32x4_t qv[G][NV];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int v = 0; v < NV; ++v)
      qv[h][v] = *reinterpret_cast<const u32x4_t*>(q + (int64_t(b) * hq + g * G + h) * D +
                                                   (v * 8 + u) * EPV);
#pragma unroll
  for (int r = 0; r < kStages - 1; ++r)
    if (r < nr) rg.issue(ring, r);

  float m[G], l[G], acc[G][DPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int d = 0; d < DPL; ++d) acc[h][d] = 0.f;
  }

  for (int r = 0; r < nr; ++r) {
    if (r + kStages - 1 < nr) {
      rg.issue(ring, r + kStages - 1);
      wait_vmcnt<Geo::IN_FLIGHT_LOADS>();
    } else {
      wait_vmcnt<0>();
    }
    const int base = begin + r * kRound;
    const uint8_t* sk = ring + (r % kStages) * Geo::STAGE_BYTES;
    const uint8_t* sv = sk + Geo::ROUND_BYTES;

    float sc[TPG][G];
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
      const int t = grp * TPG + i;
      const bool valid = base + t < end;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float dot = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const u32x4_t kk = *reinterpret_cast<const u32x4_t*>(sk + Geo::slot(t, v * 8 + u));
#pragma unroll
          for (int w = 0; w < 4; ++w)
            dot = fmaf(__uint_as_float(kk[w]), __uint_as_float(qv[h][v][w]), dot);
        }
        dot = group8_sum(dot) * scale_log2e;
        sc[i][h] = valid ? dot : -INFINITY;
      }
    }
    bool need = false;
    float mx[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mx[h] = fmaxf(sc[0][h], sc[1][h]);
      need |= mx[h] > m[h] + kLazyRescale;
    }
    if (__any(need)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float wm = fmaxf(mx[h], dpp<kDppRowRor8>(mx[h]));
        wm = xor32_max(xor16_max(wm));
        const float mn = fmaxf(m[h], wm);
        const float alpha = fast_exp2(m[h] - mn);
        l[h] *= alpha;
#pragma unroll
        for (int d = 0; d < DPL; ++d) acc[h][d] *= alpha;
        m[h] = mn;
      }
    }
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
      const int t = grp * TPG + i;
      u32x4_t vv[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) vv[v] = *reinterpret_cast<const u32x4_t*>(sv + Geo::slot(t, v * 8 + u));
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = fast_exp2(sc[i][h] - m[h]);
        l[h] += p;
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
          for (int e = 0; e < EPV; ++e)
            acc[h][v * EPV + e] = fmaf(p, __uint_as_float(vv[v][e]), acc[h][v * EPV + e]);
      }
    }
  }

#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = group_sum_all(l[h]);
#pragma unroll
    for (int d = 0; d < DPL; ++d) acc[h][d] = group_sum_all(acc[h][d]);
  }
  const int64_t row0 = int64_t(b) * hq + g * G;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (grp != h) continue;  // group h writes head h
    const int64_t row = row0 + h;
    if (nsplit == 1) {
      const float inv = 1.0f / l[h];
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < EPV; ++e) out[row * D + (v * 8 + u) * EPV + e] = acc[h][v * EPV + e] * inv;
    } else {
      const int64_t slot = row * max_splits + split;
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < EPV; ++e) ws_acc[slot * D + (v * 8 + u) * EPV + e] = acc[h][v * EPV + e];
      if (u == 0) {
        ws_ml[slot * 2 + 0] = m[h];
        ws_ml[slot * 2 + 1] = l[h];
      }
    }
  }
}

// Merge the splits of each (sequence, Q head): weights exp2(m_s - max_s m_s).
template <class S, int D>
__global__ void __launch_bounds__(64)
decode_reduce_kernel(const int32_t* __restrict__ context_lens, int32_t split_tokens,
                     int32_t max_splits, int32_t num_q_heads,
                     const float* __restrict__ ws_ml, const float* __restrict__ ws_acc,
                     typename S::elem* __restrict__ out) {
  constexpr int DPT = D / 64;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int ctx = context_lens[b];
  const int ns = (ctx + split_tokens - 1) / split_tokens;
  if (ns <= 1) return;
  const int64_t row = int64_t(b) * num_q_heads + h;
  const float* ml = ws_ml + row * max_splits * 2;
  const float* acc = ws_acc + row * max_splits * D;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[2 * s]);
  float den = 0.f, num[DPT];
#pragma unroll
  for (int j = 0; j < DPT; ++j) num[j] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float w = fast_exp2(ml[2 * s] - M);
    den = fmaf(w, ml[2 * s + 1], den);
#pragma unroll
    for (int j = 0; j < DPT; ++j) num[j] = fmaf(w, acc[int64_t(s) * D + threadIdx.x + 64 * j], num[j]);
  }
  const float inv = 1.0f / den;
#pragma unroll
  for (int j = 0; j < DPT; ++j) store_elem<S>(out + row * D + threadIdx.x + 64 * j, num[j] * inv);
}

// ---- host side -----------------------------------------------------------------------

template <int D, int G>
static int streamk_blocks_per_cu() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_streamk_kernel<D, G>, 64, 0) !=
            hipSuccess ||
        n <= 0)
      n = 4;
    cached[dev] = n;
  }
  return cached[dev];
}

static int streamk_occupancy(int d, int grp) {
  if (d == 128) {
    switch (grp) {
      case 1: return streamk_blocks_per_cu<128, 1>();
      case 2: return streamk_blocks_per_cu<128, 2>();
      case 4: return streamk_blocks_per_cu<128, 4>();
      case 8: return streamk_blocks_per_cu<128, 8>();
    }
  } else {
    switch (grp) {
      case 1: return streamk_blocks_per_cu<64, 1>();
      case 2: return streamk_blocks_per_cu<64, 2>();
      case 4: return streamk_blocks_per_cu<64, 4>();
      case 8: return streamk_blocks_per_cu<64, 8>();
    }
  }
  return 4;
}

static size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

DecodePlan plan_decode(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                       int num_cus) {
  DecodePlan p{};
  const int64_t max_tokens = int64_t(max_blocks_per_seq) * block_size;
  const int64_t pairs = int64_t(num_seqs) * num_kv_heads;
  const int grp = num_q_heads / num_kv_heads;

  // fp32 split-K: largest split that still gives ~8 single-wave workgroups per CU when
  // every sequence is at its maximum length; at most 2048 positions per workgroup.
  int32_t split = 256;
  const char* env = getenv("NKV_DECODE_SPLIT_TOKENS");
  if (env && atoi(env) >= kRound && atoi(env) % kRound == 0 && atoi(env) <= 16 * kMaxSplitBlocks) {
    split = atoi(env);
  } else {
    for (int32_t cand = 2048; cand >= 256; cand /= 2) {
      const int64_t wgs = pairs * ((max_tokens + cand - 1) / cand);
      if (wgs >= int64_t(8) * num_cus) {
        split = cand;
        break;
      }
    }
  }
  p.split_tokens = split;
  p.max_splits = int32_t((max_tokens + split - 1) / split);
  if (p.max_splits < 1) p.max_splits = 1;
  const size_t ws_f32 = p.max_splits <= 1 ? 0
                                          : size_t(num_seqs) * num_q_heads * p.max_splits *
                                                (head_dim + 2) * sizeof(float);

  // bf16 stream-K: one workgroup per resident slot, never more than there are rounds.
  p.seq_chunk = num_seqs < kMaxChunkSeqs ? num_seqs : kMaxChunkSeqs;
  const int64_t max_rounds =
      int64_t(num_kv_heads) * p.seq_chunk * ((max_tokens + kRound - 1) / kRound);
  int64_t wgs = int64_t(num_cus) * streamk_occupancy(head_dim, grp);
  const char* wenv = getenv("NKV_DECODE_WORKGROUPS");
  if (wenv && atoi(wenv) > 0) wgs = atoi(wenv);
  if (wgs > max_rounds) wgs = max_rounds;
  if (wgs < 1) wgs = 1;
  p.wgs = int32_t(wgs);
  // partial slots: one pair of slots per workgroup range, plus per tail unit when the
  // kernel's own condition can hold (rounds can reach kSkDynMinPerWg per workgroup and
  // the chunk has at least as many pairs as workgroups); units have >= kSkUnitMin rounds
  const int64_t max_pairs = int64_t(num_kv_heads) * p.seq_chunk;
  int64_t units = 0;
  if (max_rounds >= int64_t(kSkDynMinPerWg) * p.wgs && max_pairs >= p.wgs) {
    const int64_t rd = max_rounds * kSkDynNum / kSkDynDen;
    units = (rd + kSkUnitMin - 1) / kSkUnitMin;
    if (units > kSkMaxUnits) units = kSkMaxUnits;
  }
  p.pieces = int32_t(p.wgs + units);
  const size_t ws_bf16 = num_seqs <= 0 ? 0
                                       : align16(size_t(p.pieces) * 2 * grp * head_dim * sizeof(float)) +
                                             align16(size_t(p.pieces) * 2 * grp * 2 * sizeof(float)) +
                                             align16(size_t(p.seq_chunk + 1) * sizeof(int32_t)) +
                                             16;   // the unit counter
  p.workspace_bytes = ws_f32 > ws_bf16 ? ws_f32 : ws_bf16;
  return p;
}

template <int D, int G>
static hipError_t launch_bf16_t(const DecodeArgs& a, const DecodePlan& plan, hipStream_t st) {
  const PagedArgs& p = a.p;
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  float* ws_part = reinterpret_cast<float*>(ws);
  float* ws_ml = reinterpret_cast<float*>(ws + align16(size_t(plan.pieces) * 2 * G * D * sizeof(float)));
  int32_t* ws_prefix = reinterpret_cast<int32_t*>(
      reinterpret_cast<uint8_t*>(ws_ml) + align16(size_t(plan.pieces) * 2 * G * 2 * sizeof(float)));
  int32_t* ws_claim = reinterpret_cast<int32_t*>(
      reinterpret_cast<uint8_t*>(ws_prefix) + align16(size_t(plan.seq_chunk + 1) * sizeof(int32_t)));
  const int64_t row = int64_t(p.num_q_heads) * D;
  for (int32_t c0 = 0; c0 < p.num_seqs; c0 += plan.seq_chunk) {
    const int32_t n = p.num_seqs - c0 < plan.seq_chunk ? p.num_seqs - c0 : plan.seq_chunk;
    const uint16_t* q = static_cast<const uint16_t*>(a.q) + c0 * row;
    uint16_t* out = static_cast<uint16_t*>(a.out) + c0 * row;
    const int32_t* lens = a.context_lens + c0;
    const int32_t* table = p.block_table + int64_t(c0) * p.max_blocks_per_seq;
    hipLaunchKernelGGL((decode_streamk_kernel<D, G>), dim3(plan.wgs), dim3(64), 0, st, q,
                       static_cast<const uint16_t*>(p.k_cache), static_cast<const uint16_t*>(p.v_cache),
                       lens, table, p.max_blocks_per_seq, n, p.num_kv_heads, p.log2_block_size,
                       p.scale_log2e, out, ws_part, ws_ml, ws_prefix, ws_claim);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_fixup_kernel<D, G>), dim3(p.num_q_heads, n), dim3(64), 0, st,
                       ws_prefix, n, p.num_kv_heads, plan.wgs, ws_part, ws_ml, ws_claim, out);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int D, int G>
static hipError_t launch_f32_t(const DecodeArgs& a, const DecodePlan& plan, hipStream_t st) {
  const PagedArgs& p = a.p;
  float* ws_ml = static_cast<float*>(a.workspace);
  float* ws_acc = ws_ml ? ws_ml + size_t(p.num_seqs) * p.num_q_heads * plan.max_splits * 2
                        : nullptr;
  const dim3 grid(plan.max_splits, p.num_kv_heads, p.num_seqs);
  hipLaunchKernelGGL((decode_split_f32_kernel<D, G>), grid, dim3(64), 0, st,
                     static_cast<const float*>(a.q), static_cast<const float*>(p.k_cache),
                     static_cast<const float*>(p.v_cache), a.context_lens, p.block_table,
                     p.max_blocks_per_seq, p.num_kv_heads, p.log2_block_size, p.scale_log2e,
                     plan.split_tokens, plan.max_splits, static_cast<float*>(a.out), ws_ml, ws_acc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.max_splits <= 1) return e;
  hipLaunchKernelGGL((decode_reduce_kernel<F32, D>), dim3(p.num_q_heads, p.num_seqs), dim3(64), 0,
                     st, a.context_lens, plan.split_tokens, plan.max_splits, p.num_q_heads,
                     ws_ml, ws_acc, static_cast<float*>(a.out));
  return hipGetLastError();
}

template <int D>
static hipError_t dispatch_g(const DecodeArgs& a, const DecodePlan& plan, hipStream_t st) {
  const bool bf = a.p.dtype == Dtype::BF16;
  switch (a.p.num_q_heads / a.p.num_kv_heads) {
    case 1: return bf ? launch_bf16_t<D, 1>(a, plan, st) : launch_f32_t<D, 1>(a, plan, st);
    case 2: return bf ? launch_bf16_t<D, 2>(a, plan, st) : launch_f32_t<D, 2>(a, plan, st);
    case 4: return bf ? launch_bf16_t<D, 4>(a, plan, st) : launch_f32_t<D, 4>(a, plan, st);
    case 8: return bf ? launch_bf16_t<D, 8>(a, plan, st) : launch_f32_t<D, 8>(a, plan, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan, hipStream_t st) {
  if (a.p.head_dim == 128) return dispatch_g<128>(a, plan, st);
  if (a.p.head_dim == 64) return dispatch_g<64>(a, plan, st);
  return hipErrorInvalidValue;
}

}  // namespace nkv
