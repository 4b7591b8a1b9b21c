// Paged causal varlen prefill attention.
//
// Semantics: 「同一个 Qwen3，两种写法」 §3.2 (flat [T, H, D] batch cut by cu_seqlens,
// causal inside each segment, no work across segments), §3.3 (K/V read from the paged
// pool through the block table) and §3.4 (GQA handled inside the kernel);
// 「Nano-vLLM深度解读（下）」 §4 (flash_attn_varlen_func(..., causal=True,
// block_table=...)).  Query i of a segment with Lq queries and Lk keys sits at position
// Lk - Lq + i and sees keys j <= Lk - Lq + i.
//
// bf16 path (dense contraction -> MFMA, v_mfma_f32_16x16x32_bf16):
//   grid (seq * kv_head, pair of consecutive q-tiles), longest pairs dispatched first.  A
//   workgroup of 8 waves (two per SIMD) holds the G query heads of one KV head; each wave
//   owns 32 queries of one head, two 16-query MFMA column blocks.  The second q-tile of a
//   pair starts on the first one's last K/V tile, still in LDS, and its q is copied into
//   LDS during that tile, so it needs no prologue of its own.  K/V tiles of 128 keys are
//   gathered through the block table into a double-buffered LDS stage shared by all
//   waves: K and V rows are copied HBM -> LDS directly, by waves 0-3 only (global_load_lds,
//   chunk c of row t at c ^ kv_swz(t), free of bank conflicts for both kinds of read).  K fragments are 16-byte LDS reads; V^T
//   fragments come from the transposing LDS read (ds_read_b64_tr_b16), two per fragment,
//   in the key order of the P^T operand.  The next tile's copies are in flight while the current
//   tile is computed.
//   Scores are computed transposed, S^T = K Q^T, in 16x16 blocks: a lane holds 4 keys of
//   one query per block, so the max of a query spans four lanes.  P goes from the S^T accumulators straight into the B
//   operand of O^T += V^T P^T.  A tile is processed as four 32-key halves, each QK ->
//   softmax -> PV; the 16x16 blocks let the softmax of the half's first key block start
//   after 4 of the QK MFMAs instead of all of them (a 32x32 block needs every k-step).
//   The softmax uses one FMA + exp2 per score (scale folded in), the running max is
//   raised lazily (rescale only past 2^8 headroom, detected from the weights' sum), and
//   the row sum of the rounded bf16 weights comes from one more MFMA per query block and
//   half, with a fragment of ones in place of V^T, which hands every lane of a query its
//   full sum (8 dot2 per half on the VALU cost more than the 2 MFMAs).  Only halves that cross the
//   causal diagonal or the end of the keys are masked.  The output goes through LDS so
//   each row is written as one contiguous run, with nontemporal stores.
// fp32 path: a plain VALU kernel (one lane per query and head, online softmax), used
//   for correctness-sized fp32 inputs.
#include <math.h>
#include <stdlib.h>

#include "common.hpp"
#include "launch.hpp"

namespace nkv {

#ifndef NKV_PREFILL_BK
#define NKV_PREFILL_BK 128
#endif
#ifndef NKV_PREFILL_NW
#define NKV_PREFILL_NW 8
#endif
#ifndef NKV_PREFILL_PRIO
#define NKV_PREFILL_PRIO 0
#endif
#ifndef NKV_PREFILL_PAIR
#define NKV_PREFILL_PAIR 1
#endif

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;   // one transposing LDS read

constexpr int kBK = NKV_PREFILL_BK;     // keys per tile (a multiple of 32)
constexpr int kStages = 2;              // K/V tiles in LDS (one computed, one landing)
constexpr float kLazyBound = 256.0f;    // largest weight kept before rescaling (2^8 headroom)
constexpr int kMaxIds = kBK / 16;       // block ids per tile (block_size >= 16)
constexpr int kLog2BK = kBK == 128 ? 7 : 6;
constexpr bool kPairQTiles = NKV_PREFILL_PAIR;   // two consecutive q-tiles per workgroup
static_assert(kBK == 64 || kBK == 128, "64- or 128-key tiles");

// Swizzle of the 16-byte chunks of a K/V tile row in LDS: logical chunk c of row t sits at
// c ^ kv_swz(t).  It must keep two read patterns free of bank conflicts: the K fragment
// reads (ds_read_b128, 16 consecutive rows at one logical chunk per 16 lanes) and the V^T
// transposing reads (ds_read_b64_tr_b16, 4 consecutive rows x 2 adjacent chunks per 16
// lanes).  Plain c ^ (t % 16) leaves the transposing reads 2 extra cycles each (a third
// of all LDS cycles in conflict); the map below was found by counting
// SQ_LDS_BANK_CONFLICT over candidate maps in a read-only probe and is conflict-free for
// both (bits of the result, high to low: t0, t2 ^ t3, t1 ^ t2, t3).  Rows of 64 dims keep
// c ^ (t % 8).
template <int CPR>
__device__ __forceinline__ int kv_swz(int t) {
  if constexpr (CPR == 16)
    return ((t & 1) << 3) | ((((t >> 2) ^ (t >> 3)) & 1) << 2) | ((((t >> 1) ^ (t >> 2)) & 1) << 1) | ((t >> 3) & 1);
  else
    return t & (CPR - 1);
}

// Eight waves of 32 queries run two per SIMD inside one workgroup.  Four waves with
// 64-key tiles (NKV_PREFILL_NW=4, NKV_PREFILL_BK=64: 64 KB of LDS) let two workgroups
// share a CU, with independent barriers, prologues and epilogues; it measured ~6% slower
// on Qwen3-8B shapes, as each K/V tile then feeds half as many queries.
template <int D, int G, int NWAVES>
struct PfGeom {
  static constexpr int NW = NWAVES;             // waves per workgroup
  static constexpr int NT = NW * kWave;
  static constexpr int WQ = 32;                 // queries per wave: two 16-query MFMA blocks
  static constexpr int QSUB = NW / G;           // query sub-tiles per workgroup
  static constexpr int BQ = WQ * QSUB;          // queries per workgroup
  static constexpr int KS = D / 32;             // k-steps of S^T = K Q^T (32 dims each)
  static constexpr int DT = D / 16;             // 16-dim tiles of O^T
  static constexpr int CPR = D / 8;             // 16-byte chunks per K row
  static constexpr int K_BYTES = kBK * D * 2;   // one K (or V) tile
  static constexpr int STAGE = 2 * K_BYTES;     // K rows, then V rows, same layout
  static constexpr int CW = NW / 2;             // waves that issue the K/V copies (the first half)
  static constexpr int K_DMA = K_BYTES / 1024 / CW;   // copy instructions per copying wave per tile (K or V)
  static_assert(G >= 1 && G <= NW && NW % G == 0, "GQA group must divide the waves");
  static_assert(K_DMA >= 1 && K_BYTES % (1024 * CW) == 0, "K tile must split over the copying waves");
  // a q-tile's q (NW * WQ rows of D) fills one stage exactly: the next q-tile's q lands in
  // the stage the last tile leaves free, and each wave stages its output rows in its share
  static_assert(NW * WQ == 2 * kBK, "a q-tile's q must fill one stage");
  static constexpr int SMEM = kStages * STAGE;
};

template <int D, int G, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
prefill_bf16_kernel(const uint16_t* __restrict__ q, int64_t q_row,
                    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
                    int64_t k_stride, int64_t v_stride,
                    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                    const int32_t* __restrict__ block_table, int32_t max_blocks,
                    int32_t num_kv_heads, int32_t log2_bs, float scale_log2e, int32_t xcd_group,
                    uint16_t* __restrict__ out) {
  using Geo = PfGeom<D, G, NW>;
  constexpr int KS = Geo::KS, DT = Geo::DT, CPR = Geo::CPR, WQ = Geo::WQ;
  __shared__ __attribute__((aligned(16))) uint8_t smem[Geo::SMEM];
  __shared__ int32_t s_ids[3][kMaxIds];               // block ids of positions p, p+1, p+2

  // Workgroup L (launch order) runs on XCD L mod 8.  With xcd_group > 0 the (sequence x
  // KV head) slices of each XCD are taken xcd_group at a time, longest pairs first within
  // each group, so that fewer slices' K/V share the XCD's L2 at once; otherwise every
  // slice's longest pairs come first.  (The host sets it only when the grid's x extent is
  // a multiple of 8 * xcd_group.)
  int slice = blockIdx.x, level = blockIdx.y;
  if (xcd_group > 0) {
    const int L = blockIdx.y * gridDim.x + blockIdx.x;
    const int per_group = gridDim.y * xcd_group;
    const int m = L >> 3, grp = m / per_group, r = m - grp * per_group;
    level = r / xcd_group;
    slice = (L & 7) + 8 * (grp * xcd_group + (r - level * xcd_group));
  }
  const int b = slice / num_kv_heads;
  const int g = slice - b * num_kv_heads;
  const int qt = (gridDim.y - 1 - level) * (kPairQTiles ? 2 : 1);   // longest tiles first
  const int qstart = cu_q[b];
  const int lq = cu_q[b + 1] - qstart;
  const int lk = cu_k[b + 1] - cu_k[b];
  int q0 = qt * Geo::BQ;
  if (q0 >= lq) return;
  const int diag = lk - lq;                           // query i sees keys <= diag + i
  // A workgroup computes q-tile qt and then, if it exists, q-tile qt + 1 ("b").  Tile
  // buffer positions p = 0 .. nsteps-1 hold K/V tile p mod nb: q-tile qt takes positions
  // 0 .. na-1 (tiles 0 .. na-1), and b starts on position na-1 again, the last tile of qt,
  // still in LDS (b's keys include all of qt's), then takes na .. nsteps-1 (tiles na ..
  // nb-1, then 0 .. na-2).  b's q is copied into the free stage during qt's last tile.
  const bool has_b = kPairQTiles && q0 + Geo::BQ < lq;
  const int na = (diag + min(q0 + Geo::BQ, lq) + kBK - 1) / kBK;
  const int nb = has_b ? (diag + min(q0 + 2 * Geo::BQ, lq) + kBK - 1) / kBK : na;
  const int nsteps = has_b ? na + nb - 1 : na;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = g * G + wave % G;
  if (NKV_PREFILL_PRIO && NW == 8 && wave < 4) __builtin_amdgcn_s_setprio(3);   // waves 0-3 lead their SIMD partners
  const int hq = G * num_kv_heads;
  const int col = lane & 15;                          // MFMA column: query of a 16-block
  const int quad = lane >> 4;                         // MFMA lane quarter
  int wq0 = q0 + (wave / G) * WQ;                     // this wave's first query
  int wkend = wq0 < lq ? diag + min(wq0 + WQ, lq) : 0;   // keys this wave needs
  // paged: keys through the block table; otherwise rows kv0.. of contiguous k/v
  const bool paged = block_table != nullptr;
  const int64_t kv0 = paged ? 0 : cu_k[b];
  const int32_t* __restrict__ trow = paged ? block_table + int64_t(b) * max_blocks : nullptr;
  const int bs_mask = (1 << log2_bs) - 1;
  const int last_blk = (lk > 0 ? lk - 1 : 0) >> log2_bs;
  const int ids_per_tile = log2_bs >= kLog2BK ? 1 : (kBK >> log2_bs);
  const int64_t row_elems = int64_t(num_kv_heads) * D;   // pool row
  const uint16_t* kbase = k_cache + int64_t(g) * D;
  const uint16_t* vbase = v_cache + int64_t(g) * D;

  // ---- Q fragments (B operand of S^T = K Q^T): per 16-query block, 8 dims per lane ----
  bf16x8_t qf[2][KS];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int qi = wq0 + 16 * j + col;
    const bool ok = qi < lq;
    const uint16_t* qp = q + int64_t(qstart + (ok ? qi : 0)) * q_row + int64_t(h) * D + 8 * quad;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4_t v = ok ? *reinterpret_cast<const u32x4_t*>(qp + ks * 32) : u32x4_t{0, 0, 0, 0};
      qf[j][ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // ---- copies: block ids two tiles ahead (LDS), K and V rows by DMA ----
  // Position p holds tile p mod nb in stage p % kStages, its block ids in s_ids[p % 3].
  auto tile_at = [&](int p) __attribute__((always_inline)) { return p < nb ? p : p - nb; };
  auto issue_ids = [&](int p) __attribute__((always_inline)) {                       // wave 0: ids of position p -> s_ids[p % 3]
    if (paged && wave == 0 && lane < ids_per_tile) {
      const int blk = min(((tile_at(p) * kBK) >> log2_bs) + lane, last_blk);
      load_lds4(trow + blk, &s_ids[p % 3][0]);
    }
  };
  auto row_off = [&](int p, int key) __attribute__((always_inline)) -> int64_t {     // element offset of (key, head g)
    const int64_t phys = s_ids[p % 3][((key - tile_at(p) * kBK) >> log2_bs) & (kMaxIds - 1)];
    return ((phys << log2_bs) + (key & bs_mask)) * row_elems;
  };
  // The K/V copies of a tile are issued by waves 0..NW/2-1 only.  A wave waits at each copy
  // instruction until the CU takes it, slowly for a whole tile's worth: issued by all
  // waves at the top of a tile they held both waves of every SIMD (about 1500 cycles per
  // tile); issued by one wave of each SIMD pair (w, w + NW/2), the partner computes
  // meanwhile (8 prompts of 2048 tokens: the loop from 3.80 to 3.49 us per tile).
  const bool copier = wave < Geo::CW;
  const int cwave = wave % Geo::CW;
  // Copy j of a copying wave fills LDS slots (cwave * K_DMA + j) * 64 + lane: the lane's
  // row is r0 + j * RPI and its element the swizzled chunk of that row, which repeats
  // every NE copies (the swizzle sees the row mod 16, or mod 8 for 64-dim rows).
  constexpr int RPI = 64 / CPR;                        // rows per copy instruction
  constexpr int NE = CPR == 16 ? 16 / RPI : 1;         // distinct chunk swizzles over j
  static_assert(Geo::K_DMA % NE == 0, "copies per wave must cover whole swizzle periods");
  const int r0 = cwave * Geo::K_DMA * RPI + lane / CPR;
  auto k_row = [&](int j) __attribute__((always_inline)) { return r0 + j * RPI; };
  auto k_elem = [&](int j) __attribute__((always_inline)) { return ((lane % CPR) ^ kv_swz<CPR>(r0 + j * RPI)) * 8; };
  // With block_size >= kBK a tile lies inside one physical block: its base is uniform
  // (one LDS read, scalar math) and each lane adds only row * stride.  Contiguous K/V is
  // one such "block".
  const bool tile_in_block = !paged || log2_bs >= kLog2BK;
  auto tile_base = [&](int p, const uint16_t* base, int64_t stride) __attribute__((always_inline)) {
    const int t = tile_at(p);
    if (!paged) return base + (kv0 + int64_t(t) * kBK) * stride;
    const int phys = __builtin_amdgcn_readfirstlane(s_ids[p % 3][0]);
    return base + ((int64_t(phys) << log2_bs) + ((t * kBK) & bs_mask)) * stride;
  };
  // K and V rows of the tile at position p go HBM -> LDS directly, each into its half of
  // stage p % 2 (region 0: K, K_BYTES: V) in the same swizzled row layout.  Inside a tile
  // the rows are at most kBK - 1 strides from its base; with strides below 2^23 elements
  // the byte offsets fit 32 bits, so a copy of a full tile is a wave-uniform base (the
  // tile's, plus j * RPI rows) and a per-lane offset fixed for the whole kernel (one of
  // NE) instead of 64-bit lane arithmetic (8 prompts of 2048 tokens: 310 -> 304 us).
  const bool off32 = k_stride < (int64_t(1) << 23) && v_stride < (int64_t(1) << 23);
  uint32_t koff[NE], voff[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    koff[e] = uint32_t((r0 * k_stride + k_elem(e)) * 2);
    voff[e] = uint32_t((r0 * v_stride + k_elem(e)) * 2);
  }
  auto issue_rows_at = [&](int p, const uint16_t* tb, int64_t stride, int region) __attribute__((always_inline)) {   // tile inside one block
    uint8_t* sk = smem + (p % kStages) * Geo::STAGE + region;
    const int rmax = lk - 1 - tile_at(p) * kBK;      // rows past the keys repeat the last
    if (off32) {
      if (rmax >= kBK - 1) {
#pragma unroll
        for (int j = 0; j < Geo::K_DMA; ++j) {
          load_lds16_s(tb, region == 0 ? koff[j % NE] : voff[j % NE], sk + (cwave * Geo::K_DMA + j) * 1024);
          tb += RPI * stride;
          asm volatile("" : "+s"(tb));     // advanced copy by copy, not precomputed for all j
        }
      } else {
#pragma unroll
        for (int j = 0; j < Geo::K_DMA; ++j)
          load_lds16_s(tb, uint32_t((min(k_row(j), rmax) * stride + k_elem(j)) * 2),
                       sk + (cwave * Geo::K_DMA + j) * 1024);
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < Geo::K_DMA; ++j)
      load_lds16(tb + min(k_row(j), rmax) * stride + k_elem(j), sk + (cwave * Geo::K_DMA + j) * 1024);
  };
  auto issue_rows = [&](int p, const uint16_t* base, int64_t stride, int region) __attribute__((always_inline)) {
    if (!copier) return;
    if (tile_in_block) {
      issue_rows_at(p, tile_base(p, base, stride), stride, region);
    } else {
      uint8_t* sk = smem + (p % kStages) * Geo::STAGE + region;
      const int t = tile_at(p);
      const int rmax = lk - 1 - t * kBK;
#pragma unroll
      for (int j = 0; j < Geo::K_DMA; ++j) {
        const int key = t * kBK + min(k_row(j), rmax);
        load_lds16(base + row_off(p, key) + k_elem(j), sk + (cwave * Geo::K_DMA + j) * 1024);
      }
    }
  };
  // q of q-tile b into the stage at position p, in MFMA fragment order: fragment
  // f = (wave w, query block j, k-step ks) is 1 KB at f * 1024, lane L's 16 bytes being
  // dims 32 ks + 8 (L >> 4) .. of query 16 j + (L & 15) of wave w, so a wave later reads
  // each of its fragments with one conflict-free 16-byte LDS read per lane.  Every wave
  // copies its own fragments (the last tile has no K/V copies to issue, and split this
  // way no wave holds its SIMD partner up at the barrier) from a uniform base (the
  // q-tile's first row) and a per-lane byte offset (query block and k-step; the
  // instruction's own offset field would move the LDS destination too).  A partial
  // q-tile repeats its last query (never written out).  The offsets stay below 2^31 when
  // q_row * BQ < 2^30; otherwise each lane takes a 64-bit address.
  auto issue_q = [&](int p) __attribute__((always_inline)) {
    // the wave's fragments are one run of 2 * KS KB; the LDS address advances copy by
    // copy (opaque, so the compiler keeps one register, not one per copy)
    uint32_t la = lds_addr(smem + (p % kStages) * Geo::STAGE + wave * (2 * KS * 1024));
    const int qb0 = q0 + Geo::BQ;
    const uint16_t* qb = q + int64_t(qstart + qb0) * q_row + int64_t(g) * G * D;
    const bool off32 = q_row * Geo::BQ < (int64_t(1) << 30);
    int ln = lane;
    asm volatile("" : "+v"(ln));                    // as in the epilogue: no hoisted lane math
    const int col = ln & 15, quad = ln >> 4;
    auto next = [&]() __attribute__((always_inline)) {
      la += 1024;
      asm volatile("" : "+s"(la));
    };
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int qr = min((wave / G) * WQ + 16 * j + col, lq - 1 - qb0);   // row in the q-tile
      const int eo = (wave % G) * D + 8 * quad;                            // element in the row
      if (off32) {
        const uint32_t voff = uint32_t((qr * q_row + eo) * 2);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          load_lds16_s_at(qb, voff + 64 * ks, la);
          next();
        }
      } else {
        const uint16_t* lp = qb + int64_t(qr) * q_row + eo;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          load_lds16_at(lp + 32 * ks, la);
          next();
        }
      }
    }
  };

  f32x4_t o[2][DT];                                   // O^T per (query block, 16 dims)
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[j][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};
  const uint32_t ones = 0x3f803f80u;   // bf16 pair (1, 1)

  // Fragments of the 32-key half `kb` of the tile in stage `st`: K rows of its two
  // 16-key blocks (A operand of S^T = K Q^T) and V^T rows of its 16-dim tiles (A operand
  // of O^T += V^T P^T), read ahead of their MFMAs.
  // A lane's fragment rows are a multiple of 16 plus col (K) or v_row (V^T), so their
  // swizzle is fixed per lane.
  const int swz_k = kv_swz<CPR>(col);
  auto read_k = [&](const uint8_t* st, int kb, bf16x8_t (&kf)[2][KS]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int t = kb * 32 + 16 * i + col;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[i][ks] = *reinterpret_cast<const bf16x8_t*>(st + (t * CPR + ((4 * ks + quad) ^ swz_k)) * 16);
    }
  };
  // V^T fragments by the transposing LDS read: in each 16-lane quarter, lane col addresses
  // 4 dims (8 bytes) of key row 4*quad + (col >> 2) of a 16-key block, and the read hands
  // it dim col of the quarter's 4 rows.  Two reads (key blocks 0 and 1) make the 8 keys
  // 4*quad + r and 16 + 4*quad + r that the lane's P^T operand holds, in that order.
  const int v_row = 4 * quad + (col >> 2), v_dim = 4 * (col & 3);
  const int swz_v = kv_swz<CPR>(v_row);
  auto read_v = [&](const uint8_t* st, int kb, bf16x8_t (&vf)[DT]) __attribute__((always_inline)) {
    const uint8_t* sv = st + Geo::K_BYTES;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      s16x4_t h[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int t = kb * 32 + 16 * i + v_row, d = dt * 16 + v_dim;
        const uint8_t* a = sv + (t * CPR + ((d >> 3) ^ swz_v)) * 16 + (d & 7) * 2;
        h[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(a));
      }
      vf[dt] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto qk = [&](const bf16x8_t (&kf)[KS], int j, f32x4_t& s) __attribute__((always_inline)) {
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0], qf[j][0], f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
    for (int ks = 1; ks < KS; ++ks)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qf[j][ks], s, 0, 0, 0);
  };
  // Weights of one 16x16 block of S^T against max mq, as two bf16 pairs, and their sum.
  auto weights = [&](const f32x4_t& s, float cs, float mq, uint32_t& w0, uint32_t& w1) __attribute__((always_inline)) {
    w0 = pack_bf16x2(fast_exp2(fmaf(s[0], cs, -mq)), fast_exp2(fmaf(s[1], cs, -mq)));
    w1 = pack_bf16x2(fast_exp2(fmaf(s[2], cs, -mq)), fast_exp2(fmaf(s[3], cs, -mq)));
  };
  const bf16x8_t onesf = __builtin_bit_cast(bf16x8_t, u32x4_t{ones, ones, ones, ones});
  // Row sums of one query block's weights in a half: ones^T P^T puts the sum over the 32
  // keys of query col in every output element of that column, so each lane reads its own.
  auto rowsum = [&](const bf16x8_t& pf) __attribute__((always_inline)) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(onesf, pf, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0)[0];
  };
  // Softmax and P.V of one half.  s[i][j] is S^T of key block i and query block j; a
  // lane holds keys 16i + 4*quad + r of query 16j + col.  Masked halves are scaled
  // before the mask is applied (cs = 1 afterwards) so that a zero softmax_scale cannot
  // turn -inf into NaN; unmasked halves fold the scale into the exponent's FMA.  The
  // running max m is raised lazily and without a max pass in the common case: the
  // weights are taken against the current m, and only when some query's sum of its 32
  // rounded weights in the half exceeds kLazyBound (or is not finite: m = -inf
  // before the first half) does the wave raise m to the max of the half's scores of
  // that block (over the four lanes of each query), rescale O and l, and take the
  // weights again.  Every weight is at most that sum, so no weight kept exceeds
  // kLazyBound, the same headroom as testing the max itself.  The first half a q-tile
  // computes holds a key every one of its queries sees (key 0; for the second q-tile of a
  // pair, the first key of the first one's last tile, which lies before its first
  // query's diagonal), so m is finite from then on.  Block 0's weights are computed while
  // block 1's QK MFMAs run.
  bool fresh = true;                                  // the next half is a q-tile's first
  auto softmax_pv = [&](f32x4_t (&s)[2][2], int k0h, const bf16x8_t (&vf)[DT]) __attribute__((always_inline)) {
    const bool masked = (k0h + 31 > diag + wq0) || (k0h + 32 > lk);
    const float cs = masked ? 1.0f : scale_log2e;
    if (masked) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int qi = wq0 + 16 * j + col;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = k0h + 16 * i + 4 * quad + r;
            s[i][j][r] = (key < lk && key <= diag + qi) ? s[i][j][r] * scale_log2e : -INFINITY;
          }
        }
    }
    uint32_t w[2][2][2];
    float hs[2];
    bf16x8_t pf[2];
    if (fresh) {
      // first half of a q-tile: m = -inf and O = l = 0, so the max is taken at once
      // (a first pass of weights against -inf and a rescale of zeros would be thrown away)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float x = s[0][j][0];
#pragma unroll
        for (int r = 1; r < 4; ++r) x = fmaxf(x, s[0][j][r]);
#pragma unroll
        for (int r = 0; r < 4; ++r) x = fmaxf(x, s[1][j][r]);
        m[j] = xor32_max(xor16_max(x)) * cs;
        weights(s[0][j], cs, m[j], w[0][j][0], w[0][j][1]);
        weights(s[1][j], cs, m[j], w[1][j][0], w[1][j][1]);
        pf[j] = __builtin_bit_cast(bf16x8_t, u32x4_t{w[0][j][0], w[0][j][1], w[1][j][0], w[1][j][1]});
        lsum[j] = rowsum(pf[j]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          o[j][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pf[j], f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      }
      fresh = false;
      return;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) weights(s[0][j], cs, m[j], w[0][j][0], w[0][j][1]);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      weights(s[1][j], cs, m[j], w[1][j][0], w[1][j][1]);
      pf[j] = __builtin_bit_cast(bf16x8_t, u32x4_t{w[0][j][0], w[0][j][1], w[1][j][0], w[1][j][1]});
      hs[j] = rowsum(pf[j]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (__any(!(hs[j] <= kLazyBound))) {
        float x = s[0][j][0];
#pragma unroll
        for (int r = 1; r < 4; ++r) x = fmaxf(x, s[0][j][r]);
#pragma unroll
        for (int r = 0; r < 4; ++r) x = fmaxf(x, s[1][j][r]);
        const float mn = fmaxf(m[j], xor32_max(xor16_max(x)) * cs);
        const float alpha = fast_exp2(m[j] - mn);
        lsum[j] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[j][dt] *= alpha;
        m[j] = mn;
        weights(s[0][j], cs, mn, w[0][j][0], w[0][j][1]);
        weights(s[1][j], cs, mn, w[1][j][0], w[1][j][1]);
        pf[j] = __builtin_bit_cast(bf16x8_t, u32x4_t{w[0][j][0], w[0][j][1], w[1][j][0], w[1][j][1]});
        hs[j] = rowsum(pf[j]);
      }
      lsum[j] += hs[j];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        o[j][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pf[j], o[j][dt], 0, 0, 0);
    }
  };
  // One 32-key half: QK of key block 0 for both query blocks, then of key block 1 (the
  // softmax of block 0 can run beside those MFMAs), then softmax and P.V.
  auto half = [&](const uint8_t* st, int kb, int k0h) __attribute__((always_inline)) {
    bf16x8_t kf[2][KS], vf[DT];
    f32x4_t s[2][2];
    read_k(st, kb, kf);
    // all K fragment reads go out before the first MFMA, which then waits only for its
    // own (left to itself the compiler reads one fragment, waits, multiplies, and so on)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) qk(kf[i], j, s[i][j]);
    read_v(st, kb, vf);
    softmax_pv(s, k0h, vf);
  };

  // ---- epilogue: O^T / l -> bf16 rows staged in LDS, then contiguous row writes ----
  // The wave's 32 output rows go to `ost` (its own 64 * D bytes), 16-byte chunk c of row r
  // at c ^ (r mod CPR), and are read back a row per CPR lanes.  A wave reads back only the
  // rows it wrote, and LDS keeps one wave's accesses in order, so no barrier sits between.
  auto epilogue = [&](uint8_t* ost) __attribute__((always_inline)) {
    // lane-derived addresses are made here, not hoisted out of the tile loop (where this
    // also runs, between the two q-tiles) to sit in registers through every tile
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int col = ln & 15, quad = ln >> 4;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // every lane of a query holds its whole row sum (from the ones MFMA)
      const float inv = 1.0f / lsum[j];
      if (wq0 + 16 * j < lq) {
        const int r = 16 * j + col;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int c = 2 * dt + (quad >> 1);
          const u32x2_t w = {pack_bf16x2(o[j][dt][0] * inv, o[j][dt][1] * inv),
                             pack_bf16x2(o[j][dt][2] * inv, o[j][dt][3] * inv)};
          *reinterpret_cast<u32x2_t*>(ost + r * (D * 2) + (c ^ (r & (CPR - 1))) * 16 + (quad & 1) * 8) = w;
        }
      }
    }
    if (wq0 < lq) {
      constexpr int RPI = 64 / CPR;               // rows per 64-lane pass
      const int rr = ln / CPR, cc = ln % CPR;
#pragma unroll 1
      for (int i = 0; i < WQ / RPI; ++i) {
        const int row = i * RPI + rr;
        const int qi = wq0 + row;
        if (qi < lq) {
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ost + row * (D * 2) + (cc ^ (row & (CPR - 1))) * 16);
          // nontemporal: the output is not read again here, and cached it would evict K/V lines
          // that the other workgroups of the sequence still read from L2 (8 prompts of 2048
          // tokens: 275 -> 262 us)
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(out + (int64_t(qstart + qi) * hq + h) * D + cc * 8));
        }
      }
    }
  };

  // ---- prologue: tile 0 into stage 0, ids of positions 1..2 ----
  if (tile_in_block) {
    // tile 0's block id comes straight from the table (one scalar load), so its copies
    // go out beside the q loads instead of after a round trip through s_ids
    const uint16_t* k0b = kbase + kv0 * k_stride;
    const uint16_t* v0b = vbase + kv0 * v_stride;
    if (paged) {
      const int64_t phys0 = __builtin_amdgcn_readfirstlane(trow[0]);
      k0b = kbase + (phys0 << log2_bs) * k_stride;
      v0b = vbase + (phys0 << log2_bs) * v_stride;
    }
    if (copier) {
      issue_rows_at(0, k0b, k_stride, 0);
      issue_rows_at(0, v0b, v_stride, Geo::K_BYTES);
    }
    if (nsteps > 1) issue_ids(1);
    if (nsteps > 2) issue_ids(2);
  } else {
    issue_ids(0);
    if (nsteps > 1) issue_ids(1);
    wait_vmem_all();
    __syncthreads();
    issue_rows(0, kbase, k_stride, 0);
    issue_rows(0, vbase, v_stride, Geo::K_BYTES);
    if (nsteps > 2) issue_ids(2);
  }
  wait_vmem_all();
  __syncthreads();

  // One tile step at position p: the next position's copies (or, on qt's last tile, b's
  // q) go out first and fly during this tile's math; ids go two positions further ahead.
  auto step = [&](int p, bool a_last, bool b_first) __attribute__((always_inline)) {
    if (a_last) {
      if (has_b) issue_q(p + 1);
    } else if (p + 1 < nsteps) {
      issue_rows(p + 1, kbase, k_stride, 0);
      issue_rows(p + 1, vbase, v_stride, Geo::K_BYTES);
    }
    if (!b_first && p + 3 < nsteps) issue_ids(p + 3);
    const int k0 = tile_at(p) * kBK;
    const uint8_t* st = smem + (p % kStages) * Geo::STAGE;
#pragma unroll
    for (int kb = 0; kb < kBK / 32; ++kb)
      if (k0 + 32 * kb < wkend) half(st, kb, k0 + 32 * kb);
    wait_vmem_all();
    __syncthreads();
  };
  int p = 0;
  bool in_b = false;                                  // computing q-tile b
  for (;;) {
    const bool a_last = !in_b && p == na - 1;
    step(p, a_last, in_b && p == na - 1);
    if (a_last) {
      if (!has_b) break;
      // switch to q-tile b: its q fragments from the stage they landed in, then qt's
      // output staged in the same wave-owned bytes, then fresh running sums
      uint8_t* qw = smem + ((p + 1) % kStages) * Geo::STAGE + wave * (2 * KS * 1024);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          qf[j][ks] = *reinterpret_cast<const bf16x8_t*>(qw + (j * KS + ks) * 1024 + lane * 16);
      epilogue(qw);
      fresh = true;                                 // b's first half sets m, l and O
      q0 += Geo::BQ;
      wq0 += Geo::BQ;
      wkend = wq0 < lq ? diag + min(wq0 + WQ, lq) : 0;
      __syncthreads();                              // staging read back before the stage refills
      in_b = true;
      continue;                                     // b starts on qt's last tile
    }
    if (++p == nsteps) break;
  }

  // the barrier that closed the last tile has every wave done with the stages
  epilogue(smem + wave * (2 * KS * 1024));
}

// ---- fp32 VALU path --------------------------------------------------------------------

template <int D>
__global__ void __launch_bounds__(64)
prefill_f32_kernel(const float* __restrict__ q, int64_t q_row,
                   const float* __restrict__ k_cache, const float* __restrict__ v_cache,
                   int64_t k_stride, int64_t v_stride,
                   const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                   const int32_t* __restrict__ block_table, int32_t max_blocks,
                   int32_t num_q_heads, int32_t num_kv_heads, int32_t log2_bs,
                   float scale_log2e, float* __restrict__ out) {
  const int b = blockIdx.z;
  const int h = blockIdx.y;
  const int qstart = cu_q[b];
  const int lq = cu_q[b + 1] - qstart;
  const int lk = cu_k[b + 1] - cu_k[b];
  const int qi = blockIdx.x * 64 + threadIdx.x;
  if (qi >= lq) return;
  const int g = h / (num_q_heads / num_kv_heads);
  const int limit = lk - lq + qi;                     // last visible key
  const bool paged = block_table != nullptr;
  const int64_t kv0 = paged ? 0 : cu_k[b];
  const int32_t* trow = paged ? block_table + int64_t(b) * max_blocks : nullptr;
  const int bs_mask = (1 << log2_bs) - 1;

  float qv[D], acc[D];
  const float* qp = q + int64_t(qstart + qi) * q_row + int64_t(h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = qp[d];
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j <= limit; ++j) {
    const int64_t row = paged ? (int64_t(trow[j >> log2_bs]) << log2_bs) + (j & bs_mask) : kv0 + j;
    const float* kp = k_cache + row * k_stride + int64_t(g) * D;
    const float* vp = v_cache + row * v_stride + int64_t(g) * D;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = fmaf(qv[d], kp[d], s);
    s *= scale_log2e;
    const float mn = fmaxf(m, s);
    const float alpha = fast_exp2(m - mn);
    const float p = fast_exp2(s - mn);
    l = l * alpha + p;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vp[d], acc[d] * alpha);
    m = mn;
  }
  float* op = out + (int64_t(qstart + qi) * num_q_heads + h) * D;
  const float inv = 1.0f / l;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
}

// ---- host side -----------------------------------------------------------------------

template <int D, int G>
static hipError_t launch_bf16(const PrefillArgs& a, hipStream_t st) {
  // G must divide the waves: the eight-wave kernel serves groups wider than the default
  constexpr int NW = NKV_PREFILL_NW > G ? NKV_PREFILL_NW : G;
  using Geo = PfGeom<D, G, NW>;
  const PagedArgs& p = a.p;
  const int qtiles = (a.max_seqlen_q + Geo::BQ - 1) / Geo::BQ;
  const int groups = kPairQTiles ? (qtiles + 1) / 2 : qtiles;   // workgroups per (sequence, KV head)
  // XCD grouping: each XCD takes its slices in two halves, when a half still gives every CU
  // of the XCD a workgroup (8 prompts of 2048 tokens, 8 KV heads: 4 of an XCD's 8 slices
  // x 16 levels; 16 chunks of 512 tokens after a 1024-token prefix: 8 of 16 x 4 levels).
  // One slice at a time per group, or a quarter, was slower (the XCD's CUs then wait on
  // the last long pairs of a group); halves against one order over all slices, on two
  // boxes: 265.9-266.9 vs 271.5-273.3 us and 264.7-267.8 vs 267.9-271.4 us for the 2048-
  // token prompts, 161.6-163.0 vs 163.1-164.4 us and 162.3-164.4 vs 163.1-165.1 us for the
  // chunks.  NKV_PREFILL_XCD_GROUP in the environment (read at every call) sets the group
  // size, 0 for one order.
  const int slices = p.num_seqs * p.num_kv_heads;
  const int cus_per_xcd = (p.num_cus > 0 ? p.num_cus : 256) / 8;
  int xcd_group = slices % 16 == 0 ? slices / 16 : 0;
  if (xcd_group * groups < cus_per_xcd) xcd_group = 0;
  if (const char* e = getenv("NKV_PREFILL_XCD_GROUP")) xcd_group = atoi(e);
  if (xcd_group <= 0 || slices % (8 * xcd_group) != 0 || 8 * xcd_group >= slices) xcd_group = 0;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, G, NW>), dim3(p.num_seqs * p.num_kv_heads, groups),
                     dim3(Geo::NT), 0, st, static_cast<const uint16_t*>(a.q), a.q_row_elems,
                     static_cast<const uint16_t*>(p.k_cache), static_cast<const uint16_t*>(p.v_cache),
                     a.k_row_elems, a.v_row_elems, a.cu_seqlens_q, a.cu_seqlens_k, p.block_table, p.max_blocks_per_seq,
                     p.num_kv_heads, p.log2_block_size, p.scale_log2e, xcd_group,
                     static_cast<uint16_t*>(a.out));
  return hipGetLastError();
}

template <int D>
static hipError_t launch_f32(const PrefillArgs& a, hipStream_t st) {
  const PagedArgs& p = a.p;
  hipLaunchKernelGGL((prefill_f32_kernel<D>),
                     dim3((a.max_seqlen_q + 63) / 64, p.num_q_heads, p.num_seqs), dim3(64), 0, st,
                     static_cast<const float*>(a.q), a.q_row_elems,
                     static_cast<const float*>(p.k_cache), static_cast<const float*>(p.v_cache),
                     a.k_row_elems, a.v_row_elems, a.cu_seqlens_q, a.cu_seqlens_k, p.block_table, p.max_blocks_per_seq,
                     p.num_q_heads, p.num_kv_heads, p.log2_block_size, p.scale_log2e,
                     static_cast<float*>(a.out));
  return hipGetLastError();
}

template <int D>
static hipError_t dispatch_bf16(const PrefillArgs& a, hipStream_t st) {
  switch (a.p.num_q_heads / a.p.num_kv_heads) {
    case 1: return launch_bf16<D, 1>(a, st);
    case 2: return launch_bf16<D, 2>(a, st);
    case 4: return launch_bf16<D, 4>(a, st);
    case 8: return launch_bf16<D, 8>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  if (a.p.num_seqs == 0 || a.max_seqlen_q == 0) return hipSuccess;
  if (a.p.dtype == Dtype::BF16)
    return a.p.head_dim == 128 ? dispatch_bf16<128>(a, st) : dispatch_bf16<64>(a, st);
  return a.p.head_dim == 128 ? launch_f32<128>(a, st) : launch_f32<64>(a, st);
}

}  // namespace nkv
