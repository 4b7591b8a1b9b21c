// Paged causal varlen prefill attention.
//
// Semantics: 「同一个 Qwen3，两种写法」 §3.2 (flat [T, H, D] batch cut by cu_seqlens,
// causal inside each segment, no work across segments), §3.3 (K/V read from the paged
// pool through the block table) and §3.4 (GQA handled inside the kernel);
// 「Nano-vLLM深度解读（下）」 §4 (flash_attn_varlen_func(..., causal=True,
// block_table=...)).  Query i of a segment with Lq queries and Lk keys sits at position
// Lk - Lq + i and sees keys j <= Lk - Lq + i.
//
// bf16 path (dense contraction -> MFMA, v_mfma_f32_32x32x16_bf16 on gfx950):
//   grid (seq * kv_head, q-tile) with q-tiles dispatched longest-first; one workgroup
//   holds the G query heads of one KV head for BQ queries: max(G,4) waves, each wave
//   32 queries of one head.  K/V tiles of 64 keys are gathered through the block table
//   into LDS once and used by all waves (every head of the GQA group and every query
//   sub-tile), K row-major, V transposed (dims x keys) so both MFMA operands are
//   16-byte LDS reads.  Scores are computed transposed, S^T = K Q^T, so each lane owns
//   one query: the row max needs one cross-half exchange and the row sum stays in the
//   lane until the end.  P goes from the S^T accumulator registers straight into the
//   B operand of O^T += V^T P^T (the key order inside each 16-key step is permuted the
//   same way on both operands, so no shuffle is needed).  The running max is raised
//   lazily (rescale only past 2^8 headroom).  Only tiles that cross the causal
//   diagonal or the end of the keys apply the mask.
// fp32 path: a plain VALU kernel (one lane per query and head, online softmax), used
//   for correctness-sized fp32 inputs.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace nkv {

constexpr int kBK = 64;                 // keys per tile
constexpr float kLazy = 8.0f;           // log2 headroom before rescaling
constexpr int kKPad = 8;                // bf16 elements of padding per K row in LDS
constexpr int kVPad = 8;                // bf16 elements of padding per Vt row in LDS

template <int D, int G>
struct PfGeom {
  static constexpr int NW = G > 4 ? G : 4;   // waves per workgroup
  static constexpr int NT = NW * kWave;
  static constexpr int QSUB = NW / G;        // 32-query sub-tiles per workgroup
  static constexpr int BQ = 32 * QSUB;       // queries per workgroup
  static constexpr int KS = D / 16;          // k-steps of the QK^T MFMA
  static constexpr int DT = D / 32;          // 32-dim tiles of O^T
  static constexpr int KROW = D + kKPad;     // LDS K row stride (elements)
  static constexpr int VROW = kBK + kVPad;   // LDS Vt row stride (elements)
  static constexpr int KCH = D / 8;          // 16-byte chunks per K row
  static constexpr int K_LOADS = kBK * KCH / NT;            // per thread
  static constexpr int V_QUADS = (kBK / 4) * KCH;          // (key quad, chunk) items
  static constexpr int V_LOADS = (V_QUADS + NT - 1) / NT;   // per thread
  static_assert(kBK * KCH % NT == 0, "K tile must split evenly over threads");
};

// Position of key k (0..63) of a tile inside the transposed V rows: within every
// 16-key step, bits 2 and 3 of the key index are swapped.  This matches the order in
// which the S^T accumulator of a 32x32 MFMA hands its keys to the PV step.
__device__ __forceinline__ int vt_quad_pos(int kq) {  // kq = key / 4
  return (kq & ~3) | ((kq & 1) << 1) | ((kq >> 1) & 1);
}

template <int D, int G>
__global__ void __launch_bounds__((G > 4 ? G : 4) * 64)
prefill_bf16_kernel(const uint16_t* __restrict__ q, int64_t q_row,
                    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
                    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                    const int32_t* __restrict__ block_table, int32_t max_blocks,
                    int32_t num_kv_heads, int32_t log2_bs, float scale_log2e,
                    uint16_t* __restrict__ out) {
  using Geo = PfGeom<D, G>;
  constexpr int NT = Geo::NT, KS = Geo::KS, DT = Geo::DT;
  constexpr int KROW = Geo::KROW, VROW = Geo::VROW, KCH = Geo::KCH;

  __shared__ __attribute__((aligned(16))) uint16_t s_k[kBK * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[D * VROW];

  const int pair = blockIdx.x;
  const int b = pair / num_kv_heads;
  const int g = pair - b * num_kv_heads;
  const int qt = gridDim.y - 1 - blockIdx.y;          // longest tiles first
  const int qstart = cu_q[b];
  const int lq = cu_q[b + 1] - qstart;
  const int lk = cu_k[b + 1] - cu_k[b];
  const int q0 = qt * Geo::BQ;
  if (q0 >= lq) return;
  const int diag = lk - lq;                           // query i sees keys <= diag + i

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = wave % G;
  const int qs = wave / G;
  const int h = g * G + hl;
  const int hq = G * num_kv_heads;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int wq0 = q0 + qs * 32;                       // this wave's first query
  const int qi = wq0 + l32;                           // this lane's query

  const int kend = diag + min(q0 + Geo::BQ, lq);      // keys the workgroup needs
  const int ntiles = (kend + kBK - 1) / kBK;
  const int wkend = wq0 < lq ? diag + min(wq0 + 32, lq) : 0;  // keys this wave needs
  const int32_t* __restrict__ trow = block_table + int64_t(b) * max_blocks;
  const int bs_mask = (1 << log2_bs) - 1;
  const int64_t row_elems = int64_t(num_kv_heads) * D;
  const uint16_t* kbase = k_cache + int64_t(g) * D;
  const uint16_t* vbase = v_cache + int64_t(g) * D;

  // ---- Q fragments (B operand of S^T = K Q^T): 8 dims per lane per k-step ----
  bf16x8_t qf[KS];
  {
    const bool ok = qi < lq && wq0 < lq;
    const uint16_t* qp = q + int64_t(qstart + qi) * q_row + int64_t(h) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t v = ok ? *reinterpret_cast<const u32x4_t*>(qp + ks * 16) : u32x4_t{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY;
  float l_part = 0.f;

  // ---- global -> register prefetch of one K/V tile ----
  u32x4_t kreg[Geo::K_LOADS];
  u32x4_t vreg[Geo::V_LOADS][4];

  auto key_off = [&](int key) -> int64_t {  // element offset of (key, head g) row
    const int64_t phys = trow[key >> log2_bs];
    return ((phys << log2_bs) + (key & bs_mask)) * row_elems;
  };

  auto prefetch = [&](int kt) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < Geo::K_LOADS; ++i) {
      const int idx = tid + i * NT;
      const int key = idx / KCH, c = idx % KCH;
      const int ka = k0 + key;
      kreg[i] = ka < lk ? *reinterpret_cast<const u32x4_t*>(kbase + key_off(ka) + c * 8)
                        : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < Geo::V_LOADS; ++i) {
      const int idx = tid + i * NT;
      const int kq = idx % 16, c = idx / 16;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ka = k0 + 4 * kq + j;
        vreg[i][j] = (idx < Geo::V_QUADS && ka < lk)
                         ? *reinterpret_cast<const u32x4_t*>(vbase + key_off(ka) + c * 8)
                         : u32x4_t{0, 0, 0, 0};
      }
    }
  };

  auto commit = [&]() {
#pragma unroll
    for (int i = 0; i < Geo::K_LOADS; ++i) {
      const int idx = tid + i * NT;
      const int key = idx / KCH, c = idx % KCH;
      *reinterpret_cast<u32x4_t*>(&s_k[key * KROW + c * 8]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < Geo::V_LOADS; ++i) {
      const int idx = tid + i * NT;
      if (idx >= Geo::V_QUADS) continue;
      const int kq = idx % 16, c = idx / 16;
      const int pos = 4 * vt_quad_pos(kq);
      // 4 keys x 8 dims -> for each dim, its 4 keys as two packed bf16 pairs
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t a0 = vreg[i][0][w], a1 = vreg[i][1][w];
        const uint32_t a2 = vreg[i][2][w], a3 = vreg[i][3][w];
        const u32x2_t lo = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
        const u32x2_t hi = {(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
        *reinterpret_cast<u32x2_t*>(&s_vt[(c * 8 + 2 * w) * VROW + pos]) = lo;
        *reinterpret_cast<u32x2_t*>(&s_vt[(c * 8 + 2 * w + 1) * VROW + pos]) = hi;
      }
    }
  };

  prefetch(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();                                   // previous tile fully consumed
    commit();
    __syncthreads();
    if (kt + 1 < ntiles) prefetch(kt + 1);
    const int k0 = kt * kBK;
    if (k0 >= wkend) continue;                         // this wave is past its keys

    // ---- S^T = K Q^T for the two 32-key halves of the tile ----
    f32x16_t s[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[t2][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            &s_k[(t2 * 32 + l32) * KROW + ks * 16 + 8 * hh]);
        s[t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[t2], 0, 0, 0);
      }
    }

    // ---- scale, mask (diagonal / tail tiles only), running max ----
    const bool masked = (k0 + kBK - 1 > diag + wq0) || (k0 + kBK > lk);
    float mloc = -INFINITY;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[t2][r] * scale_log2e;
        if (masked) {
          const int key = k0 + t2 * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          x = (key < lk && key <= diag + qi) ? x : -INFINITY;
        }
        s[t2][r] = x;
        mloc = fmaxf(mloc, x);
      }
    mloc = fmaxf(mloc, shfl_xor(mloc, 32));
    if (__any(mloc > m_run + kLazy)) {
      const float mn = fmaxf(m_run, mloc);
      const float alpha = fast_exp2(m_run - mn);
      l_part *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      m_run = mn;
    }

    // ---- P = exp2(S - m), packed to bf16 in PV k-step order ----
    bf16x8_t pf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int mm = 0; mm < 8; ++mm) {
        const float p = fast_exp2(s[kk >> 1][8 * (kk & 1) + mm] - m_run);
        l_part += p;
        pf[kk][mm] = (__bf16)p;
      }
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            &s_vt[(dt * 32 + l32) * VROW + kk * 16 + 8 * hh]);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kk], o[dt], 0, 0, 0);
      }
  }

  // ---- epilogue: O / l -> bf16 ----
  const float l_tot = l_part + shfl_xor(l_part, 32);
  if (qi < lq && wq0 < lq) {
    const float inv = 1.0f / l_tot;
    uint16_t* op = out + (int64_t(qstart + qi) * hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = dt * 32 + 8 * r4 + 4 * hh;
        const u32x2_t w = {pack_bf16x2(o[dt][4 * r4 + 0] * inv, o[dt][4 * r4 + 1] * inv),
                           pack_bf16x2(o[dt][4 * r4 + 2] * inv, o[dt][4 * r4 + 3] * inv)};
        *reinterpret_cast<u32x2_t*>(op + d0) = w;
      }
  }
}

// ---- fp32 VALU path --------------------------------------------------------------------

template <int D>
__global__ void __launch_bounds__(64)
prefill_f32_kernel(const float* __restrict__ q, int64_t q_row,
                   const float* __restrict__ k_cache, const float* __restrict__ v_cache,
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
  const int32_t* trow = block_table + int64_t(b) * max_blocks;
  const int bs_mask = (1 << log2_bs) - 1;
  const int64_t row_elems = int64_t(num_kv_heads) * D;

  float qv[D], acc[D];
  const float* qp = q + int64_t(qstart + qi) * q_row + int64_t(h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = qp[d];
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j <= limit; ++j) {
    const int64_t off = ((int64_t(trow[j >> log2_bs]) << log2_bs) + (j & bs_mask)) * row_elems +
                        int64_t(g) * D;
    const float* kp = k_cache + off;
    const float* vp = v_cache + off;
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
  using Geo = PfGeom<D, G>;
  const PagedArgs& p = a.p;
  const int qtiles = (a.max_seqlen_q + Geo::BQ - 1) / Geo::BQ;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, G>), dim3(p.num_seqs * p.num_kv_heads, qtiles),
                     dim3(Geo::NT), 0, st, static_cast<const uint16_t*>(a.q), a.q_row_elems,
                     static_cast<const uint16_t*>(p.k_cache), static_cast<const uint16_t*>(p.v_cache),
                     a.cu_seqlens_q, a.cu_seqlens_k, p.block_table, p.max_blocks_per_seq,
                     p.num_kv_heads, p.log2_block_size, p.scale_log2e,
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
                     a.cu_seqlens_q, a.cu_seqlens_k, p.block_table, p.max_blocks_per_seq,
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
