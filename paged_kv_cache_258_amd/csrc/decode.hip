// Paged single-token decode attention, split over long contexts.
//
// Semantics: 「Nano-vLLM深度解读（下）」 §4 and 「同一个 Qwen3，两种写法」 §3.4
// (flash_attn_with_kvcache with cache_seqlens and block_table): the single query of
// sequence b attends to its context_lens[b] cached positions, read through its block
// table; Q head h uses KV head h / G (G = Hq/Hkv, the repeat_kv grouping).
//
// Work decomposition (MI355X):
//   grid (split, kv_head, seq); 256 threads = 4 waves per workgroup.  A split is
//   `split_tokens` consecutive logical positions; splits past a sequence's length exit
//   at once.  Inside a wave, 8 lanes own one cache row of one KV head (head_dim
//   elements, 256 B for bf16/128), each lane two 16-byte vectors, so one load
//   instruction covers eight rows with contiguous 128-byte runs.  Each group of 8 lanes
//   takes 2 positions per round (16 per wave, 64 per workgroup) and the block-table
//   entry of a round is one scalar load (a round never crosses a block).
//   All G query heads of the group are kept in registers, so every K/V byte read from
//   HBM serves the G heads that share it.
//   q.k partial dot products use v_dot2_f32_bf16 and are summed over the 8 lanes with
//   DPP (quad_perm, row_half_mirror).  The softmax is online with one running max per
//   wave and head, raised lazily: the accumulators are rescaled only when a new score
//   exceeds the running max by more than 2^8, which keeps every weight <= 256.
//   At the end the 8 groups and 4 waves are merged in LDS; a sequence with one split
//   writes `out` directly, otherwise (max, sum, weighted values) go to the workspace
//   and decode_reduce_kernel merges the splits with log-sum-exp weights.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace nkv {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = 4;
constexpr int kTokPerGroup = 2;                       // positions per 8-lane group per round
constexpr int kTokPerWave = 8 * kTokPerGroup;         // 16
constexpr int kTokPerRound = kDecWaves * kTokPerWave; // 64
constexpr float kLazyRescale = 8.0f;                  // log2 headroom before rescaling

template <class S, int D>
struct DecGeom {
  static constexpr int EPV = 16 / S::bytes;  // elements per 16-byte vector
  static constexpr int NV = D / (8 * EPV);   // vectors per lane per row
  static constexpr int DPL = NV * EPV;       // dims per lane
  static_assert(NV >= 1, "head_dim too small");
  // element offset (inside a row) of vector v of lane u
  __device__ static constexpr int vec_off(int v, int u) { return (v * 8 + u) * EPV; }
};

template <class S>
__device__ __forceinline__ float elem_at(const u32x4_t& x, int e) {
  if constexpr (S::bytes == 2) {
    const uint32_t w = x[e >> 1];
    return (e & 1) ? bf16_hi(w) : bf16_lo(w);
  } else {
    return __uint_as_float(x[e]);
  }
}

template <class S>
__device__ __forceinline__ void store_elem(typename S::elem* p, float x) {
  if constexpr (S::bytes == 2) {
    *p = __builtin_bit_cast(uint16_t, (__bf16)x);  // round to nearest even
  } else {
    *p = x;
  }
}

template <class S, int D, int G>
__global__ void __launch_bounds__(kDecThreads)
decode_split_kernel(const typename S::elem* __restrict__ q,
                    const typename S::elem* __restrict__ k_cache,
                    const typename S::elem* __restrict__ v_cache,
                    const int32_t* __restrict__ context_lens,
                    const int32_t* __restrict__ block_table, int32_t max_blocks,
                    int32_t num_kv_heads, int32_t log2_bs, float scale_log2e,
                    int32_t split_tokens, int32_t max_splits,
                    typename S::elem* __restrict__ out,
                    float* __restrict__ ws_ml, float* __restrict__ ws_acc) {
  using Geo = DecGeom<S, D>;
  constexpr int NV = Geo::NV, EPV = Geo::EPV, DPL = Geo::DPL;
  constexpr int HC = G < 4 ? G : 4;  // heads merged per LDS pass

  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int ctx = context_lens[b];
  const int begin = split * split_tokens;
  if (begin >= ctx) return;
  const int end = min(ctx, begin + split_tokens);
  const int nsplit = (ctx + split_tokens - 1) / split_tokens;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 3;
  const int u = lane & 7;
  const int hq = G * num_kv_heads;
  const int32_t* __restrict__ trow = block_table + int64_t(b) * max_blocks;
  const int bs_mask = (1 << log2_bs) - 1;
  const int64_t row_elems = int64_t(num_kv_heads) * D;
  const typename S::elem* kbase = k_cache + int64_t(g) * D;
  const typename S::elem* vbase = v_cache + int64_t(g) * D;

  // ---- the G query vectors, this lane's dims ----
  u32x4_t qv[G][NV];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int v = 0; v < NV; ++v)
      qv[h][v] = *reinterpret_cast<const u32x4_t*>(
          q + (int64_t(b) * hq + g * G + h) * D + Geo::vec_off(v, u));

  float m[G], l[G], acc[G][DPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int d = 0; d < DPL; ++d) acc[h][d] = 0.f;
  }

  auto load_round = [&](int base, u32x4_t (&kr)[kTokPerGroup][NV],
                        u32x4_t (&vr)[kTokPerGroup][NV]) {
    const int64_t phys = trow[base >> log2_bs];  // one block per round (base % 16 == 0)
#pragma unroll
    for (int i = 0; i < kTokPerGroup; ++i) {
      const int t = base + grp * kTokPerGroup + i;
      if (t < end) {
        const int64_t off = ((phys << log2_bs) + (t & bs_mask)) * row_elems;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          kr[i][v] = *reinterpret_cast<const u32x4_t*>(kbase + off + Geo::vec_off(v, u));
          vr[i][v] = *reinterpret_cast<const u32x4_t*>(vbase + off + Geo::vec_off(v, u));
        }
      } else {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          kr[i][v] = u32x4_t{0, 0, 0, 0};
          vr[i][v] = u32x4_t{0, 0, 0, 0};
        }
      }
    }
  };

  auto compute_round = [&](int base, const u32x4_t (&kr)[kTokPerGroup][NV],
                           const u32x4_t (&vr)[kTokPerGroup][NV]) {
    float sc[kTokPerGroup][G];
#pragma unroll
    for (int i = 0; i < kTokPerGroup; ++i) {
      const bool valid = base + grp * kTokPerGroup + i < end;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float dot = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            if constexpr (S::bytes == 2)
              dot = dot2_bf16(kr[i][v][w], qv[h][v][w], dot);
            else
              dot = fmaf(__uint_as_float(kr[i][v][w]), __uint_as_float(qv[h][v][w]), dot);
          }
        dot = group8_sum(dot) * scale_log2e;
        sc[i][h] = valid ? dot : -INFINITY;
      }
    }
    // lazy running max: rescale only when some score clears the headroom
    bool need = false;
    float mx[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mx[h] = sc[0][h];
#pragma unroll
      for (int i = 1; i < kTokPerGroup; ++i) mx[h] = fmaxf(mx[h], sc[i][h]);
      need |= mx[h] > m[h] + kLazyRescale;
    }
    if (__any(need)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float wm = mx[h];
        wm = fmaxf(wm, shfl_xor(wm, 8));
        wm = fmaxf(wm, shfl_xor(wm, 16));
        wm = fmaxf(wm, shfl_xor(wm, 32));
        const float mn = fmaxf(m[h], wm);
        const float alpha = fast_exp2(m[h] - mn);  // 0 on the first valid round
        l[h] *= alpha;
#pragma unroll
        for (int d = 0; d < DPL; ++d) acc[h][d] *= alpha;
        m[h] = mn;
      }
    }
#pragma unroll
    for (int i = 0; i < kTokPerGroup; ++i) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = fast_exp2(sc[i][h] - m[h]);
        l[h] += p;
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
          for (int e = 0; e < EPV; ++e)
            acc[h][v * EPV + e] = fmaf(p, elem_at<S>(vr[i][v], e), acc[h][v * EPV + e]);
      }
    }
  };

  // ---- main loop: rounds of 64 positions, next round's loads in flight ----
  u32x4_t ka[kTokPerGroup][NV], va[kTokPerGroup][NV];
  u32x4_t kb[kTokPerGroup][NV], vb[kTokPerGroup][NV];
  int base = begin + wave * kTokPerWave;
  if (base < end) load_round(base, ka, va);
  while (base < end) {
    if (base + kTokPerRound < end) load_round(base + kTokPerRound, kb, vb);
    compute_round(base, ka, va);
    base += kTokPerRound;
    if (base >= end) break;
    if (base + kTokPerRound < end) load_round(base + kTokPerRound, ka, va);
    compute_round(base, kb, vb);
    base += kTokPerRound;
  }

  // ---- merge: group pairs by DPP (they share m), then 16 partials in LDS ----
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] += dpp<kDppRowRor8>(l[h]);
#pragma unroll
    for (int d = 0; d < DPL; ++d) acc[h][d] += dpp<kDppRowRor8>(acc[h][d]);
  }
  constexpr int NP = kDecWaves * 4;  // partials per workgroup
  __shared__ float s_acc[NP][HC][D];
  __shared__ float s_l[NP][G];
  __shared__ float s_m[kDecWaves][G];
  const int part = wave * 4 + (grp >> 1);
  const bool writer = (grp & 1) == 0;
  if (lane == 0)
#pragma unroll
    for (int h = 0; h < G; ++h) s_m[wave][h] = m[h];
  if (writer && u == 0)
#pragma unroll
    for (int h = 0; h < G; ++h) s_l[part][h] = l[h];

  const int64_t out_row0 = int64_t(b) * hq + g * G;  // row of head g*G in [B*Hq]
#pragma unroll
  for (int hc = 0; hc < G; hc += HC) {
    if (writer)
#pragma unroll
      for (int hl = 0; hl < HC; ++hl)
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
          for (int e = 0; e < EPV; ++e)
            s_acc[part][hl][Geo::vec_off(v, u) + e] = acc[hc + hl][v * EPV + e];
    __syncthreads();
    for (int o = threadIdx.x; o < HC * D; o += kDecThreads) {
      const int hl = o / D;
      const int d = o % D;
      const int h = hc + hl;
      float M = s_m[0][h];
#pragma unroll
      for (int w = 1; w < kDecWaves; ++w) M = fmaxf(M, s_m[w][h]);
      float wt[kDecWaves];
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) wt[w] = fast_exp2(s_m[w][h] - M);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        num = fmaf(wt[p / 4], s_acc[p][hl][d], num);
        den = fmaf(wt[p / 4], s_l[p][h], den);
      }
      const int64_t row = out_row0 + h;
      if (nsplit == 1) {
        store_elem<S>(out + row * D + d, num / den);
      } else {
        const int64_t slot = row * max_splits + split;
        ws_acc[slot * D + d] = num;
        if (d == 0) {
          ws_ml[slot * 2 + 0] = M;
          ws_ml[slot * 2 + 1] = den;
        }
      }
    }
    __syncthreads();
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

DecodePlan plan_decode(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                       int num_cus) {
  DecodePlan p{};
  const int64_t max_tokens = int64_t(max_blocks_per_seq) * block_size;
  const int64_t pairs = int64_t(num_seqs) * num_kv_heads;
  // Largest split (fewest partials) that still gives ~4 workgroups per CU when every
  // sequence is at its maximum length; never more than 4096 positions per workgroup so
  // one long sequence cannot become the critical path.
  int32_t split = 256;
  const char* env = getenv("NKV_DECODE_SPLIT_TOKENS");
  if (env && atoi(env) >= kTokPerRound && atoi(env) % kTokPerRound == 0) {
    split = atoi(env);
  } else {
    for (int32_t cand = 4096; cand >= 256; cand /= 2) {
      const int64_t wgs = pairs * ((max_tokens + cand - 1) / cand);
      if (wgs >= int64_t(4) * num_cus) {
        split = cand;
        break;
      }
    }
  }
  p.split_tokens = split;
  p.max_splits = int32_t((max_tokens + split - 1) / split);
  if (p.max_splits < 1) p.max_splits = 1;
  p.workspace_bytes = p.max_splits <= 1
                          ? 0
                          : size_t(num_seqs) * num_q_heads * p.max_splits * (head_dim + 2) *
                                sizeof(float);
  return p;
}

template <class S, int D, int G>
static hipError_t launch_decode_t(const DecodeArgs& a, const DecodePlan& plan, hipStream_t st) {
  using E = typename S::elem;
  const PagedArgs& p = a.p;
  float* ws_ml = static_cast<float*>(a.workspace);
  float* ws_acc = ws_ml ? ws_ml + size_t(p.num_seqs) * p.num_q_heads * plan.max_splits * 2
                        : nullptr;
  hipLaunchKernelGGL((decode_split_kernel<S, D, G>),
                     dim3(plan.max_splits, p.num_kv_heads, p.num_seqs), dim3(kDecThreads), 0, st,
                     static_cast<const E*>(a.q), static_cast<const E*>(p.k_cache),
                     static_cast<const E*>(p.v_cache), a.context_lens, p.block_table,
                     p.max_blocks_per_seq, p.num_kv_heads, p.log2_block_size, p.scale_log2e,
                     plan.split_tokens, plan.max_splits, static_cast<E*>(a.out), ws_ml, ws_acc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.max_splits <= 1) return e;
  hipLaunchKernelGGL((decode_reduce_kernel<S, D>), dim3(p.num_q_heads, p.num_seqs), dim3(64), 0,
                     st, a.context_lens, plan.split_tokens, plan.max_splits, p.num_q_heads,
                     ws_ml, ws_acc, static_cast<E*>(a.out));
  return hipGetLastError();
}

template <class S, int D>
static hipError_t dispatch_g(const DecodeArgs& a, const DecodePlan& plan, hipStream_t st) {
  switch (a.p.num_q_heads / a.p.num_kv_heads) {
    case 1: return launch_decode_t<S, D, 1>(a, plan, st);
    case 2: return launch_decode_t<S, D, 2>(a, plan, st);
    case 4: return launch_decode_t<S, D, 4>(a, plan, st);
    case 8: return launch_decode_t<S, D, 8>(a, plan, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan, hipStream_t st) {
  const bool bf = a.p.dtype == Dtype::BF16;
  if (a.p.head_dim == 128) return bf ? dispatch_g<BF16, 128>(a, plan, st) : dispatch_g<F32, 128>(a, plan, st);
  if (a.p.head_dim == 64) return bf ? dispatch_g<BF16, 64>(a, plan, st) : dispatch_g<F32, 64>(a, plan, st);
  return hipErrorInvalidValue;
}

}  // namespace nkv
