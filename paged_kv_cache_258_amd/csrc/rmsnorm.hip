// Fused residual add + RMSNorm between decoder blocks (bf16).
//
// 「同一个 Qwen3，两种写法」 §3.6 (add_rms_forward): the hidden state and the residual are
// added in float32; that sum, cast to bf16, is the new residual; the float32 sum is
// normalised by the root of its mean square plus eps, cast to bf16 and multiplied by the
// weight (a bf16 product).  Without a residual (the first block) it is the plain RMSNorm
// of the hidden state, and the hidden state itself is the new residual.  Fused, a token's
// row is read once (hidden state and residual) and written once (output and new
// residual): 32 KiB per 4096-wide token instead of the 40 KiB of an add kernel followed by
// a norm kernel (the same section's count).
//
// Layout of the work: one 256-thread workgroup per token row, grid-stride over rows.  A
// thread owns the 16-byte chunks c, c + 256, ... of the row (CPT of them), issues every
// load of its chunks first, keeps the float32 sums in registers across the row's sum of
// squares (wave sums by DPP and lane swaps, then the 4 waves' partial sums through LDS,
// added in a fixed order so every thread gets the same bits), and writes only its own
// chunks after it has read them.  So the output may alias the hidden state and the new
// residual may alias the residual (the in-place use).  Rows are touched once, so their
// stores are nontemporal; their loads are plain (16384 x 4096 rows: 77 us, about 7 TB/s,
// against 91 us with nontemporal loads, and 98 us with neither hint).  The grid
// has a workgroup per row up to 64 per CU.  Float contraction is off so that
// products and sums round as float32 tensor arithmetic does; the mean is a correctly
// rounded division and the reciprocal root is v_rsq_f32 (within an ulp).
#include "common.hpp"
#include "launch.hpp"

namespace nkv {

constexpr int kNormThreads = 256;
constexpr int kNormWaves = kNormThreads / kWave;
#ifndef NKV_NORM_WGS_PER_CU
#define NKV_NORM_WGS_PER_CU 64
#endif
constexpr int kNormWgsPerCu = NKV_NORM_WGS_PER_CU;

__device__ __forceinline__ void unpack8f(const u32x4_t& w, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
}

__device__ __forceinline__ u32x4_t pack8f(const float (&x)[8]) {
  return u32x4_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                 pack_bf16x2(x[6], x[7])};
}

// x, residual, out and residual_out are not __restrict__: out may be x and residual_out
// may be residual.
template <int CPT>
__global__ void __launch_bounds__(kNormThreads)
add_rms_norm_kernel(const uint16_t* x, const uint16_t* residual,
                    const uint16_t* __restrict__ weight, float eps, int32_t num_tokens,
                    int32_t hidden, uint16_t* out, uint16_t* residual_out) {
#pragma clang fp contract(off)
  __shared__ float s_part[2][kNormWaves];
  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int chunks = hidden / 8;
  int par = 0;                        // alternating LDS slots: no second barrier per row
  for (int t = blockIdx.x; t < num_tokens; t += gridDim.x, par ^= 1) {
    const int64_t row = int64_t(t) * hidden;
    u32x4_t xa[CPT], ra[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {   // every load of the row first
      const int c = tid + k * kNormThreads;
      if (c < chunks) {
        xa[k] = *reinterpret_cast<const u32x4_t*>(x + row + 8 * c);
        if (residual)
          ra[k] = *reinterpret_cast<const u32x4_t*>(residual + row + 8 * c);
      }
    }
    float v[CPT][8];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int c = tid + k * kNormThreads;
      if (c < chunks) {
        unpack8f(xa[k], v[k]);
        if (residual) {
          float r[8];
          unpack8f(ra[k], r);
#pragma unroll
          for (int i = 0; i < 8; ++i) v[k][i] = v[k][i] + r[i];
          if (residual_out)
            __builtin_nontemporal_store(pack8f(v[k]), reinterpret_cast<u32x4_t*>(residual_out + row + 8 * c));
        } else if (residual_out) {
          __builtin_nontemporal_store(xa[k], reinterpret_cast<u32x4_t*>(residual_out + row + 8 * c));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += v[k][i] * v[k][i];
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[k][i] = 0.f;
      }
    }
    // the row's sum: within the wave (the same bits in every lane), then the waves in order
    ss = group8_sum(ss);
    ss += dpp<kDppRowRor8>(ss);
    ss = xor32_sum(xor16_sum(ss));
    if (lane == 0) s_part[par][wave] = ss;
    __syncthreads();
    float tot = s_part[par][0];
#pragma unroll
    for (int w = 1; w < kNormWaves; ++w) tot += s_part[par][w];
    const float rinv = __builtin_amdgcn_rsqf(tot / float(hidden) + eps);
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int c = tid + k * kNormThreads;
      if (c < chunks) {
        float wv[8];
        unpack8f(*reinterpret_cast<const u32x4_t*>(weight + 8 * c), wv);
        u32x4_t ow;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t n = pack_bf16x2(v[k][2 * i] * rinv, v[k][2 * i + 1] * rinv);   // cast
          ow[i] = pack_bf16x2(bf16_lo(n) * wv[2 * i], bf16_hi(n) * wv[2 * i + 1]);     // weight
        }
        __builtin_nontemporal_store(ow, reinterpret_cast<u32x4_t*>(out + row + 8 * c));
      }
    }
  }
}

hipError_t launch_add_rms_norm(const AddRmsNormArgs& a, hipStream_t st) {
  if (a.num_tokens == 0) return hipSuccess;
  int64_t blocks = a.num_tokens;
  const int64_t cap = int64_t(a.num_cus) * kNormWgsPerCu;   // beyond, workgroups walk more rows
  if (blocks > cap) blocks = cap;
  const auto* x = static_cast<const uint16_t*>(a.x);
  const auto* r = static_cast<const uint16_t*>(a.residual);
  const auto* w = static_cast<const uint16_t*>(a.weight);
  auto* o = static_cast<uint16_t*>(a.out);
  auto* ro = static_cast<uint16_t*>(a.residual_out);
  const int chunks_per_thread = (a.hidden / 8 + kNormThreads - 1) / kNormThreads;
  const dim3 g{unsigned(blocks)}, b{unsigned(kNormThreads)};
  switch (chunks_per_thread) {
    case 1: hipLaunchKernelGGL(add_rms_norm_kernel<1>, g, b, 0, st, x, r, w, a.eps, a.num_tokens, a.hidden, o, ro); break;
    case 2: hipLaunchKernelGGL(add_rms_norm_kernel<2>, g, b, 0, st, x, r, w, a.eps, a.num_tokens, a.hidden, o, ro); break;
    case 3:
    case 4: hipLaunchKernelGGL(add_rms_norm_kernel<4>, g, b, 0, st, x, r, w, a.eps, a.num_tokens, a.hidden, o, ro); break;
    case 5: case 6: case 7:
    case 8: hipLaunchKernelGGL(add_rms_norm_kernel<8>, g, b, 0, st, x, r, w, a.eps, a.num_tokens, a.hidden, o, ro); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nkv
