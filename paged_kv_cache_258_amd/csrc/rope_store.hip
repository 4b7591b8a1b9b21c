// The step right before the KV store of a Qwen3 attention layer, fused into one pass:
// per-head RMSNorm of q and k, rotary embedding by position, the store of the rotated k
// and of v through slot_mapping, and the rotated q written out for attention.
//
// 「Nano-vLLM深度解读（下）」 §2 (Qwen3Attention.forward: split of the fused projection,
// q_norm / k_norm over head_dim, rotary_emb(positions, q, k), then attention, which
// stores k and v first, §4); 「同一个 Qwen3，两种写法」 §3.5 (the cos/sin table looked
// up by position, the rotation of the two halves in float32) and §3.6 (RMSNorm in float32
// with the cast back to the input dtype before the weight product).
//
// Without fusion, q and k make three round trips through HBM (norm, rope, store); here
// the projection output is read once with plain loads and each result written once with
// the nontemporal hint (16384 tokens of Qwen3-8B heads: 69 us; 77 us with nontemporal
// loads too, 84 us with neither hint).
//
// Layout of the work: one wave per token (grid-stride over tokens), so the position, the
// slot, the cos/sin row and the norm weights are read once per token and every head's
// loads go out together.  A head of D dims is handled by D/8 lanes, lane j holding the
// 8 consecutive dims [8j, 8j+8) as one 16-byte access.  The rotation pairs dim i with
// dim i + D/2, which the lane D/16 positions away holds: after normalising, each lane
// swaps its four packed bf16 words with that partner (a DPP row rotation by 8 for D = 128)
// and computes the half of the rotation that lands in its own dims.  A head's mean
// square is a sum over its D/8 lanes, in an order that gives every lane the same bits.
// The 64/(D/8) lane groups of a wave take head slots g, g + 64/(D/8), ... (q heads, then
// k, then v, as the projection lays them out), up to 64 slots per pass.  Float
// contraction is off so that the rotation rounds its two products and their sum
// separately, as the listing's float32 tensor arithmetic does; the reciprocal root is
// the hardware's v_rsq_f32 (within an ulp, like the listing's rsqrt).
#include "common.hpp"
#include "launch.hpp"

namespace nkv {

#ifndef NKV_ROPE_WGS_PER_CU
#define NKV_ROPE_WGS_PER_CU 16
#endif
constexpr int kRopeThreads = 256;
constexpr int kRopeWaves = kRopeThreads / kWave;

// the bf16 values of a packed pair, as floats
__device__ __forceinline__ void unpack8(const u32x4_t& w, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
}

// the partner's word: lane j of a D/8-lane head group <- lane j ^ (D/16)
template <int LPH>
__device__ __forceinline__ uint32_t partner(uint32_t v) {
  if constexpr (LPH == 16)
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), kDppRowRor8, 0xf, 0xf, true));
  else
    return uint32_t(__shfl_xor(int(v), LPH / 2));
}

template <int D>
__global__ void __launch_bounds__(kRopeThreads)
qk_norm_rope_store_kernel(const uint16_t* __restrict__ qkv, int64_t qkv_row,
                          const int32_t* __restrict__ positions,
                          const uint16_t* __restrict__ q_weight, const uint16_t* __restrict__ k_weight,
                          const float* __restrict__ cos_sin, float eps,
                          const int32_t* __restrict__ slot_mapping, int32_t num_tokens,
                          int32_t num_q_heads, int32_t num_kv_heads,
                          uint16_t* __restrict__ q_out, uint16_t* __restrict__ k_cache,
                          uint16_t* __restrict__ v_cache) {
#pragma clang fp contract(off)
  constexpr int LPH = D / 8;             // lanes per head
  constexpr int GL = kWave / LPH;        // heads side by side in a wave
  constexpr int KR = kWave / GL;         // head rows per pass: GL * KR = 64 slots
  constexpr int H2 = D / 2;
  static_assert(LPH == 8 || LPH == 16, "head_dim 64 or 128");
  const int lane = threadIdx.x % kWave;
  const int j = lane % LPH;
  const int g = lane / LPH;
  const bool second = j >= LPH / 2;      // this lane's dims are in the second half
  const int fi = 8 * j - (second ? H2 : 0);   // frequency index of its first dim
  const int nslots = num_q_heads + 2 * num_kv_heads;
  const int first_v = num_q_heads + num_kv_heads;
  const int64_t row_kv = int64_t(num_kv_heads) * D;   // pool row, elements
  float wq[8], wk[8];                    // the norm weights of this lane's dims
  unpack8(*reinterpret_cast<const u32x4_t*>(q_weight + 8 * j), wq);
  unpack8(*reinterpret_cast<const u32x4_t*>(k_weight + 8 * j), wk);

  for (int t = blockIdx.x * kRopeWaves + threadIdx.x / kWave; t < num_tokens;
       t += gridDim.x * kRopeWaves) {
    const int pos = __builtin_amdgcn_readfirstlane(positions[t]);
    const int32_t slot = __builtin_amdgcn_readfirstlane(slot_mapping[t]);
    const float* row = cos_sin + int64_t(pos) * D;
    const f32x4_t c0 = *reinterpret_cast<const f32x4_t*>(row + fi);
    const f32x4_t c1 = *reinterpret_cast<const f32x4_t*>(row + fi + 4);
    const f32x4_t s0 = *reinterpret_cast<const f32x4_t*>(row + H2 + fi);
    const f32x4_t s1 = *reinterpret_cast<const f32x4_t*>(row + H2 + fi + 4);
    const float c[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
    // the sine with the sign of this lane's half: o = y c + y' sn (negation is exact)
    float sn[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
    for (int i = 0; i < 8; ++i) sn[i] = second ? sn[i] : -sn[i];
    const uint16_t* src = qkv + int64_t(t) * qkv_row;
    for (int sb = 0; sb < nslots; sb += GL * KR) {
      u32x4_t a[KR];
#pragma unroll
      for (int k = 0; k < KR; ++k) {                      // every load of the pass first
        const int s = sb + k * GL + g;
        a[k] = s < nslots ? *reinterpret_cast<const u32x4_t*>(src + int64_t(s) * D + 8 * j)
                          : u32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int k = 0; k < KR; ++k) {
        const int s = sb + k * GL + g;
        if (sb + k * GL >= nslots) break;                 // no group of this row has a slot
        if (s >= first_v) {                               // v: stored as it is
          if (s < nslots && slot >= 0)
            __builtin_nontemporal_store(a[k], reinterpret_cast<u32x4_t*>(v_cache + int64_t(slot) * row_kv +
                                        int64_t(s - first_v) * D + 8 * j));
          continue;
        }
        // q or k head: mean square, norm, cast, weight, cast; swap with the partner;
        // this lane's half of the rotation, cast
        const bool is_q = s < num_q_heads;
        float x[8];
        unpack8(a[k], x);
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
        ss = group8_sum(ss);
        if constexpr (LPH == 16) ss += dpp<kDppRowRor8>(ss);
        const float r = __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
        u32x4_t yw;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float n0 = bf16_lo(pack_bf16x2(x[2 * i] * r, x[2 * i + 1] * r));
          const float n1 = bf16_hi(pack_bf16x2(x[2 * i] * r, x[2 * i + 1] * r));
          yw[i] = pack_bf16x2(n0 * (is_q ? wq[2 * i] : wk[2 * i]),
                              n1 * (is_q ? wq[2 * i + 1] : wk[2 * i + 1]));
        }
        u32x4_t pw;
#pragma unroll
        for (int i = 0; i < 4; ++i) pw[i] = partner<LPH>(yw[i]);
        float y[8], yp[8], o[8];
        unpack8(yw, y);
        unpack8(pw, yp);
#pragma unroll
        for (int i = 0; i < 8; ++i)   // first half: y1 c - y2 s; second half: y2 c + y1 s
          o[i] = y[i] * c[i] + yp[i] * sn[i];
        const u32x4_t ow = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                            pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
        uint16_t* dst = nullptr;
        if (is_q)
          dst = q_out + (int64_t(t) * num_q_heads + s) * D;
        else if (slot >= 0)
          dst = k_cache + int64_t(slot) * row_kv + int64_t(s - num_q_heads) * D;
        if (dst) __builtin_nontemporal_store(ow, reinterpret_cast<u32x4_t*>(dst + 8 * j));
      }
    }
  }
}

hipError_t launch_qk_norm_rope_store(const RopeStoreArgs& a, hipStream_t st) {
  if (a.num_tokens == 0) return hipSuccess;
  int64_t blocks = (int64_t(a.num_tokens) + kRopeWaves - 1) / kRopeWaves;   // a wave per token
  const int64_t cap = int64_t(a.num_cus) * NKV_ROPE_WGS_PER_CU;   // beyond, waves walk more tokens
  if (blocks > cap) blocks = cap;
  const auto* qkv = static_cast<const uint16_t*>(a.qkv);
  auto* q_out = static_cast<uint16_t*>(a.q_out);
  auto* kc = static_cast<uint16_t*>(a.k_cache);
  auto* vc = static_cast<uint16_t*>(a.v_cache);
  const auto* wq = static_cast<const uint16_t*>(a.q_weight);
  const auto* wk = static_cast<const uint16_t*>(a.k_weight);
  if (a.head_dim == 128)
    hipLaunchKernelGGL((qk_norm_rope_store_kernel<128>), dim3(int(blocks)), dim3(kRopeThreads), 0, st,
                       qkv, a.qkv_row, a.positions, wq, wk, a.cos_sin, a.eps, a.slot_mapping,
                       a.num_tokens, a.num_q_heads, a.num_kv_heads, q_out, kc, vc);
  else if (a.head_dim == 64)
    hipLaunchKernelGGL((qk_norm_rope_store_kernel<64>), dim3(int(blocks)), dim3(kRopeThreads), 0, st,
                       qkv, a.qkv_row, a.positions, wq, wk, a.cos_sin, a.eps, a.slot_mapping,
                       a.num_tokens, a.num_q_heads, a.num_kv_heads, q_out, kc, vc);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace nkv
