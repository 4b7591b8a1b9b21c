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
// the projection output is read once and each result written once.
//
// Layout of the work: one wave per token (grid-stride over tokens), so the position, the
// slot, the cos/sin row and the norm weights are read once per token and every head's
// loads go out together.  A head of D dims is handled by D/8 lanes: lane j of a head holds
// dims [4j, 4j+4) of the first half and the same dims of the second half, so the rotation
// pairs live in one lane, and a head's mean square is a butterfly over its D/8 lanes.  The
// 64/(D/8) lane groups of a wave take head slots g, g + 64/(D/8), ... (q heads, then k,
// then v, as the projection lays them out), up to 64 slots per pass.  Float contraction
// is off so that the rotation rounds its two products and their sum separately, as the
// listing's float32 tensor arithmetic does.  The head sums run over DPP lane moves in an
// order that gives every lane of a head the same bits, and the reciprocal root is the
// hardware's v_rsq_f32 (within an ulp, like the listing's rsqrt).
#include "common.hpp"
#include "launch.hpp"

namespace nkv {

constexpr int kRopeThreads = 256;
constexpr int kRopeWaves = kRopeThreads / kWave;

__device__ __forceinline__ float round_bf16(float x) {   // round to nearest even, to bf16
  return __builtin_bit_cast(float, uint32_t(__builtin_bit_cast(uint16_t, (__bf16)x)) << 16);
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
  const int lane = threadIdx.x % kWave;
  const int j = lane % LPH;
  const int g = lane / LPH;
  const int nslots = num_q_heads + 2 * num_kv_heads;
  const int first_v = num_q_heads + num_kv_heads;
  const int64_t row_kv = int64_t(num_kv_heads) * D;   // pool row, elements
  // per-lane constants: the norm weights of this lane's dims
  const u32x2_t qa = *reinterpret_cast<const u32x2_t*>(q_weight + 4 * j);
  const u32x2_t qb = *reinterpret_cast<const u32x2_t*>(q_weight + H2 + 4 * j);
  const u32x2_t ka = *reinterpret_cast<const u32x2_t*>(k_weight + 4 * j);
  const u32x2_t kb = *reinterpret_cast<const u32x2_t*>(k_weight + H2 + 4 * j);
  const float wq1[4] = {bf16_lo(qa[0]), bf16_hi(qa[0]), bf16_lo(qa[1]), bf16_hi(qa[1])};
  const float wq2[4] = {bf16_lo(qb[0]), bf16_hi(qb[0]), bf16_lo(qb[1]), bf16_hi(qb[1])};
  const float wk1[4] = {bf16_lo(ka[0]), bf16_hi(ka[0]), bf16_lo(ka[1]), bf16_hi(ka[1])};
  const float wk2[4] = {bf16_lo(kb[0]), bf16_hi(kb[0]), bf16_lo(kb[1]), bf16_hi(kb[1])};

  for (int t = blockIdx.x * kRopeWaves + threadIdx.x / kWave; t < num_tokens;
       t += gridDim.x * kRopeWaves) {
    const int pos = __builtin_amdgcn_readfirstlane(positions[t]);
    const int32_t slot = __builtin_amdgcn_readfirstlane(slot_mapping[t]);
    const f32x4_t c = *reinterpret_cast<const f32x4_t*>(cos_sin + int64_t(pos) * D + 4 * j);
    const f32x4_t sn = *reinterpret_cast<const f32x4_t*>(cos_sin + int64_t(pos) * D + H2 + 4 * j);
    const uint16_t* src = qkv + int64_t(t) * qkv_row;
    for (int s0 = 0; s0 < nslots; s0 += GL * KR) {
      u32x2_t a[KR], b[KR];
#pragma unroll
      for (int k = 0; k < KR; ++k) {                      // every load of the pass first
        const int s = s0 + k * GL + g;
        if (s < nslots) {
          a[k] = *reinterpret_cast<const u32x2_t*>(src + int64_t(s) * D + 4 * j);
          b[k] = *reinterpret_cast<const u32x2_t*>(src + int64_t(s) * D + H2 + 4 * j);
        } else {
          a[k] = u32x2_t{0, 0};
          b[k] = u32x2_t{0, 0};
        }
      }
#pragma unroll
      for (int k = 0; k < KR; ++k) {
        const int s = s0 + k * GL + g;
        if (s0 + k * GL >= nslots) break;                // no group of this row has a slot
        if (s >= first_v) {                              // v: stored as it is
          if (s < nslots && slot >= 0) {
            uint16_t* dst = v_cache + int64_t(slot) * row_kv + int64_t(s - first_v) * D;
            *reinterpret_cast<u32x2_t*>(dst + 4 * j) = a[k];
            *reinterpret_cast<u32x2_t*>(dst + H2 + 4 * j) = b[k];
          }
          continue;
        }
        // q or k head: mean square over the head (8 squares here, a butterfly over its
        // LPH lanes), then norm, cast, weight, cast, rotation, cast
        const bool is_q = s < num_q_heads;
        const float x1[4] = {bf16_lo(a[k][0]), bf16_hi(a[k][0]), bf16_lo(a[k][1]), bf16_hi(a[k][1])};
        const float x2[4] = {bf16_lo(b[k][0]), bf16_hi(b[k][0]), bf16_lo(b[k][1]), bf16_hi(b[k][1])};
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) ss += x1[i] * x1[i] + x2[i] * x2[i];
        ss = group8_sum(ss);                             // DPP: every lane of the group
        if constexpr (LPH == 16) ss += dpp<kDppRowRor8>(ss);   // gets the same sum
        const float r = __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);   // v_rsq_f32
        float o1[4], o2[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float y1 = round_bf16(round_bf16(x1[i] * r) * (is_q ? wq1[i] : wk1[i]));
          const float y2 = round_bf16(round_bf16(x2[i] * r) * (is_q ? wq2[i] : wk2[i]));
          o1[i] = y1 * c[i] - y2 * sn[i];
          o2[i] = y2 * c[i] + y1 * sn[i];
        }
        const u32x2_t p1 = {pack_bf16x2(o1[0], o1[1]), pack_bf16x2(o1[2], o1[3])};
        const u32x2_t p2 = {pack_bf16x2(o2[0], o2[1]), pack_bf16x2(o2[2], o2[3])};
        uint16_t* dst = nullptr;
        if (is_q)
          dst = q_out + (int64_t(t) * num_q_heads + s) * D;
        else if (slot >= 0)
          dst = k_cache + int64_t(slot) * row_kv + int64_t(s - num_q_heads) * D;
        if (dst) {
          *reinterpret_cast<u32x2_t*>(dst + 4 * j) = p1;
          *reinterpret_cast<u32x2_t*>(dst + H2 + 4 * j) = p2;
        }
      }
    }
  }
}

hipError_t launch_qk_norm_rope_store(const RopeStoreArgs& a, hipStream_t st) {
  if (a.num_tokens == 0) return hipSuccess;
  int64_t blocks = (int64_t(a.num_tokens) + kRopeWaves - 1) / kRopeWaves;   // a wave per token
  const int64_t cap = int64_t(a.num_cus) * 8;   // beyond that, waves walk more tokens
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
