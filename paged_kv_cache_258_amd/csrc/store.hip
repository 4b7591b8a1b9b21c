// KV store: scatter new K/V rows into the paged pools through slot_mapping.
//
// 「Nano-vLLM深度解读（下）」 §4, store_kvcache_kernel: one program per new token reads
// its slot, skips the token when the slot is -1, and copies the token's
// num_kv_heads*head_dim key and value elements to row `slot` of k_cache / v_cache.
//
// MI355X layout of the work: one wave per token, each lane moving 16-byte vectors
// (a 2 KiB bf16 Qwen3-8B row is 128 vectors, two per lane for K and two for V, all
// loads issued before the stores).  The slot is loaded once per wave.  Waves walk the
// tokens grid-stride so the launch fills every CU without one workgroup per token.
// The copy is a bit copy: no type conversion, so bf16 and fp32 share the kernel.
// The pool rows are written with the nontemporal hint (16384 tokens of 8 KV heads x 128:
// 23.8 vs 25.4 us per call; 512 tokens x 16 chunks back to back: 10.0 vs 11.0 us).
#include "common.hpp"
#include "launch.hpp"

namespace nkv {

constexpr int kStoreThreads = 256;
constexpr int kStoreWaves = kStoreThreads / kWave;
constexpr int kStoreUnroll = 4;  // 16-byte vectors per lane per pass, for K and for V

__global__ void __launch_bounds__(kStoreThreads)
store_kvcache_kernel(const char* __restrict__ key, int64_t key_row_bytes,
                     const char* __restrict__ value, int64_t value_row_bytes,
                     char* __restrict__ k_cache, char* __restrict__ v_cache,
                     const int32_t* __restrict__ slot_mapping, int32_t num_tokens,
                     int32_t row_vecs /* row bytes / 16 */) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int64_t row_bytes = int64_t(row_vecs) * 16;
  for (int t = blockIdx.x * kStoreWaves + wave; t < num_tokens; t += gridDim.x * kStoreWaves) {
    const int32_t slot = __builtin_amdgcn_readfirstlane(slot_mapping[t]);
    if (slot == -1) continue;
    const u32x4_t* ksrc = reinterpret_cast<const u32x4_t*>(key + int64_t(t) * key_row_bytes);
    const u32x4_t* vsrc = reinterpret_cast<const u32x4_t*>(value + int64_t(t) * value_row_bytes);
    u32x4_t* kdst = reinterpret_cast<u32x4_t*>(k_cache + int64_t(slot) * row_bytes);
    u32x4_t* vdst = reinterpret_cast<u32x4_t*>(v_cache + int64_t(slot) * row_bytes);
    for (int base = 0; base < row_vecs; base += kWave * kStoreUnroll) {
      u32x4_t kb[kStoreUnroll], vb[kStoreUnroll];
#pragma unroll
      for (int u = 0; u < kStoreUnroll; ++u) {
        const int i = base + u * kWave + lane;
        if (i < row_vecs) {
          kb[u] = ksrc[i];
          vb[u] = vsrc[i];
        }
      }
#pragma unroll
      for (int u = 0; u < kStoreUnroll; ++u) {
        const int i = base + u * kWave + lane;
        if (i < row_vecs) {
          __builtin_nontemporal_store(kb[u], kdst + i);
          __builtin_nontemporal_store(vb[u], vdst + i);
        }
      }
    }
  }
}

hipError_t launch_store(const StoreArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const int row_vecs = int(a.row_bytes / 16);
  int blocks = (a.num_tokens + kStoreWaves - 1) / kStoreWaves;
  const int cap = a.num_cus * 8;  // enough resident waves to cover HBM latency
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(store_kvcache_kernel, dim3(blocks), dim3(kStoreThreads), 0, stream,
                     static_cast<const char*>(a.key), a.key_row_bytes,
                     static_cast<const char*>(a.value), a.value_row_bytes,
                     static_cast<char*>(a.k_cache), static_cast<char*>(a.v_cache),
                     a.slot_mapping, a.num_tokens, row_vecs);
  return hipGetLastError();
}

}  // namespace nkv
