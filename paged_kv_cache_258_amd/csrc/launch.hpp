// Host-side launch descriptors shared by the C ABI layer (api.hip) and the kernel
// files.  The ABI layer validates arguments and fills these; the launchers only size
// grids and enqueue kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nkv {

enum class Dtype { F32 = 0, BF16 = 1 };

struct StoreArgs {
  const void* key;
  int64_t key_row_bytes;
  const void* value;
  int64_t value_row_bytes;
  void* k_cache;
  void* v_cache;
  const int32_t* slot_mapping;
  int32_t num_tokens;
  int64_t row_bytes;  // num_kv_heads * head_dim * element size
  int num_cus;
};

// q/k RMSNorm + rotary + store (bf16).  Strides in elements.
struct RopeStoreArgs {
  const void* qkv;
  int64_t qkv_row;
  const int32_t* positions;
  const void* q_weight;
  const void* k_weight;
  const float* cos_sin;
  float eps;
  const int32_t* slot_mapping;
  int32_t num_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  void* q_out;
  void* k_cache;
  void* v_cache;
  int num_cus;
};
hipError_t launch_qk_norm_rope_store(const RopeStoreArgs& a, hipStream_t st);

// Residual add + RMSNorm over contiguous [num_tokens, hidden] bf16 rows.  residual and
// residual_out may be null; out may equal x and residual_out may equal residual.
struct AddRmsNormArgs {
  const void* x;
  const void* residual;
  const void* weight;
  float eps;
  int32_t num_tokens;
  int32_t hidden;
  void* out;
  void* residual_out;
  int num_cus;
};
hipError_t launch_add_rms_norm(const AddRmsNormArgs& a, hipStream_t st);
constexpr int32_t kAddRmsNormMaxHidden = 16384;

struct PagedArgs {
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  int32_t max_blocks_per_seq;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t log2_block_size;
  float scale_log2e;  // softmax_scale * log2(e)
  Dtype dtype;
  int num_cus;
};

// Prefill over the paged pools, or (p.block_table == nullptr) over contiguous varlen K/V:
// sequence b's keys are rows cu_seqlens_k[b] .. cu_seqlens_k[b+1] of k/v (p.k_cache /
// p.v_cache), rows k_row_elems / v_row_elems elements apart.  Paged: both Hkv * D.
struct PrefillArgs {
  PagedArgs p;
  const void* q;
  int64_t q_row_elems;
  int64_t k_row_elems;
  int64_t v_row_elems;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int32_t max_seqlen_q;
  int32_t max_seqlen_k;
  void* out;
};

struct DecodeArgs {
  PagedArgs p;
  const void* q;
  const int32_t* context_lens;
  void* out;
  void* workspace;
};

// Work plan of a decode call.
//   fp32 (split-K): each (sequence, KV head) is cut into chunks of `split_tokens`
//   logical positions; `max_splits` bounds the chunks of any sequence.
//   bf16 (stream-K): `wgs` persistent workgroups share the batch's rounds equally;
//   sequences are processed `seq_chunk` at a time.
// `workspace_bytes` covers whichever path the dtype selects.
struct DecodePlan {
  int32_t split_tokens;
  int32_t max_splits;
  int32_t wgs;
  int32_t pieces;           // stream-K partial-slot pairs: wgs ranges + tail units
  int32_t seq_chunk;
  size_t workspace_bytes;
};

DecodePlan plan_decode(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                       int num_cus);

// Checking mode: violation bits and the first offending index (token or sequence).
enum : int {
  kValidateSlotRange = 1,       // slot not -1 and outside [0, num_blocks*block_size)
  kValidateSlotDuplicate = 2,   // a non-negative slot appears twice in one call
  kValidateSeqlens = 4,         // cu_seqlens not running sums / lengths out of bounds
  kValidateBlockId = 8,         // a used block_table entry outside [0, num_blocks)
  kValidateContextLen = 16,     // context_lens[b] outside [1, max_blocks_per_seq*block_size]
  kValidatePosition = 32,       // positions[t] outside [0, max_position)
};
struct ValidateResult {
  int mask;
  int index;
};
hipError_t validate_store(const int32_t* slots, int32_t n, int64_t rows, hipStream_t st,
                          ValidateResult* r);
// total_k: rows of contiguous K/V (no block table), or -1 for the paged pools.
hipError_t validate_prefill(const PrefillArgs& a, int32_t total_q, int32_t total_k,
                            int32_t num_blocks, hipStream_t st, ValidateResult* r);
hipError_t validate_decode(const DecodeArgs& a, int32_t num_blocks, hipStream_t st,
                           ValidateResult* r);

hipError_t validate_rope_store(const int32_t* positions, const int32_t* slots, int32_t n,
                              int32_t max_position, int64_t rows, hipStream_t st, ValidateResult* r);

hipError_t launch_store(const StoreArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream);

}  // namespace nkv
