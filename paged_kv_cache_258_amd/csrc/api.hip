// C ABI of libnkv.so (declared in include/nkv.h): argument checks, then launches.
//
// Only host-checkable arguments are validated here; the contents of device-resident
// index arrays are preconditions of the kernels (as in the reference store kernel,
// 「Nano-vLLM深度解读（下）」 §4, which only tests for slot == -1).
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "nkv.h"  // include/ is on the include path
#include "launch.hpp"
#include "status.hpp"

#define NKV_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[512] = "";

nkv_status_t fail(nkv_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

nkv_status_t ok() {
  g_last_error[0] = '\0';
  return NKV_OK;
}

nkv_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(NKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Compute-unit count of the current device, cached per device.
int num_cus() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The value of an enum argument as the int the caller passed.  Across the C ABI any int
// may arrive; reading one outside the enumerators' range through the C++ enum type would
// be undefined behaviour, so it is read as an int and compared with the enumerators.
template <class E>
int abi_int(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized here");
  int v;
  memcpy(&v, &e, sizeof v);
  return v;
}

int ilog2_exact(int x) {
  if (x <= 0 || (x & (x - 1)) != 0) return -1;
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

int elem_bytes(int dt) { return dt == NKV_BF16 ? 2 : 4; }

// Checks shared by prefill and decode; fills the common launch descriptor.
nkv_status_t check_paged(const void* k_cache, const void* v_cache, const int32_t* block_table,
                         int32_t max_blocks_per_seq, int32_t num_seqs, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                         int32_t block_size, float softmax_scale, int dtype,
                         nkv::PagedArgs* pa) {
  if (dtype != NKV_F32 && dtype != NKV_BF16) return fail(NKV_ERR_INVALID_ARG, "unknown dtype %d", int(dtype));
  if (num_seqs < 0) return fail(NKV_ERR_INVALID_ARG, "num_seqs < 0");
  if (num_q_heads <= 0 || num_kv_heads <= 0)
    return fail(NKV_ERR_INVALID_ARG, "head counts must be positive");
  if (num_q_heads % num_kv_heads != 0)
    return fail(NKV_ERR_INVALID_ARG, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                num_q_heads, num_kv_heads);
  const int grp = num_q_heads / num_kv_heads;
  if (grp != 1 && grp != 2 && grp != 4 && grp != 8)
    return fail(NKV_ERR_UNSUPPORTED, "GQA group size %d not in {1,2,4,8}", grp);
  if (head_dim != 64 && head_dim != 128)
    return fail(NKV_ERR_UNSUPPORTED, "head_dim %d not in {64,128}", head_dim);
  const int lb = ilog2_exact(block_size);
  if (lb < 4 || lb > 10)
    return fail(NKV_ERR_UNSUPPORTED, "block_size %d is not a power of two in [16,1024]", block_size);
  if (num_blocks <= 0) return fail(NKV_ERR_INVALID_ARG, "num_blocks must be positive");
  if (int64_t(num_blocks) * block_size > int64_t(INT32_MAX))
    return fail(NKV_ERR_UNSUPPORTED, "pool has more than 2^31-1 rows");
  if (max_blocks_per_seq <= 0) return fail(NKV_ERR_INVALID_ARG, "max_blocks_per_seq must be positive");
  if (int64_t(max_blocks_per_seq) * block_size > int64_t(INT32_MAX))
    return fail(NKV_ERR_UNSUPPORTED, "max_blocks_per_seq * block_size exceeds 2^31-1");
  if (!(softmax_scale == softmax_scale) || softmax_scale < 0.f)
    return fail(NKV_ERR_INVALID_ARG, "softmax_scale must be a non-negative number");
  if (num_seqs > 0 && (!k_cache || !v_cache || !block_table))
    return fail(NKV_ERR_INVALID_ARG, "null pool or block_table pointer");
  if (num_seqs > 0 && (!aligned16(k_cache) || !aligned16(v_cache)))
    return fail(NKV_ERR_INVALID_ARG, "pools must be 16-byte aligned");
  pa->k_cache = k_cache;
  pa->v_cache = v_cache;
  pa->block_table = block_table;
  pa->max_blocks_per_seq = max_blocks_per_seq;
  pa->num_seqs = num_seqs;
  pa->num_q_heads = num_q_heads;
  pa->num_kv_heads = num_kv_heads;
  pa->head_dim = head_dim;
  pa->block_size = block_size;
  pa->log2_block_size = lb;
  pa->scale_log2e = softmax_scale * 1.4426950408889634f;
  pa->dtype = dtype == NKV_BF16 ? nkv::Dtype::BF16 : nkv::Dtype::F32;
  pa->num_cus = num_cus();
  return NKV_OK;
}

// Checking mode: NKV_VALIDATE=1 in the environment (read at every call).
bool validating() {
  const char* v = getenv("NKV_VALIDATE");
  return v && v[0] == '1' && v[1] == '\0';
}

const char* violation_name(int mask) {
  if (mask & nkv::kValidateSlotRange) return "slot_mapping entry outside [-1, num_blocks*block_size)";
  if (mask & nkv::kValidateSlotDuplicate) return "slot_mapping entry repeated in one call";
  if (mask & nkv::kValidateSeqlens) return "cu_seqlens not running sums within max_seqlen / total_q";
  if (mask & nkv::kValidateBlockId) return "block_table id outside [0, num_blocks)";
  if (mask & nkv::kValidateContextLen) return "context_lens entry outside [1, max_blocks_per_seq*block_size]";
  if (mask & nkv::kValidatePosition) return "positions entry outside [0, max_position)";
  return "unknown violation";
}

nkv_status_t checked(hipError_t e, const nkv::ValidateResult& r, const char* what) {
  if (e != hipSuccess) return fail(NKV_ERR_HIP, "%s check: %s", what, hipGetErrorString(e));
  if (r.mask != 0)
    return fail(NKV_ERR_INVALID_ARG, "%s (first at index %d; violation mask 0x%x)",
                violation_name(r.mask), r.index, r.mask);
  return NKV_OK;
}

// [a, a+na) and [b, b+nb) share a byte (null ranges share none)
bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b) return false;
  const auto pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + uintptr_t(nb) && pb < pa + uintptr_t(na);
}

}  // namespace

// The calling thread's last error, for the host-only parts of the library (status.hpp).
namespace nkv {
nkv_status_t set_error(nkv_status_t st, const char* msg) {
  snprintf(g_last_error, sizeof(g_last_error), "%s", msg);
  return st;
}
nkv_status_t clear_error() { return ok(); }
}  // namespace nkv

NKV_EXPORT int nkv_abi_version(void) { return NKV_ABI_VERSION; }

NKV_EXPORT const char* nkv_status_string(nkv_status_t status) {
  switch (abi_int(status)) {
    case NKV_OK: return "NKV_OK";
    case NKV_ERR_INVALID_ARG: return "NKV_ERR_INVALID_ARG";
    case NKV_ERR_UNSUPPORTED: return "NKV_ERR_UNSUPPORTED";
    case NKV_ERR_WORKSPACE: return "NKV_ERR_WORKSPACE";
    case NKV_ERR_HIP: return "NKV_ERR_HIP";
    case NKV_ERR_NO_SPACE: return "NKV_ERR_NO_SPACE";
  }
  return "NKV_UNKNOWN_STATUS";
}

NKV_EXPORT const char* nkv_last_error(void) { return g_last_error; }

NKV_EXPORT nkv_status_t nkv_store_kvcache(const void* key, int64_t key_row_stride,
                                          const void* value, int64_t value_row_stride,
                                          void* k_cache, void* v_cache,
                                          const int32_t* slot_mapping, int32_t num_tokens,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t num_blocks, int32_t block_size,
                                          nkv_dtype_t dtype_arg, hipStream_t stream) {
  const int dtype = abi_int(dtype_arg);
  if (dtype != NKV_F32 && dtype != NKV_BF16) return fail(NKV_ERR_INVALID_ARG, "unknown dtype %d", int(dtype));
  if (num_tokens < 0) return fail(NKV_ERR_INVALID_ARG, "num_tokens < 0");
  if (num_kv_heads <= 0 || head_dim <= 0) return fail(NKV_ERR_INVALID_ARG, "num_kv_heads and head_dim must be positive");
  if (num_blocks <= 0 || block_size <= 0) return fail(NKV_ERR_INVALID_ARG, "num_blocks and block_size must be positive");
  if (int64_t(num_blocks) * block_size > int64_t(INT32_MAX))
    return fail(NKV_ERR_UNSUPPORTED, "pool has more than 2^31-1 rows");
  const int eb = elem_bytes(dtype);
  const int64_t row = int64_t(num_kv_heads) * head_dim;
  if ((row * eb) % 16 != 0)
    return fail(NKV_ERR_UNSUPPORTED, "row of %lld elements is not a multiple of 16 bytes", (long long)row);
  if (key_row_stride < row || value_row_stride < row)
    return fail(NKV_ERR_INVALID_ARG, "row stride below num_kv_heads*head_dim");
  if ((key_row_stride * eb) % 16 != 0 || (value_row_stride * eb) % 16 != 0)
    return fail(NKV_ERR_INVALID_ARG, "row strides must be multiples of 16 bytes");
  if (num_tokens == 0) return ok();
  if (!key || !value || !k_cache || !v_cache || !slot_mapping)
    return fail(NKV_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(NKV_ERR_INVALID_ARG, "key/value/cache pointers must be 16-byte aligned");
  nkv::StoreArgs a{key, key_row_stride * eb, value, value_row_stride * eb, k_cache, v_cache,
                   slot_mapping, num_tokens, row * eb, num_cus()};
  if (validating()) {
    nkv::ValidateResult r{};
    const hipError_t e = nkv::validate_store(slot_mapping, num_tokens, int64_t(num_blocks) * block_size,
                                             stream, &r);
    const nkv_status_t vs = checked(e, r, "nkv_store_kvcache");
    if (vs != NKV_OK) return vs;
  }
  return hip_status(nkv::launch_store(a, stream), "store launch");
}

NKV_EXPORT nkv_status_t nkv_qk_norm_rope_store(
    const void* qkv, int64_t qkv_row_stride, const int32_t* positions, const void* q_norm_weight,
    const void* k_norm_weight, const float* cos_sin_cache, int32_t max_position, float eps,
    const int32_t* slot_mapping, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, void* q_out, void* k_cache, void* v_cache, int32_t num_blocks,
    int32_t block_size, nkv_dtype_t dtype_arg, hipStream_t stream) {
  const int dtype = abi_int(dtype_arg);
  if (dtype != NKV_F32 && dtype != NKV_BF16) return fail(NKV_ERR_INVALID_ARG, "unknown dtype %d", int(dtype));
  if (dtype != NKV_BF16) return fail(NKV_ERR_UNSUPPORTED, "q/k norm + rotary is implemented for bf16 only");
  if (num_tokens < 0) return fail(NKV_ERR_INVALID_ARG, "num_tokens < 0");
  if (num_q_heads <= 0 || num_kv_heads <= 0) return fail(NKV_ERR_INVALID_ARG, "head counts must be positive");
  if (head_dim != 64 && head_dim != 128) return fail(NKV_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", head_dim);
  if (num_blocks <= 0 || block_size <= 0) return fail(NKV_ERR_INVALID_ARG, "num_blocks and block_size must be positive");
  if (int64_t(num_blocks) * block_size > int64_t(INT32_MAX))
    return fail(NKV_ERR_UNSUPPORTED, "pool has more than 2^31-1 rows");
  if (max_position <= 0) return fail(NKV_ERR_INVALID_ARG, "max_position must be positive");
  if (!(eps >= 0.0f) || eps > 1.0f) return fail(NKV_ERR_INVALID_ARG, "eps must lie in [0, 1]");
  const int64_t slots_per_token = int64_t(num_q_heads) + 2 * int64_t(num_kv_heads);
  if (qkv_row_stride < slots_per_token * head_dim)
    return fail(NKV_ERR_INVALID_ARG, "qkv row stride below (num_q_heads + 2*num_kv_heads)*head_dim");
  if (qkv_row_stride % 8 != 0) return fail(NKV_ERR_INVALID_ARG, "qkv row stride must be a multiple of 8 elements");
  if (num_tokens == 0) return ok();
  if (!qkv || !positions || !q_norm_weight || !k_norm_weight || !cos_sin_cache || !slot_mapping ||
      !q_out || !k_cache || !v_cache)
    return fail(NKV_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(qkv) || !aligned16(q_norm_weight) || !aligned16(k_norm_weight) || !aligned16(q_out) ||
      !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(cos_sin_cache))
    return fail(NKV_ERR_INVALID_ARG, "qkv, weights, q_out, caches and cos_sin_cache need 16-byte alignment");
  nkv::RopeStoreArgs a{qkv, qkv_row_stride, positions, q_norm_weight, k_norm_weight, cos_sin_cache, eps,
                       slot_mapping, num_tokens, num_q_heads, num_kv_heads, head_dim, q_out, k_cache,
                       v_cache, num_cus()};
  if (validating()) {
    nkv::ValidateResult r{};
    const hipError_t e = nkv::validate_rope_store(positions, slot_mapping, num_tokens, max_position,
                                                  int64_t(num_blocks) * block_size,
                                                  stream, &r);
    const nkv_status_t vs = checked(e, r, "nkv_qk_norm_rope_store");
    if (vs != NKV_OK) return vs;
  }
  return hip_status(nkv::launch_qk_norm_rope_store(a, stream),
                    "q/k norm + rotary + store launch");
}

NKV_EXPORT nkv_status_t nkv_add_rms_norm(const void* x, const void* residual, const void* weight,
                                         float eps, int32_t num_tokens, int32_t hidden_size,
                                         void* out, void* residual_out, nkv_dtype_t dtype_arg,
                                         hipStream_t stream) {
  const int dtype = abi_int(dtype_arg);
  if (dtype != NKV_F32 && dtype != NKV_BF16) return fail(NKV_ERR_INVALID_ARG, "unknown dtype %d", int(dtype));
  if (dtype != NKV_BF16) return fail(NKV_ERR_UNSUPPORTED, "residual add + RMSNorm is implemented for bf16 only");
  if (num_tokens < 0) return fail(NKV_ERR_INVALID_ARG, "num_tokens < 0");
  if (hidden_size <= 0 || hidden_size % 8 != 0)
    return fail(NKV_ERR_INVALID_ARG, "hidden_size must be a positive multiple of 8");
  if (hidden_size > nkv::kAddRmsNormMaxHidden)
    return fail(NKV_ERR_UNSUPPORTED, "hidden_size %d above %d", hidden_size, nkv::kAddRmsNormMaxHidden);
  if (!(eps >= 0.0f) || eps > 1.0f) return fail(NKV_ERR_INVALID_ARG, "eps must lie in [0, 1]");
  if (num_tokens == 0) return ok();
  if (!x || !weight || !out) return fail(NKV_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(x) || !aligned16(residual) || !aligned16(weight) || !aligned16(out) ||
      !aligned16(residual_out))
    return fail(NKV_ERR_INVALID_ARG, "x, residual, weight, out and residual_out need 16-byte alignment");
  // each output is either the very same rows as an input (in place) or apart from every
  // other buffer
  const int64_t n = int64_t(num_tokens) * hidden_size * 2;
  const int64_t nw = int64_t(hidden_size) * 2;
  if (overlaps(out, n, residual_out, n)) return fail(NKV_ERR_INVALID_ARG, "out and residual_out overlap");
  for (void* o : {out, residual_out}) {
    if ((o != x && overlaps(o, n, x, n)) || (o != residual && overlaps(o, n, residual, n)) ||
        overlaps(o, n, weight, nw))
      return fail(NKV_ERR_INVALID_ARG, "an output overlaps an input other than as the same rows");
  }
  nkv::AddRmsNormArgs a{x, residual, weight, eps, num_tokens, hidden_size, out, residual_out, num_cus()};
  return hip_status(nkv::launch_add_rms_norm(a, stream),
                    "residual add + RMSNorm launch");
}

NKV_EXPORT nkv_status_t nkv_paged_attn_prefill(
    const void* q, int64_t q_row_stride, const void* k_cache, const void* v_cache,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, const int32_t* block_table,
    int32_t max_blocks_per_seq, int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
    int32_t max_seqlen_k, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t num_blocks, int32_t block_size, float softmax_scale, nkv_dtype_t dtype_arg, void* out,
    hipStream_t stream) {
  const int dtype = abi_int(dtype_arg);
  nkv::PrefillArgs a{};
  nkv_status_t st = check_paged(k_cache, v_cache, block_table, max_blocks_per_seq, num_seqs,
                                num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                                softmax_scale, dtype, &a.p);
  if (st != NKV_OK) return st;
  if (total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(NKV_ERR_INVALID_ARG, "negative size");
  if (max_seqlen_q > max_seqlen_k)
    return fail(NKV_ERR_INVALID_ARG, "max_seqlen_q (%d) > max_seqlen_k (%d)", max_seqlen_q, max_seqlen_k);
  if (int64_t(max_seqlen_k) > int64_t(max_blocks_per_seq) * block_size)
    return fail(NKV_ERR_INVALID_ARG, "max_seqlen_k exceeds max_blocks_per_seq*block_size");
  const int64_t qrow = int64_t(num_q_heads) * head_dim;
  if (q_row_stride < qrow) return fail(NKV_ERR_INVALID_ARG, "q_row_stride below num_q_heads*head_dim");
  const int eb = elem_bytes(dtype);
  if ((q_row_stride * eb) % 16 != 0) return fail(NKV_ERR_INVALID_ARG, "q_row_stride must be a multiple of 16 bytes");
  if (num_seqs == 0 || total_q == 0 || max_seqlen_q == 0) return ok();
  if (!q || !out || !cu_seqlens_q || !cu_seqlens_k) return fail(NKV_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(q) || !aligned16(out)) return fail(NKV_ERR_INVALID_ARG, "q/out must be 16-byte aligned");
  a.q = q;
  a.q_row_elems = q_row_stride;
  a.k_row_elems = a.v_row_elems = int64_t(num_kv_heads) * head_dim;
  a.cu_seqlens_q = cu_seqlens_q;
  a.cu_seqlens_k = cu_seqlens_k;
  a.max_seqlen_q = max_seqlen_q;
  a.max_seqlen_k = max_seqlen_k;
  a.out = out;
  if (validating()) {
    nkv::ValidateResult r{};
    const hipError_t e = nkv::validate_prefill(a, total_q, -1, num_blocks, stream, &r);
    const nkv_status_t vs = checked(e, r, "nkv_paged_attn_prefill");
    if (vs != NKV_OK) return vs;
  }
  return hip_status(nkv::launch_prefill(a, stream), "prefill launch");
}

NKV_EXPORT nkv_status_t nkv_attn_varlen_prefill(
    const void* q, int64_t q_row_stride, const void* k, int64_t k_row_stride, const void* v,
    int64_t v_row_stride, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_seqs,
    int32_t total_q, int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, float softmax_scale, nkv_dtype_t dtype_arg, void* out,
    hipStream_t stream) {
  const int dtype = abi_int(dtype_arg);
  if (dtype != NKV_F32 && dtype != NKV_BF16) return fail(NKV_ERR_INVALID_ARG, "unknown dtype %d", int(dtype));
  if (num_seqs < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(NKV_ERR_INVALID_ARG, "negative size");
  if (num_q_heads <= 0 || num_kv_heads <= 0) return fail(NKV_ERR_INVALID_ARG, "head counts must be positive");
  if (num_q_heads % num_kv_heads != 0)
    return fail(NKV_ERR_INVALID_ARG, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                num_q_heads, num_kv_heads);
  const int grp = num_q_heads / num_kv_heads;
  if (grp != 1 && grp != 2 && grp != 4 && grp != 8)
    return fail(NKV_ERR_UNSUPPORTED, "GQA group size %d not in {1,2,4,8}", grp);
  if (head_dim != 64 && head_dim != 128) return fail(NKV_ERR_UNSUPPORTED, "head_dim %d not in {64,128}", head_dim);
  if (!(softmax_scale == softmax_scale) || softmax_scale < 0.f)
    return fail(NKV_ERR_INVALID_ARG, "softmax_scale must be a non-negative number");
  if (max_seqlen_q > max_seqlen_k)
    return fail(NKV_ERR_INVALID_ARG, "max_seqlen_q (%d) > max_seqlen_k (%d)", max_seqlen_q, max_seqlen_k);
  if (max_seqlen_k > total_k) return fail(NKV_ERR_INVALID_ARG, "max_seqlen_k exceeds total_k");
  const int eb = elem_bytes(dtype);
  const int64_t qrow = int64_t(num_q_heads) * head_dim, kvrow = int64_t(num_kv_heads) * head_dim;
  if (q_row_stride < qrow) return fail(NKV_ERR_INVALID_ARG, "q_row_stride below num_q_heads*head_dim");
  if (k_row_stride < kvrow || v_row_stride < kvrow)
    return fail(NKV_ERR_INVALID_ARG, "k/v row stride below num_kv_heads*head_dim");
  if ((q_row_stride * eb) % 16 != 0 || (k_row_stride * eb) % 16 != 0 || (v_row_stride * eb) % 16 != 0)
    return fail(NKV_ERR_INVALID_ARG, "row strides must be multiples of 16 bytes");
  if (num_seqs == 0 || total_q == 0 || max_seqlen_q == 0) return ok();
  if (!q || !k || !v || !out || !cu_seqlens_q || !cu_seqlens_k)
    return fail(NKV_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(NKV_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  nkv::PrefillArgs a{};
  a.p.k_cache = k;
  a.p.v_cache = v;
  a.p.block_table = nullptr;                 // contiguous keys: rows cu_seqlens_k[b] ..
  a.p.max_blocks_per_seq = 0;
  a.p.num_seqs = num_seqs;
  a.p.num_q_heads = num_q_heads;
  a.p.num_kv_heads = num_kv_heads;
  a.p.head_dim = head_dim;
  a.p.block_size = 1 << 10;
  a.p.log2_block_size = 10;                  // unused without a block table
  a.p.scale_log2e = softmax_scale * 1.4426950408889634f;
  a.p.dtype = dtype == NKV_BF16 ? nkv::Dtype::BF16 : nkv::Dtype::F32;
  a.p.num_cus = num_cus();
  a.q = q;
  a.q_row_elems = q_row_stride;
  a.k_row_elems = k_row_stride;
  a.v_row_elems = v_row_stride;
  a.cu_seqlens_q = cu_seqlens_q;
  a.cu_seqlens_k = cu_seqlens_k;
  a.max_seqlen_q = max_seqlen_q;
  a.max_seqlen_k = max_seqlen_k;
  a.out = out;
  if (validating()) {
    nkv::ValidateResult r{};
    const hipError_t e = nkv::validate_prefill(a, total_q, total_k, 0, stream, &r);
    const nkv_status_t vs = checked(e, r, "nkv_attn_varlen_prefill");
    if (vs != NKV_OK) return vs;
  }
  return hip_status(nkv::launch_prefill(a, stream), "varlen prefill launch");
}

NKV_EXPORT size_t nkv_paged_attn_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                                      int32_t num_kv_heads, int32_t head_dim,
                                                      int32_t max_blocks_per_seq,
                                                      int32_t block_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_blocks_per_seq <= 0 || block_size <= 0)
    return 0;
  return nkv::plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                          block_size, num_cus())
      .workspace_bytes;
}

// Scratch of the allocation-free decode: a file-scope device array, one copy per device,
// held until the process ends.  Host code never names it directly (in host code the
// symbol is a host-side stand-in, not a device address): its device address is looked up
// once per device with that device current, and that pointer is what the kernels get.
// Its contents on entry do not matter to the decode kernels (the tail-unit counter is
// reset by the kernels themselves), so nothing is cleared between calls.
static __device__ __align__(256) uint8_t scratch[NKV_DECODE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device.
nkv_status_t scratch_ptr(void** out) {
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {nullptr};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(NKV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(NKV_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table covers", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(NKV_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return NKV_OK;
}

// Decode with the workspace given (the caller's buffer, or the library's static scratch).
nkv_status_t decode_impl(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* context_lens, const int32_t* block_table,
                         int32_t max_blocks_per_seq, int32_t num_seqs, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                         int32_t block_size, float softmax_scale, int dtype, void* out,
                         void* workspace, size_t workspace_bytes, bool scratch, hipStream_t stream) {
  nkv::DecodeArgs a{};
  nkv_status_t st = check_paged(k_cache, v_cache, block_table, max_blocks_per_seq, num_seqs,
                                num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                                softmax_scale, dtype, &a.p);
  if (st != NKV_OK) return st;
  if (num_seqs == 0) return ok();
  if (!q || !out || !context_lens) return fail(NKV_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(q) || !aligned16(out)) return fail(NKV_ERR_INVALID_ARG, "q/out must be 16-byte aligned");
  const nkv::DecodePlan plan = nkv::plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                max_blocks_per_seq, block_size, a.p.num_cus);
  if (plan.workspace_bytes > 0) {
    if (scratch) {   // the library's static scratch stands in for the caller's workspace
      if (plan.workspace_bytes > size_t(NKV_DECODE_SCRATCH_BYTES))
        return fail(NKV_ERR_WORKSPACE,
                    "decode of these sizes needs %zu bytes of scratch; the library's static scratch holds %zu "
                    "(use nkv_paged_attn_decode with a workspace)",
                    plan.workspace_bytes, size_t(NKV_DECODE_SCRATCH_BYTES));
      const nkv_status_t ss = scratch_ptr(&workspace);
      if (ss != NKV_OK) return ss;
      workspace_bytes = size_t(NKV_DECODE_SCRATCH_BYTES);
    }
    if (!workspace || workspace_bytes < plan.workspace_bytes)
      return fail(NKV_ERR_WORKSPACE, "decode needs %zu workspace bytes, got %zu", plan.workspace_bytes,
                  workspace ? workspace_bytes : size_t(0));
    if (!aligned16(workspace)) return fail(NKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  a.q = q;
  a.context_lens = context_lens;
  a.out = out;
  a.workspace = workspace;
  if (validating()) {
    nkv::ValidateResult r{};
    const hipError_t e = nkv::validate_decode(a, num_blocks, stream, &r);
    const nkv_status_t vs = checked(e, r, "nkv_paged_attn_decode");
    if (vs != NKV_OK) return vs;
  }
  return hip_status(nkv::launch_decode(a, plan, stream), "decode launch");
}

}  // namespace

NKV_EXPORT nkv_status_t nkv_paged_attn_decode(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* context_lens,
    const int32_t* block_table, int32_t max_blocks_per_seq, int32_t num_seqs, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
    float softmax_scale, nkv_dtype_t dtype_arg, void* out, void* workspace, size_t workspace_bytes,
    hipStream_t stream) {
  const int dtype = abi_int(dtype_arg);
  return decode_impl(q, k_cache, v_cache, context_lens, block_table, max_blocks_per_seq, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, num_blocks, block_size, softmax_scale, dtype,
                     out, workspace, workspace_bytes, false, stream);
}

NKV_EXPORT nkv_status_t nkv_paged_attn_decode_noalloc(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* context_lens,
    const int32_t* block_table, int32_t max_blocks_per_seq, int32_t num_seqs, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
    float softmax_scale, nkv_dtype_t dtype_arg, void* out, hipStream_t stream) {
  const int dtype = abi_int(dtype_arg);
  return decode_impl(q, k_cache, v_cache, context_lens, block_table, max_blocks_per_seq, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, num_blocks, block_size, softmax_scale, dtype,
                     out, nullptr, 0, true, stream);
}
