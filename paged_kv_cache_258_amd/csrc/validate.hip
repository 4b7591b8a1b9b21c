// Checking mode (NKV_VALIDATE=1): the contents of the device-resident index arrays,
// which the kernels otherwise take as preconditions, are checked on the device before
// anything else is launched.
//
// What is checked, and where the pages define it:
//   slot_mapping  each entry -1 ("skip", 「Nano-vLLM深度解读（下）」 §4 store kernel) or a
//                 row of the pool, [0, num_blocks*block_size); non-negative entries
//                 unique within one call (two programs writing one row would race);
//   block_table   the ids of the logical blocks a sequence uses lie in [0, num_blocks)
//                 (「同一个 Qwen3，两种写法」 §3.3, the per-sequence page table);
//   cu_seqlens    running sums of the flat varlen batch (same page, §3.2): start at 0,
//                 non-decreasing, cu_q[B] = total_q, per sequence 0 <= Lq <= Lk,
//                 Lq <= max_seqlen_q, Lk <= max_seqlen_k;
//   context_lens  1 <= L <= max_blocks_per_seq*block_size (the decode query attends to
//                 the token stored just before the call);
//   positions     rows of the cos/sin table, [0, max_position) (「同一个 Qwen3，两种写法」
//                 §3.5, the table is indexed by position).
// A violation sets one bit of a mask and lowers the first offending index.  The host
// copies both back after the stream has drained and returns NKV_ERR_INVALID_ARG, so
// invalid arrays never reach the store or attention kernels.  The flags live in a
// file-scope device array: checking mode allocates nothing, but it synchronises the
// stream and so is for debugging, not for the hot loop.
#include <limits.h>

#include "common.hpp"
#include "launch.hpp"

namespace nkv {

__device__ int32_t g_validate_flags[2];   // violation mask, first offending index

__device__ __forceinline__ void report(int bit, int index) {
  atomicOr(&g_validate_flags[0], bit);
  atomicMin(&g_validate_flags[1], index);
}

__global__ void __launch_bounds__(64) validate_reset_kernel() {
  if (threadIdx.x == 0) {
    g_validate_flags[0] = 0;
    g_validate_flags[1] = INT_MAX;
  }
}

// One thread per token i: range of slot i, then slot i against the slots j > i, the
// candidates staged through LDS 1024 at a time.
__global__ void __launch_bounds__(256)
validate_slots_kernel(const int32_t* __restrict__ slots, int32_t n, int64_t rows) {
  __shared__ int32_t s_c[1024];
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int32_t si = i < n ? slots[i] : -1;
  if (i < n && (si < -1 || int64_t(si) >= rows)) report(kValidateSlotRange, i);
  for (int base = blockIdx.x * 256; base < n; base += 1024) {
    __syncthreads();
    for (int k = threadIdx.x; k < 1024; k += 256) s_c[k] = base + k < n ? slots[base + k] : -1;
    __syncthreads();
    if (si >= 0) {
      const int lim = n - base < 1024 ? n - base : 1024;
      for (int k = 0; k < lim; ++k)
        if (base + k > i && s_c[k] == si) {
          report(kValidateSlotDuplicate, i);
          break;
        }
    }
  }
}

// One thread per sequence: the block ids of its first `len` positions.
__device__ __forceinline__ void check_blocks(const int32_t* __restrict__ row, int64_t len,
                                             int32_t log2_bs, int32_t num_blocks, int b) {
  const int64_t nblk = (len + (int64_t(1) << log2_bs) - 1) >> log2_bs;
  for (int64_t i = 0; i < nblk; ++i) {
    const int32_t id = row[i];
    if (id < 0 || id >= num_blocks) {
      report(kValidateBlockId, b);
      return;
    }
  }
}

__global__ void __launch_bounds__(64)
validate_prefill_kernel(const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                        const int32_t* __restrict__ block_table, int32_t max_blocks,
                        int32_t num_seqs, int32_t total_q, int32_t total_k, int32_t max_seqlen_q,
                        int32_t max_seqlen_k, int32_t log2_bs, int32_t num_blocks) {
  const int b = blockIdx.x * 64 + threadIdx.x;
  if (b >= num_seqs) return;
  if (b == 0 && (cu_q[0] != 0 || cu_k[0] != 0)) report(kValidateSeqlens, 0);
  if (b == num_seqs - 1 && cu_q[num_seqs] != total_q) report(kValidateSeqlens, b);
  // contiguous K/V (no block table): the keys must lie in the total_k rows given
  if (total_k >= 0 && b == num_seqs - 1 && cu_k[num_seqs] > total_k) report(kValidateSeqlens, b);
  const int32_t lq = cu_q[b + 1] - cu_q[b];
  const int32_t lk = cu_k[b + 1] - cu_k[b];
  if (lq < 0 || lk < 0 || lq > lk || lq > max_seqlen_q || lk > max_seqlen_k) {
    report(kValidateSeqlens, b);
    return;
  }
  if (block_table) check_blocks(block_table + int64_t(b) * max_blocks, lk, log2_bs, num_blocks, b);
}

__global__ void __launch_bounds__(64)
validate_decode_kernel(const int32_t* __restrict__ context_lens,
                       const int32_t* __restrict__ block_table, int32_t max_blocks,
                       int32_t num_seqs, int32_t log2_bs, int32_t num_blocks) {
  const int b = blockIdx.x * 64 + threadIdx.x;
  if (b >= num_seqs) return;
  const int32_t len = context_lens[b];
  if (len < 1 || int64_t(len) > (int64_t(max_blocks) << log2_bs)) {
    report(kValidateContextLen, b);
    return;
  }
  check_blocks(block_table + int64_t(b) * max_blocks, len, log2_bs, num_blocks, b);
}

__global__ void __launch_bounds__(256)
validate_positions_kernel(const int32_t* __restrict__ positions, int32_t n, int32_t max_position) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n && (positions[i] < 0 || positions[i] >= max_position)) report(kValidatePosition, i);
}

namespace {

// Drain the checks and read the flags back (the stream is synchronised here).
hipError_t collect(hipStream_t st, ValidateResult* r) {
  int32_t h[2] = {0, INT_MAX};
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipMemcpyFromSymbolAsync(h, HIP_SYMBOL(g_validate_flags), sizeof(h), 0,
                               hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return e;
  r->mask = h[0];
  r->index = h[1];
  return hipSuccess;
}

}  // namespace

hipError_t validate_store(const int32_t* slots, int32_t n, int64_t rows, hipStream_t st,
                          ValidateResult* r) {
  hipLaunchKernelGGL(validate_reset_kernel, dim3(1), dim3(64), 0, st);
  if (n > 0)
    hipLaunchKernelGGL(validate_slots_kernel, dim3((n + 255) / 256), dim3(256), 0, st, slots, n,
                       rows);
  return collect(st, r);
}

hipError_t validate_rope_store(const int32_t* positions, const int32_t* slots, int32_t n,
                              int32_t max_position, int64_t rows, hipStream_t st, ValidateResult* r) {
  hipLaunchKernelGGL(validate_reset_kernel, dim3(1), dim3(64), 0, st);
  if (n > 0) {
    hipLaunchKernelGGL(validate_positions_kernel, dim3((n + 255) / 256), dim3(256), 0, st, positions, n,
                       max_position);
    hipLaunchKernelGGL(validate_slots_kernel, dim3((n + 255) / 256), dim3(256), 0, st, slots, n, rows);
  }
  return collect(st, r);
}

hipError_t validate_prefill(const PrefillArgs& a, int32_t total_q, int32_t total_k,
                            int32_t num_blocks, hipStream_t st, ValidateResult* r) {
  const PagedArgs& p = a.p;
  hipLaunchKernelGGL(validate_reset_kernel, dim3(1), dim3(64), 0, st);
  if (p.num_seqs > 0)
    hipLaunchKernelGGL(validate_prefill_kernel, dim3((p.num_seqs + 63) / 64), dim3(64), 0, st,
                       a.cu_seqlens_q, a.cu_seqlens_k, p.block_table, p.max_blocks_per_seq,
                       p.num_seqs, total_q, total_k, a.max_seqlen_q, a.max_seqlen_k,
                       p.log2_block_size, num_blocks);
  return collect(st, r);
}

hipError_t validate_decode(const DecodeArgs& a, int32_t num_blocks, hipStream_t st,
                           ValidateResult* r) {
  const PagedArgs& p = a.p;
  hipLaunchKernelGGL(validate_reset_kernel, dim3(1), dim3(64), 0, st);
  if (p.num_seqs > 0)
    hipLaunchKernelGGL(validate_decode_kernel, dim3((p.num_seqs + 63) / 64), dim3(64), 0, st,
                       a.context_lens, p.block_table, p.max_blocks_per_seq, p.num_seqs,
                       p.log2_block_size, num_blocks);
  return collect(st, r);
}

}  // namespace nkv
