/*
 * nkv.h -- C ABI of libnkv.so: the paged KV-cache data plane on AMD MI355X (gfx950).
 *
 * Three operations, named after the calls they replace in nano-vLLM's
 * Attention.forward (「Nano-vLLM深度解读（下）」 §4, attention.py listing):
 *
 *   nkv_store_kvcache       store_kvcache(k, v, k_cache, v_cache, slot_mapping)
 *   nkv_paged_attn_prefill  flash_attn_varlen_func(q, k_cache, v_cache, cu_seqlens_q/k,
 *                           max_seqlen_q/k, softmax_scale, causal=True, block_table)
 *   nkv_paged_attn_decode   flash_attn_with_kvcache(q.unsqueeze(1), k_cache, v_cache,
 *                           cache_seqlens=context_lens, block_table, softmax_scale,
 *                           causal=True)
 *   nkv_attn_varlen_prefill flash_attn_varlen_func(q, k, v, cu_seqlens_q/k, max_seqlen_q/k,
 *                           softmax_scale, causal=True)   (no prefix cache: fresh k, v)
 *
 * and the step right before the store in Qwen3Attention.forward (same page, §2), fused:
 *
 *   nkv_qk_norm_rope_store  q_norm(q), k_norm(k), rotary_emb(positions, q, k), then
 *                           store_kvcache(k, v, ...)
 *
 * and the residual add + RMSNorm that feeds each decoder block's q/k/v projection
 * (「同一个 Qwen3，两种写法」 §3.6, add_rms_forward):
 *
 *   nkv_add_rms_norm        x, residual = norm(x + residual), x + residual
 *
 * Data layout (「同一个 Qwen3，两种写法」 §3.3, the pool allocated once at start-up):
 *   one layer's K pool and V pool are each a contiguous
 *   [num_blocks, block_size, num_kv_heads, head_dim] array, so a cache row ("slot")
 *   is num_kv_heads*head_dim contiguous elements and slot = physical_block *
 *   block_size + offset_in_block.  Every pointer argument is a DEVICE pointer except
 *   where stated; sizes are element counts unless stated.
 *
 * Ownership and ordering:
 *   - the caller owns every buffer; the library allocates nothing and keeps no state
 *     between calls (it caches the device's compute-unit count per device);
 *   - every call is asynchronous and ordered on `stream` (NULL = the legacy default
 *     stream); nothing is read back to the host;
 *   - outside checking mode a call allocates nothing, issues no memset and never
 *     synchronises, so it can be captured into a HIP graph (stream capture) and
 *     replayed; the decode work split is derived on the device from context_lens, so
 *     a captured decode stays valid while the lengths in that buffer change;
 *   - attention never writes the pools; the store writes only the rows that
 *     slot_mapping names; attention's `out` is fully overwritten and must not alias
 *     any input (nkv_add_rms_norm alone may work in place, as stated there);
 *   - store before attention is the caller's job (the new token's K/V must be in the
 *     pool before the decode or prefix-cached prefill that reads it).
 *
 * Errors: every function returns a status and never aborts.  Arguments the host can
 * check (null pointers with non-zero sizes, dtype, head counts, head_dim, block_size,
 * strides, alignment, workspace size) are always checked and rejected with
 * NKV_ERR_INVALID_ARG or NKV_ERR_UNSUPPORTED before anything is launched.  The
 * contents of device-resident index arrays are preconditions, as in the reference
 * store kernel: slots in [0, num_blocks*block_size) or -1 and unique within a call;
 * block ids in [0, num_blocks) for every logical block a sequence uses;
 * 1 <= context_lens[b] <= max_blocks_per_seq*block_size; cu_seqlens non-decreasing
 * with 0 <= Lq <= Lk per sequence; positions in [0, max_position).  A launch failure returns NKV_ERR_HIP.
 * nkv_last_error() gives a human-readable reason for the last failure on the
 * calling thread.
 *
 * Checking mode: with NKV_VALIDATE=1 in the environment (read at every call) each
 * call first checks those device-resident preconditions on the device -- slots in
 * range and unique, the block ids each sequence uses in [0, num_blocks),
 * context_lens in [1, max_blocks_per_seq*block_size], cu_seqlens running sums from 0
 * with Lq <= Lk, Lq <= max_seqlen_q, Lk <= max_seqlen_k and cu_seqlens_q[B] = total_q,
 * positions in [0, max_position) -- waits for the stream, and returns NKV_ERR_INVALID_ARG (naming the violation and
 * the first offending token or sequence) without launching the operation.  It
 * allocates nothing but synchronises the stream: a debugging aid, not for hot loops.
 *
 * Tuning: NKV_PREFILL_XCD_GROUP=n in the environment (read at every bf16 prefill call)
 * sets how many (sequence, KV head) slices each XCD takes at a time (0: one longest-first
 * order over all of them); the default is half of an XCD's slices when that still gives
 * each of its CUs a workgroup.  It changes the order of work only, never the results.
 */
#ifndef NKV_H
#define NKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NKV_ABI_VERSION 1

/* HIP's stream handle, declared here as HIP's own runtime header declares it, so that
 * this header needs no HIP include (a repeated identical typedef is valid C11 / C++). */
typedef struct ihipStream_t* hipStream_t;

typedef enum {
  NKV_OK = 0,
  NKV_ERR_INVALID_ARG = 1, /* a host-checkable argument is wrong                  */
  NKV_ERR_UNSUPPORTED = 2, /* valid, but outside what the kernels are built for    */
  NKV_ERR_WORKSPACE = 3,   /* decode workspace missing or smaller than required    */
  NKV_ERR_HIP = 4,         /* the HIP runtime reported an error                     */
  NKV_ERR_NO_SPACE = 5     /* block manager: not enough free blocks (nothing changed) */
} nkv_status_t;

typedef enum {
  NKV_F32 = 0,  /* IEEE binary32                                 */
  NKV_BF16 = 1  /* bfloat16 (upper 16 bits of a binary32)        */
} nkv_dtype_t;

/* Version of this header's ABI (NKV_ABI_VERSION the library was built with). */
int nkv_abi_version(void);

/* Static string naming a status code. */
const char* nkv_status_string(nkv_status_t status);

/* Reason for the last non-OK status returned on this thread ("" if none). */
const char* nkv_last_error(void);

/*
 * Scatter new K/V rows into one layer's paged pools through slot_mapping.
 * 「Nano-vLLM深度解读（下）」 §4 (store_kvcache_kernel / store_kvcache): token t with
 * slot s = slot_mapping[t] copies key[t] (num_kv_heads*head_dim elements) to row s of
 * k_cache and value[t] to row s of v_cache; s == -1 skips the token.  The copy is bit
 * exact (no conversion).
 *
 *   key, value        [num_tokens, num_kv_heads, head_dim]; the last two dims are
 *                     contiguous; rows are key_row_stride / value_row_stride ELEMENTS
 *                     apart (>= num_kv_heads*head_dim, e.g. a k/v view cut from a packed
 *                     qkv projection output).  Base pointers and row strides must be
 *                     16-byte aligned.
 *   k_cache, v_cache  [num_blocks, block_size, num_kv_heads, head_dim], contiguous,
 *                     16-byte aligned.
 *   slot_mapping      [num_tokens] int32.
 *   num_tokens == 0 is a no-op.
 */
nkv_status_t nkv_store_kvcache(const void* key, int64_t key_row_stride,
                               const void* value, int64_t value_row_stride,
                               void* k_cache, void* v_cache,
                               const int32_t* slot_mapping, int32_t num_tokens,
                               int32_t num_kv_heads, int32_t head_dim,
                               int32_t num_blocks, int32_t block_size,
                               nkv_dtype_t dtype, hipStream_t stream);

/*
 * Per-head RMSNorm of q and k, rotary embedding by position, and the KV store, in one
 * pass over one layer's fused projection output (bf16 only).
 * 「Nano-vLLM深度解读（下）」 §2 (Qwen3Attention.forward: q, k, v split from the
 * projection; q_norm and k_norm over head_dim; rotary_emb(positions, q, k); attention,
 * which stores k and v first, §4); 「同一个 Qwen3，两种写法」 §3.5 (rotation of the two
 * halves by the cos/sin row of each position) and §3.6 (RMSNorm in float32).
 * For token t and every head x of q (weight q_norm_weight) and of k (k_norm_weight):
 *   n = bf16(x * rsqrt(mean(x*x) + eps)),  y = bf16(n * weight)     (float32 math)
 *   (c, s) = cos_sin_cache[positions[t]] halves;  y1, y2 = halves of y
 *   result = bf16(concat(y1*c - y2*s, y2*c + y1*s))
 * The rotated q goes to q_out[t]; the rotated k and the untouched v go to row
 * slot_mapping[t] of k_cache / v_cache (-1 skips the store, q_out is still written).
 *
 *   qkv            [num_tokens, (num_q_heads + 2*num_kv_heads) * head_dim] bf16: the q
 *                  heads, then the k heads, then the v heads of a token; rows
 *                  qkv_row_stride ELEMENTS apart (>= that width, a multiple of 8);
 *                  16-byte aligned.
 *   positions      [num_tokens] int32, each in [0, max_position).
 *   q_norm_weight, k_norm_weight   [head_dim] bf16, 16-byte aligned.
 *   cos_sin_cache  [max_position, head_dim] float32: head_dim/2 cosines, then the
 *                  head_dim/2 sines; 16-byte aligned.  A model constant the caller
 *                  builds once.
 *   eps            RMSNorm epsilon in [0, 1] (Qwen3: 1e-6).
 *   slot_mapping   [num_tokens] int32, as for nkv_store_kvcache.
 *   q_out          [num_tokens, num_q_heads, head_dim] bf16 contiguous, 16-byte aligned;
 *                  must not alias qkv.
 *   k_cache, v_cache  [num_blocks, block_size, num_kv_heads, head_dim] bf16, 16-byte
 *                  aligned.
 *   head_dim in {64, 128}; dtype must be NKV_BF16 (NKV_F32: NKV_ERR_UNSUPPORTED).
 * Preconditions checked in checking mode: positions in range, slots as for the store.
 * num_tokens == 0 is a no-op.
 */
nkv_status_t nkv_qk_norm_rope_store(const void* qkv, int64_t qkv_row_stride,
                                    const int32_t* positions, const void* q_norm_weight,
                                    const void* k_norm_weight, const float* cos_sin_cache,
                                    int32_t max_position, float eps,
                                    const int32_t* slot_mapping, int32_t num_tokens,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    void* q_out, void* k_cache, void* v_cache,
                                    int32_t num_blocks, int32_t block_size, nkv_dtype_t dtype,
                                    hipStream_t stream);

/*
 * Residual add + RMSNorm over token rows (bf16 only), the norm in front of each decoder
 * block's projections.  「同一个 Qwen3，两种写法」 §3.6 (add_rms_forward; the plain
 * RMSNorm when there is no residual).  For every row t, with float32 math:
 *   s = x[t] + residual[t]              (s = x[t] when residual is NULL)
 *   residual_out[t] = bf16(s)
 *   n = bf16(s * rsqrt(mean(s*s) + eps)),  out[t] = bf16(n * weight)
 * The norm is taken on the float32 sum, not on its bf16 copy.
 *
 *   x, residual    [num_tokens, hidden_size] bf16, contiguous rows, 16-byte aligned;
 *                  residual may be NULL (the first block).
 *   weight         [hidden_size] bf16, 16-byte aligned.
 *   eps            RMSNorm epsilon in [0, 1] (Qwen3: 1e-6).
 *   out            [num_tokens, hidden_size] bf16, 16-byte aligned.
 *   residual_out   [num_tokens, hidden_size] bf16, 16-byte aligned, or NULL (not written).
 *   hidden_size    a positive multiple of 8, at most 16384.
 * In place: out may be x and residual_out may be residual (the very same pointer);
 * any other overlap between an output and another buffer, and any overlap of out with
 * residual_out, is rejected with NKV_ERR_INVALID_ARG.  dtype must be NKV_BF16
 * (NKV_F32: NKV_ERR_UNSUPPORTED).  num_tokens == 0 is a no-op.
 */
nkv_status_t nkv_add_rms_norm(const void* x, const void* residual, const void* weight, float eps,
                              int32_t num_tokens, int32_t hidden_size, void* out,
                              void* residual_out, nkv_dtype_t dtype, hipStream_t stream);

/*
 * Causal varlen prefill attention over the paged pools.
 * 「同一个 Qwen3，两种写法」 §3.2 (flat [T, H, D] batch split by cu_seqlens, causal inside
 * each segment, nothing computed across segments) and §3.4 (GQA inside the kernel; K/V
 * read from the paged cache through the block table).  For sequence b:
 *   queries  q[cu_seqlens_q[b] .. cu_seqlens_q[b+1])            (Lq of them)
 *   keys     its first Lk = cu_seqlens_k[b+1]-cu_seqlens_k[b] positions in the pool,
 *            position p in block block_table[b*max_blocks_per_seq + p/block_size]
 *   query i (0-based) attends to keys j <= Lk - Lq + i (bottom-right alignment: a
 *   chunk of new tokens follows the cached prefix); Q head h uses KV head
 *   h / (num_q_heads/num_kv_heads).
 *   out[i, h, :] = sum_j softmax_j(softmax_scale * q_i.k_j) v_j, fp32 accumulation.
 *
 *   q           [total_q, num_q_heads, head_dim], rows q_row_stride elements apart
 *               (>= num_q_heads*head_dim, 16-byte aligned), same dtype as the pools.
 *   out         [total_q, num_q_heads, head_dim] contiguous, dtype of q.
 *   cu_seqlens_q, cu_seqlens_k  [num_seqs+1] int32;  block_table
 *               [num_seqs, max_blocks_per_seq] int32 (entries past a sequence's last
 *               block are never read).
 *   max_seqlen_q / max_seqlen_k: host upper bounds of Lq / Lk (size the grid).
 *   Supported: head_dim 64 or 128; num_q_heads/num_kv_heads in {1,2,4,8};
 *   block_size a power of two in [16, 1024]; bf16 (MFMA path) or fp32 (VALU path).
 */
nkv_status_t nkv_paged_attn_prefill(const void* q, int64_t q_row_stride,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    const int32_t* block_table, int32_t max_blocks_per_seq,
                                    int32_t num_seqs, int32_t total_q,
                                    int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t num_blocks, int32_t block_size,
                                    float softmax_scale, nkv_dtype_t dtype,
                                    void* out, hipStream_t stream);

/*
 * Causal varlen prefill over contiguous K/V: the branch without a prefix cache, where
 * attention reads the fresh k and v of this call instead of the pools.
 * 「Nano-vLLM深度解读（下）」 §4 (attention.py: flash_attn_varlen_func(q, k, v, ...) when
 * no block table is set); 「同一个 Qwen3，两种写法」 §3.2 (flat batch split by cu_seqlens).
 * Same operation as nkv_paged_attn_prefill, except that sequence b's keys are rows
 * cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of k and v.
 *
 *   q      [total_q, num_q_heads, head_dim], rows q_row_stride elements apart.
 *   k, v   [total_k, num_kv_heads, head_dim], rows k_row_stride / v_row_stride elements
 *          apart (>= num_kv_heads*head_dim; e.g. views of a packed qkv projection).
 *          Strides are multiples of 16 bytes; q, k, v, out 16-byte aligned.
 *   out    [total_q, num_q_heads, head_dim] contiguous, dtype of q; must not alias an input.
 *   cu_seqlens_q, cu_seqlens_k  [num_seqs+1] int32 running sums from 0, Lq <= Lk per
 *          sequence, cu_seqlens_q[num_seqs] = total_q, cu_seqlens_k[num_seqs] <= total_k.
 *   max_seqlen_q <= max_seqlen_k <= total_k: host upper bounds (size the grid).
 *   Supported: head_dim 64 or 128; num_q_heads/num_kv_heads in {1,2,4,8}; bf16 (MFMA
 *   path) or fp32 (VALU path).  num_seqs, total_q or max_seqlen_q == 0: a no-op.
 * Preconditions checked in checking mode: the cu_seqlens conditions above.
 */
nkv_status_t nkv_attn_varlen_prefill(const void* q, int64_t q_row_stride, const void* k,
                                     int64_t k_row_stride, const void* v, int64_t v_row_stride,
                                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                     int32_t num_seqs, int32_t total_q, int32_t total_k,
                                     int32_t max_seqlen_q, int32_t max_seqlen_k,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     float softmax_scale, nkv_dtype_t dtype, void* out,
                                     hipStream_t stream);

/*
 * Bytes of device workspace nkv_paged_attn_decode needs for these sizes (partial
 * results of sequences split over several workgroups).  Depends on the current
 * device's compute-unit count.
 */
size_t nkv_paged_attn_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t max_blocks_per_seq, int32_t block_size);

/*
 * Single-token decode attention over the paged pools.
 * 「Nano-vLLM深度解读（下）」 §4 and 「同一个 Qwen3，两种写法」 §3.4 (flash_attn_with_kvcache
 * with cache_seqlens and block_table): the one query of sequence b attends to all of
 * its context_lens[b] cached positions (which include the token stored just before
 * this call); Q head h uses KV head h / (num_q_heads/num_kv_heads).
 *
 *   q             [num_seqs, num_q_heads, head_dim] contiguous, pool dtype.
 *   context_lens  [num_seqs] int32, each in [1, max_blocks_per_seq*block_size].
 *   block_table   [num_seqs, max_blocks_per_seq] int32.
 *   out           [num_seqs, num_q_heads, head_dim] contiguous, dtype of q.
  *   workspace     device buffer of at least nkv_paged_attn_decode_workspace_size(...)
 *                 bytes, 16-byte aligned (may be NULL when that size is 0); its
 *                 contents on entry do not matter.  Calls that share a workspace must
 *                 be ordered on one stream.
 *   Work is split over workgroups by logical position: bf16 takes equal shares of
 *   (sequence, KV head, 16-position) rounds per workgroup ("stream-K"), fp32 fixed
 *   spans per sequence ("split-K").  A sequence cut by a split leaves partials (max,
 *   sum, weighted values) that are merged in a fixed order, so results are bitwise
 *   reproducible and do not depend on which physical blocks hold the data.  A second
 *   kernel merges the partials.
 *   Supported: as for prefill; bf16 uses MFMA, fp32 the VALU.
 */
nkv_status_t nkv_paged_attn_decode(const void* q,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* context_lens,
                                   const int32_t* block_table, int32_t max_blocks_per_seq,
                                   int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t num_blocks, int32_t block_size,
                                   float softmax_scale, nkv_dtype_t dtype,
                                   void* out, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/*
 * Size of the device scratch that nkv_paged_attn_decode_noalloc uses in place of a
 * workspace (a static device array: each device the library runs on holds one until the
 * process ends).
 */
#define NKV_DECODE_SCRATCH_BYTES (64u << 20)

/*
 * nkv_paged_attn_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same operation, arguments, kernels and results (bit for bit) as
 * nkv_paged_attn_decode; the partial results of split sequences go to the library's
 * static device scratch of NKV_DECODE_SCRATCH_BYTES bytes instead of a caller's buffer.
 *   - allocates nothing (no hipMalloc / hipFree, no allocating library call); the first
 *     call on a device looks up that device's scratch address once;
 *   - sizes whose workspace (nkv_paged_attn_decode_workspace_size) exceeds
 *     NKV_DECODE_SCRATCH_BYTES are rejected with NKV_ERR_WORKSPACE before anything is
 *     launched;
 *   - every call on one device shares that device's scratch, which keeps the last call's
 *     contents (the kernels need nothing cleared); calls that overlap on one device (other
 *     streams, other threads) race on it and must be ordered by the caller.
 */
nkv_status_t nkv_paged_attn_decode_noalloc(const void* q,
                                           const void* k_cache, const void* v_cache,
                                           const int32_t* context_lens,
                                           const int32_t* block_table, int32_t max_blocks_per_seq,
                                           int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t num_blocks, int32_t block_size,
                                           float softmax_scale, nkv_dtype_t dtype,
                                           void* out, hipStream_t stream);

/*
 * ---- The CPU block manager (host memory and host code only; no device calls) ----
 *
 * The control plane that feeds the calls above: it hands out the blocks of a pool of
 * num_blocks blocks of block_size slots, keeps a reference count per block, shares the
 * full blocks of equal prompt prefixes between sequences, and writes the index arrays
 * the data plane reads.  「Nano-vLLM深度解读（下）」 §4 (the CPU block manager: token
 * blocks with a hash and a reference count, block ids, prefix-cache reuse, the slot
 * mapping it provides); 「同一个 Qwen3，两种写法」 §3.3 (fixed-size blocks, block table
 * logical -> physical, slot = block * block_size + offset, equal prefixes sharing a
 * physical block by reference count and prefix hash).
 *
 * Rules where the pages stop: a full block's hash is 64-bit FNV-1a over the previous
 * block's hash (8 bytes little-endian, none for the first block) and its token ids (4
 * bytes each, little-endian), and a hit also compares the token ids; a new sequence
 * reuses its leading full blocks while they hit and always leaves at least one token to
 * compute; free blocks are a FIFO queue in which a released block keeps its hash (a later
 * prefix can revive it) until it is taken for new content; a newly hashed block becomes
 * the entry for its hash; a sequence's blocks are released in reverse order.  An
 * operation that needs more free blocks than there are returns NKV_ERR_NO_SPACE and
 * changes nothing.  Arrays are HOST arrays owned by the caller; a manager is not
 * thread-safe.  Errors set nkv_last_error() like every other call.
 */
typedef struct nkv_block_manager nkv_block_manager_t;

/* A manager over num_blocks blocks of block_size slots, all free (block ids 0..). */
nkv_status_t nkv_bm_create(int32_t num_blocks, int32_t block_size, nkv_block_manager_t** out);
void nkv_bm_destroy(nkv_block_manager_t* bm);
/* Number of free blocks (-1 for a null manager). */
int32_t nkv_bm_num_free_blocks(const nkv_block_manager_t* bm);

/* Admit sequence seq_id with its prompt token_ids[num_tokens] (num_tokens >= 1): reuse
 * the leading cached full blocks, take free blocks for the rest.  *num_cached_tokens
 * (may be NULL) receives the number of prompt tokens whose K/V is already in the pool. */
nkv_status_t nkv_bm_add_sequence(nkv_block_manager_t* bm, int64_t seq_id, const int32_t* token_ids,
                                 int32_t num_tokens, int32_t* num_cached_tokens);
/* Append one generated token (a new block when the last one is full; a block that
 * becomes full is hashed). */
nkv_status_t nkv_bm_append_token(nkv_block_manager_t* bm, int64_t seq_id, int32_t token_id);
/* Release a finished sequence's blocks. */
nkv_status_t nkv_bm_free_sequence(nkv_block_manager_t* bm, int64_t seq_id);

/* Index arrays of a prefill batch (the sequences' uncached prompt tokens as queries, all
 * their tokens as keys), for nkv_qk_norm_rope_store / nkv_store_kvcache and
 * nkv_paged_attn_prefill:
 *   cu_seqlens_q, cu_seqlens_k  [num_seqs + 1];
 *   positions, slot_mapping     [total_q], capacity = their length (if it is too small
 *                               the call fails and *total_q still gives the need);
 *   block_table                 [num_seqs, max_blocks_per_seq], -1 past each sequence's
 *                               blocks;
 *   total_q, max_seqlen_q, max_seqlen_k  outputs (may be NULL). */
nkv_status_t nkv_bm_prepare_prefill(const nkv_block_manager_t* bm, const int64_t* seq_ids, int32_t num_seqs,
                                    int32_t max_blocks_per_seq, int32_t capacity, int32_t* cu_seqlens_q,
                                    int32_t* cu_seqlens_k, int32_t* positions, int32_t* slot_mapping,
                                    int32_t* block_table, int32_t* total_q, int32_t* max_seqlen_q,
                                    int32_t* max_seqlen_k);
/* Index arrays of a decode step (each sequence's last token as the query):
 *   positions, slot_mapping, context_lens [num_seqs]; block_table as above. */
nkv_status_t nkv_bm_prepare_decode(const nkv_block_manager_t* bm, const int64_t* seq_ids, int32_t num_seqs,
                                   int32_t max_blocks_per_seq, int32_t* positions, int32_t* slot_mapping,
                                   int32_t* context_lens, int32_t* block_table);

/* Inspection (tests, debugging): a sequence's sizes; a block's reference count, hash
 * and whether it is free; the free queue front to back (returns its length, writes at
 * most capacity ids). */
nkv_status_t nkv_bm_sequence_info(const nkv_block_manager_t* bm, int64_t seq_id, int32_t* num_tokens,
                                  int32_t* num_cached_tokens, int32_t* num_blocks);
nkv_status_t nkv_bm_block_info(const nkv_block_manager_t* bm, int32_t block_id, int32_t* ref_count,
                               int32_t* is_hashed, uint64_t* hash, int32_t* is_free);
int32_t nkv_bm_free_queue(const nkv_block_manager_t* bm, int32_t* out, int32_t capacity);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* NKV_H */
