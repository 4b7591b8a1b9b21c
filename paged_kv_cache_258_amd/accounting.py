"""Algorithmic work of each call: the bytes or flop the method must move or compute.

These are the roofline numerators.  They count what the operation itself needs:
no split-K workspace traffic, no masked or padded work, no re-reads.

Sizing on the pages that pins the byte unit (「同一个 Qwen3，两种写法」 §2.2): K and V
of one token over all 36 layers of Qwen3-8B (8 KV heads, head_dim 128, bf16) take
2 * 36 * 8 * 128 * 2 = 147,456 bytes; a 256-token block is 36 MiB; a 40960-token
context is about 6.0 GB.  Per layer that is 4096 B per token and 1 MiB per block.
"""

from __future__ import annotations

import numpy as np


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K plus V of one token across ``num_layers`` layers."""
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def store_bytes(slot_mapping, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Read K and V rows of stored tokens, write them to the pool, read every slot."""
    slots = np.asarray(slot_mapping)
    written = int((slots != -1).sum())
    return 4 * written * num_kv_heads * head_dim * elem_bytes + 4 * len(slots)


def decode_bytes(context_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 block_size: int, elem_bytes: int) -> int:
    """K/V of every cached position, q in, out back, context_lens and block ids."""
    lens = np.asarray(context_lens, dtype=np.int64)
    nblk = int(((lens + block_size - 1) // block_size).sum())
    b = len(lens)
    return (2 * elem_bytes * num_kv_heads * head_dim * int(lens.sum())
            + 2 * b * num_q_heads * head_dim * elem_bytes
            + 4 * (b + nblk))


def prefill_pairs(cu_seqlens_q, cu_seqlens_k) -> int:
    """Unmasked (query, key) pairs per Q head, bottom-right causal in each segment."""
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    lq = np.diff(cq)
    lk = np.diff(ck)
    return int((lq * (lk - lq) + lq * (lq + 1) // 2).sum())


def prefill_flops(cu_seqlens_q, cu_seqlens_k, num_q_heads: int, head_dim: int) -> int:
    """2*D flop for q.k and 2*D for p*v, per unmasked pair and Q head."""
    return 4 * head_dim * num_q_heads * prefill_pairs(cu_seqlens_q, cu_seqlens_k)


def prefill_min_bytes(cu_seqlens_q, cu_seqlens_k, num_q_heads: int, num_kv_heads: int,
                      head_dim: int, elem_bytes: int) -> int:
    """q read once, out written once, each sequence's K/V read once."""
    tq = int(np.asarray(cu_seqlens_q)[-1])
    tk = int(np.asarray(cu_seqlens_k)[-1])
    return (2 * tq * num_q_heads * head_dim * elem_bytes
            + 2 * tk * num_kv_heads * head_dim * elem_bytes)


def qk_norm_rope_store_bytes(slot_mapping, num_q_heads: int, num_kv_heads: int, head_dim: int,
                             elem_bytes: int) -> int:
    """Read every token's q, k, v heads, its position and slot and its cos/sin row (fp32),
    the two norm weights once; write q back and k, v of the tokens that have a slot."""
    slots = np.asarray(slot_mapping)
    t = len(slots)
    written = int((slots != -1).sum())
    return (t * (num_q_heads + 2 * num_kv_heads) * head_dim * elem_bytes   # q, k, v in
            + t * (4 + 4 + head_dim * 4)                                  # position, slot, table row
            + 2 * head_dim * elem_bytes                                   # weights
            + t * num_q_heads * head_dim * elem_bytes                     # q out
            + written * 2 * num_kv_heads * head_dim * elem_bytes)         # k, v rows stored


def add_rms_norm_bytes(num_tokens: int, hidden_size: int, elem_bytes: int, with_residual: bool = True) -> int:
    """Fused residual add + RMSNorm: read the hidden state and the residual, write the
    normalised output and the new residual (the weight vector once).  Without a residual:
    read the hidden state, write the output."""
    row = hidden_size * elem_bytes
    per_token = 4 * row if with_residual else 2 * row
    return num_tokens * per_token + row
