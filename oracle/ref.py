"""Reference (oracle) definition of the paged KV-cache data plane, in numpy float64.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py``; never by the product path.

What is computed, and where the pages define it:

* ``store_ref`` -- the KV store.  「Nano-vLLM深度解读（下）」 §4, ``attention.py``
  listing, ``store_kvcache_kernel`` / ``store_kvcache``: one program per new token
  reads its slot from ``slot_mapping``, does nothing when the slot is -1, and
  otherwise copies the token's ``num_kv_heads*head_dim`` key (and value) elements
  to row ``slot`` of the cache viewed as rows of that width.  The slot itself is
  "physical block * block_size + offset in block" (「同一个 Qwen3，两种写法」 §3.3).
* ``gather`` -- reading a sequence's K/V back through its block table: logical
  block ``p // block_size`` maps to a physical block id (「同一个 Qwen3，两种写法」
  §3.3, the per-sequence page table).
* ``attn`` -- causal softmax attention of one sequence with grouped KV heads.
  Scores are ``scale * q.k`` (the ``softmax_scale`` argument, ``head_dim**-0.5`` in
  the model, 「Nano-vLLM深度解读（下）」 §2 ``Qwen3Attention``), masked entries get
  weight exactly zero (「同一个 Qwen3，两种写法」 §1.2), Q head ``h`` reads KV head
  ``h // (Hq/Hkv)`` (the ``repeat_kv`` grouping, §3.4).
* ``prefill_ref`` -- ``flash_attn_varlen_func(..., causal=True, block_table=...)``
  over the flat ``[T, H, D]`` batch split by ``cu_seqlens_q/k``
  (「同一个 Qwen3，两种写法」 §3.2 and §3.4; 「Nano-vLLM深度解读（下）」 §4).
* ``decode_ref`` -- ``flash_attn_with_kvcache(q.unsqueeze(1), ..., cache_seqlens=
  context_lens, block_table=...)``: one query per sequence against its cached
  keys (same sources).  Written as its own loop, independent of ``prefill_ref``.
* ``varlen_prefill_ref`` -- the branch without a prefix cache,
  ``flash_attn_varlen_func(q, k, v, cu_seqlens_q/k, ..., causal=True)`` with the
  fresh k and v (「Nano-vLLM深度解读（下）」 §4: no block table when nothing is
  cached): sequence ``b``'s keys are rows ``cu_seqlens_k[b]..cu_seqlens_k[b+1]`` of
  the flat ``[Tk, Hkv, D]`` k and v (「同一个 Qwen3，两种写法」 §3.2).

Readings where the pages are silent, each with its reason:
  * causal alignment when a chunk has fewer queries than keys: bottom-right --
    query ``i`` of a segment with ``Lq`` queries and ``Lk`` keys sits at absolute
    position ``Lk - Lq + i`` and sees keys ``j <= Lk - Lq + i``;
  * ``context_lens`` includes the token stored just before the decode call
    (store-before-read, 「同一个 Qwen3，两种写法」 §3.4);
  * slot values other than -1 outside ``[0, num_blocks*block_size)`` and duplicate
    slots in one call are precondition violations: the oracle raises.

Precision: values are upcast exactly to float64 (bf16 and fp32 are both exact in
fp64); all arithmetic is float64.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "as_f64",
    "store_ref",
    "gather",
    "attn",
    "prefill_ref",
    "varlen_prefill_ref",
    "decode_ref",
]


# --------------------------------------------------------------------------------------
# element decoding
# --------------------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 values given as their raw 16-bit patterns.

    A bfloat16 is the upper half of an IEEE-754 binary32: sign, 8 exponent bits and
    7 fraction bits.  Putting the 16 bits back in the top half of a 32-bit word and
    reading that word as binary32 recovers the value exactly; binary32 -> binary64
    is exact as well.
    """
    b = np.ascontiguousarray(bits).view(np.uint16)
    with np.errstate(invalid="ignore"):            # signalling NaN patterns stay NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def as_f64(x: np.ndarray, elem: str) -> np.ndarray:
    """Exact float64 view of stored elements: ``elem`` is "f32" or "bf16" (raw bits)."""
    if elem == "bf16":
        return bf16_bits_to_f64(x)
    if elem == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if elem == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown element type {elem!r}")


# --------------------------------------------------------------------------------------
# store (scatter through slot_mapping)
# --------------------------------------------------------------------------------------

def store_ref(key: np.ndarray, value: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
              slot_mapping: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Return copies of the pools with the new K/V rows written.

    key, value   : [N, Hkv, D]   (any element type; copied bit for bit)
    k_pool/v_pool: [num_blocks, block_size, Hkv, D]
    slot_mapping : [N] integers; -1 = skip this token.

    Token ``t`` with ``slot_mapping[t] = s != -1`` overwrites row ``s`` of the pool
    viewed as ``[num_blocks*block_size, Hkv*D]``; every other row keeps its bytes.
    """
    n = key.shape[0]
    if value.shape != key.shape:
        raise ValueError("key and value shapes differ")
    if len(slot_mapping) != n:
        raise ValueError("slot_mapping must have one entry per token")
    nb, bs, hkv, d = k_pool.shape
    if key.shape[1:] != (hkv, d) or v_pool.shape != k_pool.shape:
        raise ValueError("pool / token shapes disagree")
    k_new = k_pool.copy()
    v_new = v_pool.copy()
    k_rows = k_new.reshape(nb * bs, hkv * d)
    v_rows = v_new.reshape(nb * bs, hkv * d)
    seen: set[int] = set()
    for t in range(n):
        s = int(slot_mapping[t])
        if s == -1:
            continue
        if s < 0 or s >= nb * bs:
            raise ValueError(f"slot {s} of token {t} outside [0, {nb * bs})")
        if s in seen:
            raise ValueError(f"slot {s} written twice in one call")
        seen.add(s)
        k_rows[s] = key[t].reshape(hkv * d)
        v_rows[s] = value[t].reshape(hkv * d)
    return k_new, v_new


# --------------------------------------------------------------------------------------
# reading a sequence back through its block table
# --------------------------------------------------------------------------------------

def gather(pool: np.ndarray, table_row: np.ndarray, length: int) -> np.ndarray:
    """Logical positions ``0..length-1`` of one sequence, as ``[length, Hkv, D]``.

    Position ``p`` lives in physical block ``table_row[p // block_size]`` at offset
    ``p % block_size``.  Table entries past ``ceil(length / block_size)`` are not read.
    """
    nb, bs = pool.shape[0], pool.shape[1]
    pos = np.arange(length)
    blocks = np.asarray(table_row)[pos // bs].astype(np.int64)
    bad = (blocks < 0) | (blocks >= nb)
    if bad.any():
        p = int(pos[bad][0])
        raise ValueError(f"block id {int(blocks[bad][0])} for position {p} outside [0, {nb})")
    return pool[blocks, pos % bs]


# --------------------------------------------------------------------------------------
# attention of one sequence
# --------------------------------------------------------------------------------------

def attn(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
         return_probs: bool = False):
    """Causal GQA attention of one sequence, float64.

    q : [Lq, Hq, D]   queries, the last Lq positions of the sequence
    k : [Lk, Hkv, D]  keys of positions 0..Lk-1 (Lk >= Lq)
    v : [Lk, Hkv, D]
    Returns o [Lq, Hq, D] (and, if asked, the probability matrices [Hq, Lq, Lk]).

    Query row ``i`` is absolute position ``Lk - Lq + i`` and may attend to keys
    ``j <= Lk - Lq + i``; other keys get weight exactly 0.
    """
    lq, hq, d = q.shape
    lk, hkv, _ = k.shape
    if lk < lq:
        raise ValueError("a segment needs at least as many keys as queries")
    if hq % hkv != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    group = hq // hkv
    o = np.zeros((lq, hq, d), dtype=np.float64)
    probs = np.zeros((hq, lq, lk), dtype=np.float64) if return_probs else None
    if lq == 0:
        return (o, probs) if return_probs else o
    # visible[i, j] is True when key j is allowed for query row i
    visible = np.arange(lk)[None, :] <= (lk - lq + np.arange(lq))[:, None]
    for h in range(hq):
        g = h // group
        s = scale * (q[:, h, :] @ k[:, g, :].T)          # [Lq, Lk]
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.where(visible, np.exp(s - m), 0.0)
        p = e / e.sum(axis=1, keepdims=True)
        o[:, h, :] = p @ v[:, g, :]
        if return_probs:
            probs[h] = p
    return (o, probs) if return_probs else o


# --------------------------------------------------------------------------------------
# varlen prefill over the paged pool
# --------------------------------------------------------------------------------------

def prefill_ref(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                cu_seqlens_q: np.ndarray, cu_seqlens_k: np.ndarray,
                block_table: np.ndarray, scale: float, elem: str = "f64") -> np.ndarray:
    """Paged causal varlen prefill.

    q            : [Tq, Hq, D] (element type ``elem``)
    k_pool/v_pool: [num_blocks, block_size, Hkv, D] (element type ``elem``)
    cu_seqlens_q : [B+1], cu_seqlens_k : [B+1]
    block_table  : [B, max_blocks_per_seq]
    Returns float64 out [Tq, Hq, D]: sequence b's queries are rows
    ``cu_q[b]:cu_q[b+1]`` and its keys are its first ``cu_k[b+1]-cu_k[b]`` positions.
    """
    tq, hq, d = q.shape
    out = np.zeros((tq, hq, d), dtype=np.float64)
    nseq = len(cu_seqlens_q) - 1
    for b in range(nseq):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        lk = int(cu_seqlens_k[b + 1]) - int(cu_seqlens_k[b])
        if q1 == q0:
            continue
        kb = as_f64(gather(k_pool, block_table[b], lk), elem)
        vb = as_f64(gather(v_pool, block_table[b], lk), elem)
        out[q0:q1] = attn(as_f64(q[q0:q1], elem), kb, vb, scale)
    return out


def varlen_prefill_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens_q: np.ndarray,
                       cu_seqlens_k: np.ndarray, scale: float, elem: str = "f64") -> np.ndarray:
    """Causal varlen prefill over contiguous K/V (no block table).

    q    : [Tq, Hq, D];  k, v : [Tk, Hkv, D] (element type ``elem``)
    Sequence b's queries are rows ``cu_q[b]:cu_q[b+1]`` of q and its keys rows
    ``cu_k[b]:cu_k[b+1]`` of k and v.  Returns float64 out [Tq, Hq, D].
    """
    tq, hq, d = q.shape
    out = np.zeros((tq, hq, d), dtype=np.float64)
    for b in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
        if q1 == q0:
            continue
        out[q0:q1] = attn(as_f64(q[q0:q1], elem), as_f64(k[k0:k1], elem), as_f64(v[k0:k1], elem), scale)
    return out


# --------------------------------------------------------------------------------------
# single-token decode over the paged pool
# --------------------------------------------------------------------------------------

def decode_ref(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
               context_lens: np.ndarray, block_table: np.ndarray, scale: float,
               elem: str = "f64", seqs=None) -> np.ndarray:
    """Paged decode: one query per sequence attends to all of its cached keys.

    q            : [B, Hq, D]
    context_lens : [B], number of cached positions including the token just stored
    seqs         : optional iterable of sequence indices to compute (others stay 0);
                   used to check sampled outputs of large batches.
    Returns float64 out [B, Hq, D].
    """
    nseq, hq, d = q.shape
    hkv = k_pool.shape[2]
    if hq % hkv != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    group = hq // hkv
    out = np.zeros((nseq, hq, d), dtype=np.float64)
    for b in (range(nseq) if seqs is None else seqs):
        length = int(context_lens[b])
        if length < 1:
            raise ValueError("decode needs at least one cached key")
        kb = as_f64(gather(k_pool, block_table[b], length), elem)   # [L, Hkv, D]
        vb = as_f64(gather(v_pool, block_table[b], length), elem)
        qb = as_f64(q[b], elem)                                     # [Hq, D]
        for h in range(hq):
            g = h // group
            s = scale * (kb[:, g, :] @ qb[h])                       # [L]
            w = np.exp(s - s.max())
            out[b, h] = (w / w.sum()) @ vb[:, g, :]
    return out
