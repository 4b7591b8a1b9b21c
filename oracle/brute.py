"""Brute-force checker for the oracle: no paging, no online softmax, an explicit mask.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Tiny inputs only: it builds
the full ``[T, T]`` mask that the flat layout is designed to avoid.

It follows the other way of writing the same model that 「同一个 Qwen3，两种写法」
contrasts with the paged engine:
  * K/V of each sequence are contiguous, appended the way the transformers dynamic
    cache concatenates new keys and values (§3.3);
  * KV heads are expanded to the Q head count with ``repeat_kv`` (§3.4): a
    ``[B, Hkv, S, D]`` tensor gets a new axis after the head axis, is broadcast
    ``n_rep`` times along it and reshaped to ``[B, Hkv*n_rep, S, D]``;
  * the flat batch uses one ``[Tq, Tk]`` mask that is block diagonal across
    sequences and lower triangular inside each block (§3.2 worked 7x7 example);
  * softmax is a dense row softmax with masked entries at -inf.
"""

from __future__ import annotations

import numpy as np

__all__ = ["append_kv", "repeat_kv", "varlen_causal_mask", "brute_attention"]


def append_kv(cache: np.ndarray | None, new: np.ndarray) -> np.ndarray:
    """Contiguous cache update by concatenation along the sequence axis (axis 0)."""
    return new.copy() if cache is None else np.concatenate([cache, new], axis=0)


def repeat_kv(x: np.ndarray, n_rep: int) -> np.ndarray:
    """[B, Hkv, S, D] -> [B, Hkv*n_rep, S, D] by broadcasting a new axis after heads."""
    if n_rep == 1:
        return x
    b, hkv, s, d = x.shape
    expanded = np.broadcast_to(x[:, :, None, :, :], (b, hkv, n_rep, s, d))
    return expanded.reshape(b, hkv * n_rep, s, d)


def varlen_causal_mask(seqlens_q, seqlens_k) -> np.ndarray:
    """Boolean [sum(seqlens_q), sum(seqlens_k)] mask, True = visible.

    Sequence b's query rows and key columns form a diagonal block; inside it query
    i (of Lq) sees key j (of Lk) when j <= Lk - Lq + i.  Everything off the
    diagonal blocks is False.
    """
    tq, tk = int(np.sum(seqlens_q)), int(np.sum(seqlens_k))
    mask = np.zeros((tq, tk), dtype=bool)
    r0 = c0 = 0
    for lq, lk in zip(seqlens_q, seqlens_k):
        lq, lk = int(lq), int(lk)
        for i in range(lq):
            for j in range(lk):
                if j <= lk - lq + i:
                    mask[r0 + i, c0 + j] = True
        r0 += lq
        c0 += lk
    return mask


def brute_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                    seqlens_q, seqlens_k, scale: float) -> np.ndarray:
    """Dense masked attention over the whole flat batch.

    q : [Tq, Hq, D] float64; k, v : [Tk, Hkv, D] float64, each sequence's keys
    contiguous and in order.  Returns [Tq, Hq, D].
    """
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    n_rep = hq // hkv
    # [1, Hkv, Tk, D] -> [1, Hq, Tk, D]
    k4 = repeat_kv(np.transpose(k, (1, 0, 2))[None], n_rep)[0]
    v4 = repeat_kv(np.transpose(v, (1, 0, 2))[None], n_rep)[0]
    mask = varlen_causal_mask(seqlens_q, seqlens_k)
    out = np.zeros((tq, hq, d), dtype=np.float64)
    for h in range(hq):
        scores = scale * (q[:, h, :] @ k4[h].T)             # [Tq, Tk]
        scores = np.where(mask, scores, -np.inf)
        for i in range(tq):
            row = scores[i]
            if not mask[i].any():
                continue
            w = np.exp(row - row.max())
            w = w / w.sum()
            out[i, h] = w @ v4[h]
    return out
