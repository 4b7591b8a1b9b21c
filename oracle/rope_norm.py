"""Reference (oracle) for the step right before the KV store in a Qwen3 attention layer
(per-head RMSNorm of q and k, rotary position embedding, then the store of k and v) and
for the residual add + RMSNorm in front of each decoder block's projections.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` (and, like ``ref``, allowed in
``__graft_entry__.smoke()`` and bench.py's ``cpu_baseline`` leg); never by the product
path.

What is computed, and where the pages define it:

* The order of operations -- 「Nano-vLLM深度解读（下）」 §2, ``Qwen3Attention.forward``:
  the fused projection output is split into q, k, v and viewed as ``[T, heads, head_dim]``;
  without a qkv bias, ``q_norm`` and ``k_norm`` (an ``RMSNorm`` over ``head_dim``, eps
  ``rms_norm_eps``) are applied to every head, then ``rotary_emb(positions, q, k)``, and
  ``attn(q, k, v)`` stores k and v into the cache before attending (same page, §4).
* ``rms_norm_ref`` -- the plain RMSNorm of 「同一个 Qwen3，两种写法」 §3.6 (the
  ``add_rms_forward`` listing without its residual part): the input is taken to float32,
  divided by the root of its mean square plus eps, cast back to the input dtype, and
  multiplied by the weight in that dtype.
* ``rope_cos_sin_table`` / ``apply_rope_ref`` -- 「同一个 Qwen3，两种写法」 §3.5: a table of
  ``max_position`` rows, each the cosines then the sines of ``position * inv_freq`` for the
  ``head_dim/2`` frequencies ``inv_freq[i] = base**(-2i/head_dim)``, looked up by position;
  the rotation splits a head into halves x1, x2 (in float32) and returns
  ``(x1*cos - x2*sin, x2*cos + x1*sin)`` cast back to the input dtype.
* ``qk_norm_rope_store_ref`` -- the composition, with the store of the rotated k and the
  untouched v through ``slot_mapping`` as in ``ref.store_ref``.
* ``add_rms_norm_ref`` -- the fused residual add + RMSNorm between decoder blocks,
  「同一个 Qwen3，两种写法」 §3.6 (``add_rms_forward``): hidden state and residual are added in
  float32, that sum cast to bf16 becomes the new residual, and the float32 sum (not its
  bf16 copy) is normalised, cast to bf16 and multiplied by the weight.  Without a
  residual (the first block) it is the plain RMSNorm of the hidden state and the hidden
  state itself is the residual.

Precision.  The listings fix it: norm and rotation run in float32 with a cast back to
bf16 after the normalisation, after the weight product and after the rotation.  This
oracle does exactly that with numpy float32 arithmetic and an explicit round-to-nearest-
even to bf16 at those three points.  Differences that remain against any other float32
implementation are the order of the mean's summation and the rounding of rsqrt and of
the rotation's products, which can move an output by a bf16 unit in rare cases.

The cos/sin table is a model constant that the caller supplies.  Here it is computed in
float64 and rounded once to float32 (the pages compute it in float32, whose position *
frequency products lose up to ~4e-3 rad at position 40960; a table is an input, so both
sides of a comparison see the same one).
"""

from __future__ import annotations

import numpy as np

from .ref import store_ref

__all__ = [
    "bf16_bits_to_f32",
    "f32_to_bf16_bits",
    "bf16_round",
    "rope_cos_sin_table",
    "rms_norm_ref",
    "apply_rope_ref",
    "qk_norm_rope_store_ref",
    "add_rms_norm_ref",
]


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 values (exact: bf16 is the top half)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, rounding to nearest, ties to even (NaN kept NaN)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    return np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), rounded)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """The float32 value of x rounded to bf16 (the ``.to(torch.bfloat16)`` cast)."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def rope_cos_sin_table(max_position: int, head_dim: int, base: float) -> np.ndarray:
    """[max_position, head_dim] float32: cos of position * inv_freq, then sin of it."""
    inv_freq = 1.0 / (float(base) ** (np.arange(0, head_dim, 2, dtype=np.float64) / head_dim))
    freqs = np.outer(np.arange(max_position, dtype=np.float64), inv_freq)
    return np.concatenate([np.cos(freqs), np.sin(freqs)], axis=1).astype(np.float32)


def rms_norm_ref(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis.  x and weight hold bf16 values (as float32); the result
    holds bf16 values (as float32)."""
    x = np.asarray(x, dtype=np.float32)
    var = np.mean(x * x, axis=-1, keepdims=True, dtype=np.float32)
    r = (np.float32(1.0) / np.sqrt(var + np.float32(eps))).astype(np.float32)
    normed = bf16_round(x * r)                                     # cast back to bf16
    return bf16_round(normed * np.asarray(weight, dtype=np.float32))   # bf16 product


def apply_rope_ref(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate the two halves of the last axis; x holds bf16 values, cos/sin float32 of
    shape broadcastable to x's halves.  Returns bf16 values (as float32)."""
    x = np.asarray(x, dtype=np.float32)
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    y1 = x1 * cos - x2 * sin
    y2 = x2 * cos + x1 * sin
    return bf16_round(np.concatenate([y1, y2], axis=-1).astype(np.float32))


def qk_norm_rope_store_ref(qkv_bits: np.ndarray, positions: np.ndarray, q_weight_bits: np.ndarray,
                           k_weight_bits: np.ndarray, cos_sin: np.ndarray, slot_mapping: np.ndarray,
                           k_pool_bits: np.ndarray, v_pool_bits: np.ndarray, num_q_heads: int,
                           num_kv_heads: int, eps: float):
    """One Qwen3 attention layer's q/k preparation and KV store, on bf16 bit patterns.

    qkv_bits: [T, (Hq + 2 Hkv) * D] uint16, the projection output (q heads, then k, then v).
    positions: [T] int, rows of cos_sin ([max_position, D] float32, cos half then sin half).
    Returns (q_out_bits [T, Hq, D], k_pool_bits', v_pool_bits').
    """
    t_count = qkv_bits.shape[0]
    hq, hkv = num_q_heads, num_kv_heads
    d = qkv_bits.shape[1] // (hq + 2 * hkv)
    x = bf16_bits_to_f32(qkv_bits.reshape(t_count, hq + 2 * hkv, d))
    q, k, v_bits = x[:, :hq], x[:, hq:hq + hkv], qkv_bits.reshape(t_count, hq + 2 * hkv, d)[:, hq + hkv:]
    table = np.asarray(cos_sin, dtype=np.float32)[np.asarray(positions, dtype=np.int64)]  # [T, D]
    cos, sin = table[:, None, : d // 2], table[:, None, d // 2:]
    q_rot = apply_rope_ref(rms_norm_ref(q, bf16_bits_to_f32(q_weight_bits), eps), cos, sin)
    k_rot = apply_rope_ref(rms_norm_ref(k, bf16_bits_to_f32(k_weight_bits), eps), cos, sin)
    k_new, v_new = store_ref(f32_to_bf16_bits(k_rot), np.ascontiguousarray(v_bits), k_pool_bits,
                             v_pool_bits, slot_mapping)
    return f32_to_bf16_bits(q_rot), k_new, v_new


def add_rms_norm_ref(x_bits: np.ndarray, residual_bits: np.ndarray | None, weight_bits: np.ndarray,
                     eps: float):
    """Residual add + RMSNorm over the last axis, on bf16 bit patterns.

    Returns (out_bits, residual_out_bits): out = bf16(bf16((x + r) * rsqrt(mean((x + r)^2) + eps))
    * weight) with the sum in float32, and residual_out = bf16(x + r).  With residual None the
    sum is x itself and residual_out is x.
    """
    x = bf16_bits_to_f32(x_bits)
    if residual_bits is None:
        s, resid = x, np.array(x_bits, dtype=np.uint16, copy=True)
    else:
        s = (x + bf16_bits_to_f32(residual_bits)).astype(np.float32)
        resid = f32_to_bf16_bits(s)
    var = np.mean(s * s, axis=-1, keepdims=True, dtype=np.float32)
    r = (np.float32(1.0) / np.sqrt(var + np.float32(eps))).astype(np.float32)
    normed = bf16_round(s * r)
    out = bf16_round(normed * bf16_bits_to_f32(weight_bits))
    return f32_to_bf16_bits(out), resid
