"""Seeded synthetic inputs for the paged KV-cache data plane.

This module only PRODUCES inputs: lengths, physical-block permutations, block tables,
slot mappings, ``cu_seqlens``, ``context_lens`` and N(0,1) tensors.  It holds none of
the store or attention arithmetic, so both the HIP path and the CPU oracle can take
their inputs from it without sharing any of the method.

What the index arrays mean comes from the pages:
  * ``block_table[b, i]`` is the physical block that holds logical block ``i`` of
    sequence ``b``; K/V may sit anywhere in the pool (「同一个 Qwen3，两种写法」 §3.3).
  * ``slot_mapping[t]`` is the cache row of new token ``t``: physical block *
    block_size + offset inside the block, computed on the CPU by the block manager
    (same section); -1 means "do not store" (「Nano-vLLM深度解读（下）」 §4).
  * ``cu_seqlens`` are the running sums of sequence lengths over the flat ``[T, H, D]``
    batch, e.g. lengths 300/400/255 give [0, 300, 700, 955] (「同一个 Qwen3，两种写法」
    §3.2).
  * Head shapes follow Qwen3-8B: 32 Q heads, 8 KV heads, head_dim 128, 36 layers,
    bf16, max position 40960 (「同一个 Qwen3，两种写法」 §2); nano-vLLM uses 256-token
    blocks (§2.2).

Recipe (all configs): ``numpy.random.default_rng(258000 + k)`` draws lengths and
permutations for config number ``k``; a ``torch.Generator`` seeded with
``258000 + k`` (per layer: ``(258000 + k) * 100 + layer``) draws fp32 N(0,1) values on
the target device, cast to bf16 by round-to-nearest-even where the config is bf16.
Pool rows that no sequence has written yet are filled with NaN, so any kernel that
reads them (or multiplies them by a zero weight) poisons its output.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

SEED_BASE = 258000

# --------------------------------------------------------------------------------------
# block-manager stand-ins (CPU control plane inputs)
# --------------------------------------------------------------------------------------


def cu_seqlens(lengths) -> np.ndarray:
    """Boundaries of a flat varlen batch: [0, l0, l0+l1, ...] as int32."""
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return out.astype(np.int32)


def blocks_needed(length: int, block_size: int) -> int:
    return -(-int(length) // int(block_size))


def slots_for_positions(table_row, positions, block_size: int) -> np.ndarray:
    """Cache rows of logical positions of one sequence (the block manager's formula)."""
    positions = np.asarray(positions, dtype=np.int64)
    table_row = np.asarray(table_row, dtype=np.int64)
    phys = table_row[positions // block_size]
    if (phys < 0).any():
        raise ValueError("position maps to an unassigned logical block")
    return (phys * block_size + positions % block_size).astype(np.int32)


def assign_blocks(rng: np.random.Generator, nblocks_per_seq, num_blocks: int,
                  max_blocks_per_seq: int) -> np.ndarray:
    """Give each sequence its blocks from one random permutation of the pool.

    Returns block_table [B, max_blocks_per_seq] int32, unused entries -1.
    """
    perm = rng.permutation(num_blocks)
    table = np.full((len(nblocks_per_seq), max_blocks_per_seq), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(nblocks_per_seq):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    if pos > num_blocks:
        raise ValueError("pool too small for the requested sequences")
    return table


# --------------------------------------------------------------------------------------
# value generation
# --------------------------------------------------------------------------------------

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def randn(shape, gen: torch.Generator, device, dtype: str) -> torch.Tensor:
    """fp32 N(0,1) drawn with ``gen``, then cast (RNE) to the config's element type."""
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x if dtype == "f32" else x.to(TORCH_DTYPE[dtype])


def randn_into(dst: torch.Tensor, gen: torch.Generator, chunk_elems: int = 1 << 28) -> None:
    """Fill a (large) tensor with N(0,1) in bounded chunks of fp32 temporaries."""
    flat = dst.view(-1)
    for s in range(0, flat.numel(), chunk_elems):
        e = min(flat.numel(), s + chunk_elems)
        flat[s:e] = torch.randn(e - s, generator=gen, device=dst.device, dtype=torch.float32)


def nan_pool(num_blocks, block_size, hkv, d, dtype: str, device) -> torch.Tensor:
    return torch.full((num_blocks, block_size, hkv, d), float("nan"),
                      dtype=TORCH_DTYPE[dtype], device=device)


def _torch_gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


# --------------------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------------------


@dataclass(frozen=True)
class Shape:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str                      # "f32" or "bf16"

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


QWEN3_8B = Shape(32, 8, 128, 256, "bf16")
TINY = Shape(4, 1, 64, 16, "f32")


@dataclass
class PrefillCase:
    """One store + prefill call: new tokens are stored, then attention reads the pool."""
    name: str
    shape: Shape
    q: torch.Tensor                 # [Tq, Hq, D]
    k: torch.Tensor                 # [Tq, Hkv, D] new keys (one per query token)
    v: torch.Tensor
    slot_mapping: np.ndarray        # [Tq] int32
    k_cache: torch.Tensor           # [nb, bs, Hkv, D] pool before this call's store
    v_cache: torch.Tensor
    block_table: np.ndarray         # [B, max_blocks] int32
    cu_seqlens_q: np.ndarray        # [B+1] int32
    cu_seqlens_k: np.ndarray        # [B+1] int32
    meta: dict = field(default_factory=dict)

    @property
    def max_seqlen_q(self) -> int:
        return int(np.max(np.diff(self.cu_seqlens_q))) if len(self.cu_seqlens_q) > 1 else 0

    @property
    def max_seqlen_k(self) -> int:
        return int(np.max(np.diff(self.cu_seqlens_k))) if len(self.cu_seqlens_k) > 1 else 0


@dataclass
class DecodeCase:
    """One (optional) store of the new tokens + one decode call."""
    name: str
    shape: Shape
    q: torch.Tensor                 # [B, Hq, D]
    k: torch.Tensor | None          # [B, Hkv, D] new token K (None: nothing to store)
    v: torch.Tensor | None
    slot_mapping: np.ndarray | None # [B] int32
    k_cache: torch.Tensor           # pool before the store
    v_cache: torch.Tensor
    block_table: np.ndarray         # [B, max_blocks] int32
    context_lens: np.ndarray        # [B] int32, includes the stored token
    meta: dict = field(default_factory=dict)


def _fill_cached(pool: torch.Tensor, gen: torch.Generator, slots: np.ndarray) -> None:
    """Write N(0,1) rows at the given cache rows (the history already in the pool)."""
    nb, bs, hkv, d = pool.shape
    rows = pool.view(nb * bs, hkv * d)
    vals = torch.randn((len(slots), hkv * d), generator=gen, device=pool.device,
                       dtype=torch.float32).to(pool.dtype)
    idx = torch.as_tensor(slots.astype(np.int64), device=pool.device)
    rows.index_copy_(0, idx, vals)


# ---- C1: tiny fp32 -------------------------------------------------------------------

def c1_tiny(device="cpu", lengths=(37, 300), num_blocks=64, seed_k=1, shape=TINY):
    """Tiny paged case: prefill of both sequences, then one decode step each.

    Returns (prefill_case, decode_case).  The decode case's pool is the pool AFTER the
    prefill store; callers that chain store -> prefill -> store -> decode on the device
    must take the decode store's input pool from their own previous step.
    """
    rng = np.random.default_rng(SEED_BASE + seed_k)
    gen = _torch_gen(device, SEED_BASE + seed_k)
    bs, hq, hkv, d = shape.block_size, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    final = [l + 1 for l in lengths]                      # after the decode token
    nblk = [blocks_needed(l, bs) for l in final]
    table = assign_blocks(rng, nblk, num_blocks, max(nblk))
    t = int(sum(lengths))
    q = randn((t, hq, d), gen, device, shape.dtype)
    k = randn((t, hkv, d), gen, device, shape.dtype)
    v = randn((t, hkv, d), gen, device, shape.dtype)
    slots = np.concatenate([slots_for_positions(table[b], np.arange(l), bs)
                            for b, l in enumerate(lengths)])
    pre = PrefillCase("C1-prefill", shape, q, k, v, slots,
                      nan_pool(num_blocks, bs, hkv, d, shape.dtype, device),
                      nan_pool(num_blocks, bs, hkv, d, shape.dtype, device),
                      table, cu_seqlens(lengths), cu_seqlens(lengths))
    bsz = len(lengths)
    dq = randn((bsz, hq, d), gen, device, shape.dtype)
    dk = randn((bsz, hkv, d), gen, device, shape.dtype)
    dv = randn((bsz, hkv, d), gen, device, shape.dtype)
    dslots = np.array([slots_for_positions(table[b], [lengths[b]], bs)[0]
                       for b in range(bsz)], dtype=np.int32)
    dec = DecodeCase("C1-decode", shape, dq, dk, dv, dslots, None, None, table,
                     np.asarray(final, dtype=np.int32))
    return pre, dec


# ---- C2: Qwen3-8B single-layer decode ------------------------------------------------

def c2_decode(device="cpu", batch=64, len_lo=512, len_hi=4096, seed_k=2, shape=QWEN3_8B,
              extra_nan_block=False):
    """Batch decode: context lengths U{len_lo..len_hi} including the new token.

    The history (positions < L-1) is N(0,1); the new token's row and everything past
    it is NaN until the store writes the new token at position L-1.
    With ``extra_nan_block`` one more all-NaN block is appended to the pool and every
    unused block-table entry points at it.
    """
    rng = np.random.default_rng(SEED_BASE + seed_k)
    gen = _torch_gen(device, SEED_BASE + seed_k)
    bs, hq, hkv, d = shape.block_size, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    lens = rng.integers(len_lo, len_hi + 1, size=batch).astype(np.int32)
    nblk = [blocks_needed(l, bs) for l in lens]
    max_blk = blocks_needed(len_hi, bs)
    nb = int(sum(nblk))
    table = assign_blocks(rng, nblk, nb, max_blk)
    pool_blocks = nb + (1 if extra_nan_block else 0)
    if extra_nan_block:
        table[table < 0] = nb
    kc = nan_pool(pool_blocks, bs, hkv, d, shape.dtype, device)
    vc = nan_pool(pool_blocks, bs, hkv, d, shape.dtype, device)
    hist = np.concatenate([slots_for_positions(table[b], np.arange(lens[b] - 1), bs)
                           for b in range(batch)])
    _fill_cached(kc, gen, hist)
    _fill_cached(vc, gen, hist)
    q = randn((batch, hq, d), gen, device, shape.dtype)
    k = randn((batch, hkv, d), gen, device, shape.dtype)
    v = randn((batch, hkv, d), gen, device, shape.dtype)
    slots = np.array([slots_for_positions(table[b], [lens[b] - 1], bs)[0]
                      for b in range(batch)], dtype=np.int32)
    return DecodeCase("C2-decode", shape, q, k, v, slots, kc, vc, table, lens,
                      meta={"sum_context": int(lens.sum()), "num_blocks": pool_blocks})


# ---- C3: varlen causal prefill -------------------------------------------------------

def c3_prefill(device="cpu", num_seqs=8, seqlen=2048, seed_k=3, shape=QWEN3_8B):
    rng = np.random.default_rng(SEED_BASE + seed_k)
    gen = _torch_gen(device, SEED_BASE + seed_k)
    bs, hq, hkv, d = shape.block_size, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    nblk = [blocks_needed(seqlen, bs)] * num_seqs
    nb = int(sum(nblk))
    table = assign_blocks(rng, nblk, nb, nblk[0])
    t = num_seqs * seqlen
    q = randn((t, hq, d), gen, device, shape.dtype)
    k = randn((t, hkv, d), gen, device, shape.dtype)
    v = randn((t, hkv, d), gen, device, shape.dtype)
    slots = np.concatenate([slots_for_positions(table[b], np.arange(seqlen), bs)
                            for b in range(num_seqs)])
    cu = cu_seqlens([seqlen] * num_seqs)
    return PrefillCase("C3-prefill", shape, q, k, v, slots,
                       nan_pool(nb, bs, hkv, d, shape.dtype, device),
                       nan_pool(nb, bs, hkv, d, shape.dtype, device),
                       table, cu, cu.copy())


# ---- C4: prefix-cached chunked prefill -----------------------------------------------

def c4_prefix_chunk(device="cpu", num_seqs=16, prefix_blocks=4, chunk=512, seed_k=4,
                    shape=QWEN3_8B):
    """Shared block-aligned prefix (stored once) + a private chunk per sequence.

    Returns (prefix_store, case): ``prefix_store`` = (k, v, slot_mapping) of the
    one-off prefix store that must precede the case's own store.
    """
    rng = np.random.default_rng(SEED_BASE + seed_k)
    gen = _torch_gen(device, SEED_BASE + seed_k)
    bs, hq, hkv, d = shape.block_size, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    prefix = prefix_blocks * bs
    private = blocks_needed(prefix + chunk, bs) - prefix_blocks
    nb = prefix_blocks + num_seqs * private
    perm = rng.permutation(nb)
    shared = perm[:prefix_blocks]
    table = np.full((num_seqs, prefix_blocks + private), -1, dtype=np.int32)
    for b in range(num_seqs):
        table[b, :prefix_blocks] = shared
        table[b, prefix_blocks:] = perm[prefix_blocks + b * private:
                                        prefix_blocks + (b + 1) * private]
    pk = randn((prefix, hkv, d), gen, device, shape.dtype)
    pv = randn((prefix, hkv, d), gen, device, shape.dtype)
    pslots = slots_for_positions(table[0], np.arange(prefix), bs)
    t = num_seqs * chunk
    q = randn((t, hq, d), gen, device, shape.dtype)
    k = randn((t, hkv, d), gen, device, shape.dtype)
    v = randn((t, hkv, d), gen, device, shape.dtype)
    slots = np.concatenate([slots_for_positions(table[b], prefix + np.arange(chunk), bs)
                            for b in range(num_seqs)])
    case = PrefillCase("C4-prefix-chunk", shape, q, k, v, slots,
                       nan_pool(nb, bs, hkv, d, shape.dtype, device),
                       nan_pool(nb, bs, hkv, d, shape.dtype, device),
                       table, cu_seqlens([chunk] * num_seqs),
                       cu_seqlens([prefix + chunk] * num_seqs),
                       meta={"prefix_tokens": prefix, "shared_blocks": shared.tolist()})
    return (pk, pv, pslots), case


# ---- C5: long-context and mixed decode over 36 layers --------------------------------

NUM_LAYERS = 36


@dataclass
class MultiLayerDecode:
    """Layer-by-layer decode: every layer has its own pools and block tables."""
    name: str
    shape: Shape
    context_lens: np.ndarray
    layers: list                    # [(q, k_cache, v_cache, block_table)]
    meta: dict = field(default_factory=dict)


def c5_lengths(kind: str, seed: int):
    """Context lengths of C5a/C5b and the rng, positioned for the block permutations."""
    rng = np.random.default_rng(seed)
    if kind == "a":
        return np.full(4, 40960, dtype=np.int32), rng
    lens = np.rint(np.exp(rng.uniform(math.log(128), math.log(32768), size=256)))
    return lens.astype(np.int32), rng


def c5_decode(kind: str, device="cpu", layers=None, seed_k=None, shape=QWEN3_8B,
              max_blocks_per_seq=None):
    """C5a (kind "a": 4 x 40960) or C5b (kind "b": 256 log-uniform in [128, 32768]).

    ``layers`` selects which of the 36 layers to materialise (default: all).  The
    pool is pre-filled up to ``context_lens`` (no store in this config); rows past a
    sequence's length are NaN.
    """
    if seed_k is None:
        seed_k = 5 if kind == "a" else 6
    seed = SEED_BASE + seed_k
    lens, rng = c5_lengths(kind, seed)
    bs, hq, hkv, d = shape.block_size, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    nblk = [blocks_needed(l, bs) for l in lens]
    nb = int(sum(nblk))
    if max_blocks_per_seq is None:
        max_blocks_per_seq = 160 if kind == "a" else 128
    layer_ids = range(NUM_LAYERS) if layers is None else layers
    tables = [assign_blocks(rng, nblk, nb, max_blocks_per_seq) for _ in range(NUM_LAYERS)]
    out = []
    for layer in layer_ids:
        gen = _torch_gen(device, seed * 100 + layer)
        table = tables[layer]
        kc = torch.empty((nb, bs, hkv, d), dtype=TORCH_DTYPE[shape.dtype], device=device)
        vc = torch.empty_like(kc)
        randn_into(kc, gen)
        randn_into(vc, gen)
        for b, l in enumerate(lens):
            tail = int(l) % bs
            if tail:
                blk = int(table[b, nblk[b] - 1])
                kc[blk, tail:] = float("nan")
                vc[blk, tail:] = float("nan")
        q = randn((len(lens), hq, d), gen, device, shape.dtype)
        out.append((q, kc, vc, table))
    return MultiLayerDecode(f"C5{kind}-decode", shape, lens, out,
                            meta={"num_blocks": nb, "sum_context": int(lens.sum()),
                                  "layers": list(layer_ids), "seed": seed})


# --------------------------------------------------------------------------------------
# residual add + RMSNorm rows
# --------------------------------------------------------------------------------------

QWEN3_8B_HIDDEN = 4096


def norm_rows(num_tokens: int, hidden: int = QWEN3_8B_HIDDEN, seed: int = 6, device="cpu",
              with_residual: bool = True):
    """Inputs of one residual add + RMSNorm call: (x, residual or None, weight), bf16.

    x is a block output: N(0, 1) times a per-token scale drawn log-uniformly in [1e-2, 30];
    the residual stream is N(0, 1) times a per-token scale log-uniform in [1e-1, 1e2] (it
    grows over the layers); the weight is 1 + 0.1 N(0, 1).  Everything is drawn from one
    seeded generator on ``device``.
    """
    gen = _torch_gen(device, seed)
    def scale(lo, hi):
        u = torch.rand((num_tokens, 1), generator=gen, device=device, dtype=torch.float32)
        return torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
    x = (randn((num_tokens, hidden), gen, device, "f32") * scale(1e-2, 30.0)).to(torch.bfloat16)
    r = None
    if with_residual:
        r = (randn((num_tokens, hidden), gen, device, "f32") * scale(1e-1, 1e2)).to(torch.bfloat16)
    w = (1.0 + 0.1 * randn((hidden,), gen, device, "f32")).to(torch.bfloat16)
    return x, r, w
