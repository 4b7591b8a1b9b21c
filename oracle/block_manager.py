"""Reference (oracle) for the CPU block manager that feeds the paged KV cache: block
allocation with reference counts, prefix sharing of full blocks by hash, and the index
arrays the data plane consumes (block tables, slot mappings, cu_seqlens, context lengths,
positions).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``; never by the product path.

What the pages fix:

* 「Nano-vLLM深度解读（下）」 §4: the block manager runs on the CPU, manages token
  sequences, hands out block ids, keeps reference counts and reuses cached prefixes; a
  CPU block carries a hash and a reference count and holds token ids; it corresponds one
  to one with a GPU block; the slot mapping it provides maps each token to a cache row.
* 「同一个 Qwen3，两种写法」 §3.3: the pool is allocated once in fixed-size blocks; each
  sequence has a block table (logical block -> physical block); slot = physical block *
  block_size + offset in the block; blocks carry a reference count and a prefix hash, so
  sequences with the same prefix point at the same physical block and its K/V is stored
  once.

Readings where the pages are silent:

* hash of a full block: 64-bit FNV-1a (Fowler/Noll/Vo, the published offset basis and
  prime) over the previous block's hash (8 bytes, little-endian; absent for a sequence's
  first block) followed by the block's token ids (4 bytes each, little-endian), so a hash
  names the block's whole prefix; a hit is confirmed by comparing the token ids;
  partially filled blocks have no hash;
* a new sequence reuses its leading full blocks while they hit and stops at the first
  miss; at least one token is always left to compute (if every block hits and the last is
  full, the last hit is dropped);
* free blocks form a FIFO queue: allocation takes the front, a block whose count drops to
  0 goes to the back with its hash kept, so a later prefix can revive it until the block
  is taken for new content (then its hash entry is dropped);
* when a full block is hashed, the hash table points at it (the latest block wins);
* freeing a sequence releases its blocks in reverse table order;
* an operation that needs more free blocks than there are fails and changes nothing.
"""

from __future__ import annotations

import struct

__all__ = ["FNV_OFFSET", "FNV_PRIME", "fnv1a64", "block_hash", "BlockManagerRef", "NoSpace"]

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
_MASK = (1 << 64) - 1


def fnv1a64(data: bytes) -> int:
    """64-bit FNV-1a: for each byte, xor it in, then multiply by the prime (mod 2^64)."""
    h = FNV_OFFSET
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & _MASK
    return h


def block_hash(prev_hash: int | None, tokens) -> int:
    data = b"" if prev_hash is None else struct.pack("<Q", prev_hash)
    data += b"".join(struct.pack("<i", int(t)) for t in tokens)
    return fnv1a64(data)


class NoSpace(Exception):
    pass


class _Block:
    def __init__(self):
        self.ref = 0
        self.hash = None          # int when the block is full and hashed
        self.tokens = None        # token ids of a hashed block


class BlockManagerRef:
    def __init__(self, num_blocks: int, block_size: int):
        self.bs = block_size
        self.blocks = [_Block() for _ in range(num_blocks)]
        self.free = list(range(num_blocks))   # FIFO: take from the front, return to the back
        self.by_hash = {}                     # hash -> block id
        self.seqs = {}                        # seq id -> dict(tokens, table, cached)

    # -- helpers --------------------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def _take_free(self) -> int:
        b = self.free.pop(0)
        blk = self.blocks[b]
        if blk.hash is not None and self.by_hash.get(blk.hash) == b:
            del self.by_hash[blk.hash]
        blk.hash, blk.tokens, blk.ref = None, None, 1
        return b

    def _register(self, b: int, h: int, tokens) -> None:
        blk = self.blocks[b]
        blk.hash, blk.tokens = h, list(tokens)
        self.by_hash[h] = b

    # -- operations -----------------------------------------------------------------
    def add_sequence(self, seq_id: int, tokens) -> int:
        """Admit a sequence with its prompt; returns the number of cached (reused) tokens."""
        if seq_id in self.seqs:
            raise ValueError("sequence exists")
        tokens = [int(t) for t in tokens]
        n, bs = len(tokens), self.bs
        if n == 0:
            raise ValueError("empty prompt")
        nblocks = -(-n // bs)
        # the chain of hashes of the full blocks
        hashes, prev = [], None
        for i in range(n // bs):
            prev = block_hash(prev, tokens[i * bs:(i + 1) * bs])
            hashes.append(prev)
        hits = []
        for i, h in enumerate(hashes):
            b = self.by_hash.get(h)
            if b is None or self.blocks[b].tokens != tokens[i * bs:(i + 1) * bs]:
                break
            hits.append(b)
        if len(hits) * bs >= n:           # leave at least one token to compute
            hits.pop()
        revived = sum(1 for b in hits if self.blocks[b].ref == 0)
        if len(self.free) - revived < nblocks - len(hits):
            raise NoSpace()
        table = []
        for b in hits:
            if self.blocks[b].ref == 0:
                self.free.remove(b)
            self.blocks[b].ref += 1
            table.append(b)
        for i in range(len(hits), nblocks):
            b = self._take_free()
            if i < len(hashes):
                self._register(b, hashes[i], tokens[i * bs:(i + 1) * bs])
            table.append(b)
        self.seqs[seq_id] = dict(tokens=tokens, table=table, cached=len(hits) * bs)
        return len(hits) * bs

    def append_token(self, seq_id: int, token: int) -> None:
        s = self.seqs[seq_id]
        n, bs = len(s["tokens"]), self.bs
        if n % bs == 0:                   # the new token starts a block
            if not self.free:
                raise NoSpace()
            s["table"].append(self._take_free())
        s["tokens"].append(int(token))
        n += 1
        if n % bs == 0:                   # its block is now full: hash it
            i = n // bs - 1
            prev = self.blocks[s["table"][i - 1]].hash if i > 0 else None
            self._register(s["table"][i], block_hash(prev, s["tokens"][i * bs:]), s["tokens"][i * bs:])

    def free_sequence(self, seq_id: int) -> None:
        s = self.seqs.pop(seq_id)
        for b in reversed(s["table"]):
            self.blocks[b].ref -= 1
            if self.blocks[b].ref == 0:
                self.free.append(b)

    # -- what the data plane consumes -----------------------------------------------
    def slot(self, seq_id: int, pos: int) -> int:
        t = self.seqs[seq_id]["table"]
        return t[pos // self.bs] * self.bs + pos % self.bs

    def prepare_prefill(self, seq_ids, max_blocks: int):
        """Uncached prompt tokens of each sequence as queries, all its tokens as keys."""
        cu_q, cu_k, pos, slots, table = [0], [0], [], [], []
        for sid in seq_ids:
            s = self.seqs[sid]
            n, c = len(s["tokens"]), s["cached"]
            cu_q.append(cu_q[-1] + n - c)
            cu_k.append(cu_k[-1] + n)
            for p in range(c, n):
                pos.append(p)
                slots.append(self.slot(sid, p))
            table.append(s["table"] + [-1] * (max_blocks - len(s["table"])))
        return dict(cu_seqlens_q=cu_q, cu_seqlens_k=cu_k, positions=pos, slot_mapping=slots,
                    block_table=table)

    def prepare_decode(self, seq_ids, max_blocks: int):
        """The last token of each sequence as the query; context length = its length."""
        pos, slots, lens, table = [], [], [], []
        for sid in seq_ids:
            s = self.seqs[sid]
            n = len(s["tokens"])
            pos.append(n - 1)
            slots.append(self.slot(sid, n - 1))
            lens.append(n)
            table.append(s["table"] + [-1] * (max_blocks - len(s["table"])))
        return dict(positions=pos, slot_mapping=slots, context_lens=lens, block_table=table)
