// The CPU block manager: the control plane that hands out the paged pool's blocks and
// produces the index arrays the data plane reads (block tables, slot mappings,
// cu_seqlens, context lengths, positions).
//
// 「Nano-vLLM深度解读（下）」 §4: the block manager runs on the CPU, manages the token
// sequences, allocates block ids, keeps reference counts and reuses cached prefixes; a
// CPU block holds token ids with a hash and a reference count and stands for one GPU
// block; the slot mapping it provides maps each token to a cache row.
// 「同一个 Qwen3，两种写法」 §3.3: fixed-size blocks allocated from a pool made once; a
// per-sequence block table maps logical to physical blocks; slot = physical block *
// block_size + offset; blocks carry a reference count and a prefix hash, so sequences
// with an equal prefix point at the same physical block.
//
// Where the pages stop, this is the design (the same rules as the Python reference used
// by the tests):
//   - a full block's hash is 64-bit FNV-1a over the previous block's hash (8 bytes,
//     little-endian; none for a sequence's first block) and the block's token ids (4
//     bytes each, little-endian), so it names the whole prefix; a hit also compares the
//     token ids; partial blocks have no hash;
//   - a new sequence reuses its leading full blocks while they hit, stops at the first
//     miss, and always leaves at least one token to compute;
//   - free blocks form a FIFO queue (an intrusive doubly linked list, so a cached block
//     can be taken out of the middle in O(1) when a prefix revives it); a released block
//     keeps its hash until it is taken for new content;
//   - a newly hashed full block becomes the table's entry for its hash;
//   - releasing a sequence returns its blocks in reverse table order;
//   - an operation that does not fit in the free blocks fails with NKV_ERR_NO_SPACE and
//     changes nothing.
// Host code only: no HIP calls.  A manager is not thread-safe; one owner drives it.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "nkv.h"
#include "status.hpp"

#define NKV_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr uint64_t kFnvOffset = 0xcbf29ce484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001b3ull;

uint64_t fnv_feed(uint64_t h, uint64_t value, int nbytes) {   // little-endian bytes of value
  for (int i = 0; i < nbytes; ++i) {
    h ^= (value >> (8 * i)) & 0xffu;
    h *= kFnvPrime;
  }
  return h;
}

uint64_t block_hash(bool has_prev, uint64_t prev, const int32_t* tokens, int32_t n) {
  uint64_t h = kFnvOffset;
  if (has_prev) h = fnv_feed(h, prev, 8);
  for (int32_t i = 0; i < n; ++i) h = fnv_feed(h, uint32_t(tokens[i]), 4);
  return h;
}

struct Block {
  int32_t ref = 0;
  bool hashed = false;
  uint64_t hash = 0;
  std::vector<int32_t> tokens;   // of a hashed (full) block
};

struct Seq {
  std::vector<int32_t> tokens;
  std::vector<int32_t> table;
  int32_t cached = 0;
};

nkv_status_t err(nkv_status_t st, const char* fmt, long long a = 0, long long b = 0) {
  char msg[256];
  snprintf(msg, sizeof(msg), fmt, a, b);
  return nkv::set_error(st, msg);
}

}  // namespace

struct nkv_block_manager {
  int32_t num_blocks, block_size;
  std::vector<Block> blocks;
  // free queue: head = next to take, tail = last released
  std::vector<int32_t> prev, next;
  std::vector<uint8_t> in_free;
  int32_t head = -1, tail = -1, nfree = 0;
  std::unordered_map<uint64_t, int32_t> by_hash;
  std::unordered_map<int64_t, Seq> seqs;

  nkv_block_manager(int32_t nb, int32_t bs)
      : num_blocks(nb), block_size(bs), blocks(nb), prev(nb, -1), next(nb, -1), in_free(nb, 0) {
    for (int32_t b = 0; b < nb; ++b) push_back(b);
  }

  void push_back(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    in_free[b] = 1;
    ++nfree;
  }
  void unlink(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    prev[b] = next[b] = -1;
    in_free[b] = 0;
    --nfree;
  }
  // the front free block, cleared for new content (its old hash entry dropped)
  int32_t take_front() {
    const int32_t b = head;
    unlink(b);
    Block& blk = blocks[b];
    if (blk.hashed) {
      auto it = by_hash.find(blk.hash);
      if (it != by_hash.end() && it->second == b) by_hash.erase(it);
    }
    blk.hashed = false;
    blk.tokens.clear();
    blk.ref = 1;
    return b;
  }
  void hash_block(int32_t b, uint64_t h, const int32_t* tokens) {
    Block& blk = blocks[b];
    blk.hashed = true;
    blk.hash = h;
    blk.tokens.assign(tokens, tokens + block_size);
    by_hash[h] = b;
  }
  int32_t slot(const Seq& s, int32_t pos) const {
    return s.table[pos / block_size] * block_size + pos % block_size;
  }
};

NKV_EXPORT nkv_status_t nkv_bm_create(int32_t num_blocks, int32_t block_size, nkv_block_manager_t** out) {
  if (!out) return err(NKV_ERR_INVALID_ARG, "null output pointer");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0) return err(NKV_ERR_INVALID_ARG, "num_blocks and block_size must be positive");
  if (int64_t(num_blocks) * block_size > int64_t(INT32_MAX))
    return err(NKV_ERR_UNSUPPORTED, "pool has more than 2^31-1 rows");
  *out = new (std::nothrow) nkv_block_manager(num_blocks, block_size);
  if (!*out) return err(NKV_ERR_INVALID_ARG, "out of host memory");
  return nkv::clear_error();
}

NKV_EXPORT void nkv_bm_destroy(nkv_block_manager_t* bm) { delete bm; }

NKV_EXPORT int32_t nkv_bm_num_free_blocks(const nkv_block_manager_t* bm) { return bm ? bm->nfree : -1; }

NKV_EXPORT nkv_status_t nkv_bm_add_sequence(nkv_block_manager_t* bm, int64_t seq_id, const int32_t* token_ids,
                                            int32_t num_tokens, int32_t* num_cached_tokens) {
  if (!bm) return err(NKV_ERR_INVALID_ARG, "null block manager");
  if (num_tokens <= 0 || !token_ids) return err(NKV_ERR_INVALID_ARG, "a prompt needs at least one token");
  if (bm->seqs.count(seq_id)) return err(NKV_ERR_INVALID_ARG, "sequence %lld already exists", seq_id);
  const int32_t bs = bm->block_size;
  const int32_t nblocks = (num_tokens + bs - 1) / bs, nfull = num_tokens / bs;
  // chained hashes of the full blocks, then the leading hits
  std::vector<uint64_t> hashes(nfull);
  for (int32_t i = 0; i < nfull; ++i)
    hashes[i] = block_hash(i > 0, i > 0 ? hashes[i - 1] : 0, token_ids + int64_t(i) * bs, bs);
  std::vector<int32_t> hits;
  for (int32_t i = 0; i < nfull; ++i) {
    auto it = bm->by_hash.find(hashes[i]);
    if (it == bm->by_hash.end()) break;
    const Block& blk = bm->blocks[it->second];
    if (memcmp(blk.tokens.data(), token_ids + int64_t(i) * bs, sizeof(int32_t) * bs) != 0) break;
    hits.push_back(it->second);
  }
  if (int64_t(hits.size()) * bs >= num_tokens) hits.pop_back();   // leave a token to compute
  int32_t revived = 0;
  for (int32_t b : hits) revived += bm->blocks[b].ref == 0;
  const int32_t need = nblocks - int32_t(hits.size());
  if (bm->nfree - revived < need)
    return err(NKV_ERR_NO_SPACE, "needs %lld free blocks, %lld available", need, bm->nfree - revived);
  Seq s;
  s.tokens.assign(token_ids, token_ids + num_tokens);
  s.table.reserve(nblocks);
  for (int32_t b : hits) {
    if (bm->blocks[b].ref == 0) bm->unlink(b);
    ++bm->blocks[b].ref;
    s.table.push_back(b);
  }
  for (int32_t i = int32_t(hits.size()); i < nblocks; ++i) {
    const int32_t b = bm->take_front();
    if (i < nfull) bm->hash_block(b, hashes[i], token_ids + int64_t(i) * bs);
    s.table.push_back(b);
  }
  s.cached = int32_t(hits.size()) * bs;
  if (num_cached_tokens) *num_cached_tokens = s.cached;
  bm->seqs.emplace(seq_id, std::move(s));
  return nkv::clear_error();
}

NKV_EXPORT nkv_status_t nkv_bm_append_token(nkv_block_manager_t* bm, int64_t seq_id, int32_t token_id) {
  if (!bm) return err(NKV_ERR_INVALID_ARG, "null block manager");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return err(NKV_ERR_INVALID_ARG, "no sequence %lld", seq_id);
  Seq& s = it->second;
  const int32_t bs = bm->block_size;
  if (s.tokens.size() >= size_t(INT32_MAX)) return err(NKV_ERR_UNSUPPORTED, "sequence too long");
  if (int32_t(s.tokens.size()) % bs == 0) {       // the new token starts a block
    if (bm->nfree == 0) return err(NKV_ERR_NO_SPACE, "no free block for sequence %lld", seq_id);
    s.table.push_back(bm->take_front());
  }
  s.tokens.push_back(token_id);
  const int32_t n = int32_t(s.tokens.size());
  if (n % bs == 0) {                               // its block is now full: hash it
    const int32_t i = n / bs - 1;
    const Block* prevb = i > 0 ? &bm->blocks[s.table[i - 1]] : nullptr;
    const uint64_t h = block_hash(prevb != nullptr, prevb ? prevb->hash : 0, s.tokens.data() + int64_t(i) * bs, bs);
    bm->hash_block(s.table[i], h, s.tokens.data() + int64_t(i) * bs);
  }
  return nkv::clear_error();
}

NKV_EXPORT nkv_status_t nkv_bm_free_sequence(nkv_block_manager_t* bm, int64_t seq_id) {
  if (!bm) return err(NKV_ERR_INVALID_ARG, "null block manager");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return err(NKV_ERR_INVALID_ARG, "no sequence %lld", seq_id);
  const std::vector<int32_t>& t = it->second.table;
  for (auto b = t.rbegin(); b != t.rend(); ++b)
    if (--bm->blocks[*b].ref == 0) bm->push_back(*b);
  bm->seqs.erase(it);
  return nkv::clear_error();
}

NKV_EXPORT nkv_status_t nkv_bm_sequence_info(const nkv_block_manager_t* bm, int64_t seq_id, int32_t* num_tokens,
                                             int32_t* num_cached_tokens, int32_t* num_blocks) {
  if (!bm) return err(NKV_ERR_INVALID_ARG, "null block manager");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return err(NKV_ERR_INVALID_ARG, "no sequence %lld", seq_id);
  if (num_tokens) *num_tokens = int32_t(it->second.tokens.size());
  if (num_cached_tokens) *num_cached_tokens = it->second.cached;
  if (num_blocks) *num_blocks = int32_t(it->second.table.size());
  return nkv::clear_error();
}

NKV_EXPORT nkv_status_t nkv_bm_block_info(const nkv_block_manager_t* bm, int32_t block_id, int32_t* ref_count,
                                          int32_t* is_hashed, uint64_t* hash, int32_t* is_free) {
  if (!bm) return err(NKV_ERR_INVALID_ARG, "null block manager");
  if (block_id < 0 || block_id >= bm->num_blocks) return err(NKV_ERR_INVALID_ARG, "block %lld out of range", block_id);
  const Block& blk = bm->blocks[block_id];
  if (ref_count) *ref_count = blk.ref;
  if (is_hashed) *is_hashed = blk.hashed;
  if (hash) *hash = blk.hash;
  if (is_free) *is_free = bm->in_free[block_id];
  return nkv::clear_error();
}

NKV_EXPORT int32_t nkv_bm_free_queue(const nkv_block_manager_t* bm, int32_t* out, int32_t capacity) {
  if (!bm) return -1;
  int32_t n = 0;
  for (int32_t b = bm->head; b >= 0; b = bm->next[b]) {
    if (out && n < capacity) out[n] = b;
    ++n;
  }
  return n;
}

namespace {

// the rows of the block table for a batch; -1 past each sequence's last block
nkv_status_t fill_tables(const nkv_block_manager_t* bm, const int64_t* seq_ids, int32_t num_seqs,
                         int32_t max_blocks, int32_t* block_table, std::vector<const Seq*>* seqs) {
  seqs->resize(num_seqs);
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return err(NKV_ERR_INVALID_ARG, "no sequence %lld", seq_ids[i]);
    const Seq& s = it->second;
    if (int32_t(s.table.size()) > max_blocks)
      return err(NKV_ERR_INVALID_ARG, "sequence %lld holds %lld blocks, more than max_blocks_per_seq",
                 seq_ids[i], int64_t(s.table.size()));
    (*seqs)[i] = &s;
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Seq& s = *(*seqs)[i];
    int32_t* row = block_table + int64_t(i) * max_blocks;
    const int32_t nb = int32_t(s.table.size());
    for (int32_t j = 0; j < max_blocks; ++j) row[j] = j < nb ? s.table[j] : -1;
  }
  return NKV_OK;
}

}  // namespace

NKV_EXPORT nkv_status_t nkv_bm_prepare_prefill(const nkv_block_manager_t* bm, const int64_t* seq_ids,
                                               int32_t num_seqs, int32_t max_blocks_per_seq, int32_t capacity,
                                               int32_t* cu_seqlens_q, int32_t* cu_seqlens_k, int32_t* positions,
                                               int32_t* slot_mapping, int32_t* block_table, int32_t* total_q,
                                               int32_t* max_seqlen_q, int32_t* max_seqlen_k) {
  if (!bm) return err(NKV_ERR_INVALID_ARG, "null block manager");
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || capacity < 0) return err(NKV_ERR_INVALID_ARG, "bad sizes");
  if (num_seqs > 0 && (!seq_ids || !cu_seqlens_q || !cu_seqlens_k || !block_table))
    return err(NKV_ERR_INVALID_ARG, "null pointer argument");
  std::vector<const Seq*> seqs;
  int64_t tq = 0, tk = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return err(NKV_ERR_INVALID_ARG, "no sequence %lld", seq_ids[i]);
    tq += int64_t(it->second.tokens.size()) - it->second.cached;
    tk += int64_t(it->second.tokens.size());
  }
  if (total_q) *total_q = int32_t(tq < INT32_MAX ? tq : INT32_MAX);
  if (tk > INT32_MAX) return err(NKV_ERR_UNSUPPORTED, "batch has more than 2^31-1 keys");
  if (tq > capacity) return err(NKV_ERR_INVALID_ARG, "positions / slot_mapping hold %lld, need %lld", capacity, tq);
  if (tq > 0 && (!positions || !slot_mapping)) return err(NKV_ERR_INVALID_ARG, "null pointer argument");
  nkv_status_t st = fill_tables(bm, seq_ids, num_seqs, max_blocks_per_seq, block_table, &seqs);
  if (st != NKV_OK) return st;
  int32_t mq = 0, mk = 0, q = 0;
  if (cu_seqlens_q) cu_seqlens_q[0] = 0;
  if (cu_seqlens_k) cu_seqlens_k[0] = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Seq& s = *seqs[i];
    const int32_t n = int32_t(s.tokens.size());
    for (int32_t p = s.cached; p < n; ++p, ++q) {
      positions[q] = p;
      slot_mapping[q] = bm->slot(s, p);
    }
    cu_seqlens_q[i + 1] = q;
    cu_seqlens_k[i + 1] = cu_seqlens_k[i] + n;
    mq = n - s.cached > mq ? n - s.cached : mq;
    mk = n > mk ? n : mk;
  }
  if (max_seqlen_q) *max_seqlen_q = mq;
  if (max_seqlen_k) *max_seqlen_k = mk;
  return nkv::clear_error();
}

NKV_EXPORT nkv_status_t nkv_bm_prepare_decode(const nkv_block_manager_t* bm, const int64_t* seq_ids,
                                              int32_t num_seqs, int32_t max_blocks_per_seq, int32_t* positions,
                                              int32_t* slot_mapping, int32_t* context_lens, int32_t* block_table) {
  if (!bm) return err(NKV_ERR_INVALID_ARG, "null block manager");
  if (num_seqs < 0 || max_blocks_per_seq <= 0) return err(NKV_ERR_INVALID_ARG, "bad sizes");
  if (num_seqs > 0 && (!seq_ids || !positions || !slot_mapping || !context_lens || !block_table))
    return err(NKV_ERR_INVALID_ARG, "null pointer argument");
  std::vector<const Seq*> seqs;
  nkv_status_t st = fill_tables(bm, seq_ids, num_seqs, max_blocks_per_seq, block_table, &seqs);
  if (st != NKV_OK) return st;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Seq& s = *seqs[i];
    const int32_t n = int32_t(s.tokens.size());
    positions[i] = n - 1;
    slot_mapping[i] = bm->slot(s, n - 1);
    context_lens[i] = n;
  }
  return nkv::clear_error();
}
