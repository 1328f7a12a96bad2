// Host-side block manager of the paged KV cache (declared in include/pkv.h):
// the free list of physical blocks, per-sequence block tables and lengths,
// reference counts for blocks shared between sequences, copy-on-write, and a
// cache of full blocks keyed by their token prefix.
//
// Bookkeeping rules ("PagedAttention Explained", "Implementing a Simplified
// Paged KV Cache"): a sequence takes a new block from the front of the free
// list when its length is a multiple of the block size, and its next token
// goes to row length % block_size of its last block; freeing a sequence drops
// its references and returns blocks with no reference left to the back of the
// free list.  Forked sequences share blocks (reference count > 1), and a
// sequence that writes into a shared last block first copies it to a block of
// its own ("Master Paged Attention for LLM Inference", "How Paged Attention
// Works: The Mechanics", item 4): the (source, destination) pairs are what
// pkv_copy_blocks takes.  Full blocks are also entered in a cache under a hash
// of every token up to their end, so a later prompt that starts with the same
// tokens reuses them instead of computing and storing them again ("Paged
// Attention" glossary, "Why it matters"; "PagedAttention Explained",
// "Enabling Automatic Prefix Caching").
//
// Plain C++ on the host; no HIP calls.  One manager is not thread-safe.
#include <cstdint>
#include <cstring>
#include <new>
#include <string>
#include <unordered_map>
#include <utility>
#include <vector>

#include "../../include/pkv.h"

namespace {

// 64-bit FNV-1a over 32-bit words, chained: the hash of a full block is taken
// over the previous block's hash and the block's token ids, so it names the
// whole prefix.  A hit is confirmed by comparing the block's own tokens and
// its parent's hash, so a hash collision between prefixes that also agree on
// those is the only way to a wrong reuse (probability ~2^-64 per lookup).
uint64_t fnv_step(uint64_t h, uint32_t w) {
  for (int i = 0; i < 4; ++i) {
    h ^= (w >> (8 * i)) & 0xffu;
    h *= 0x100000001b3ull;
  }
  return h;
}

uint64_t block_hash(uint64_t parent, const int32_t* tokens, int32_t n) {
  uint64_t h = 0xcbf29ce484222325ull;
  h = fnv_step(h, (uint32_t)parent);
  h = fnv_step(h, (uint32_t)(parent >> 32));
  for (int32_t i = 0; i < n; ++i) h = fnv_step(h, (uint32_t)tokens[i]);
  return h;
}

constexpr uint64_t kNoParent = 0x9e3779b97f4a7c15ull;  // hash standing for "before the first block"

struct Sequence {
  std::vector<int32_t> blocks;
  int32_t length = 0;
  // prefix caching: token ids of the sequence's unfinished last block and the
  // hash of the prefix before it; token_tracked turns off when a caller
  // appends without token ids (the block contents are then unknown)
  std::vector<int32_t> tail_tokens;
  uint64_t prefix_hash = kNoParent;
  bool token_tracked = true;
};

struct CachedBlock {
  int32_t block;
  uint64_t parent;
  std::vector<int32_t> tokens;
};

}  // namespace

struct pkv_block_manager {
  int32_t num_blocks;
  int32_t block_size;
  std::vector<int32_t> ref;
  // free list: intrusive doubly linked list in allocation order (head first)
  std::vector<int32_t> next, prev;
  std::vector<uint8_t> is_free;
  int32_t head = -1, tail = -1, free_count = 0;
  std::unordered_map<int64_t, Sequence> seqs;
  std::vector<std::pair<int32_t, int32_t>> copies;
  // prefix cache: hash -> entry, and block -> hash of its entry (to drop it when the block is reused)
  std::unordered_map<uint64_t, CachedBlock> cache;
  std::vector<uint64_t> cached_hash;
  std::vector<uint8_t> is_cached;
  std::string error;

  void push_free(int32_t b) {
    next[b] = -1;
    prev[b] = tail;
    if (tail >= 0) next[tail] = b;
    else head = b;
    tail = b;
    is_free[b] = 1;
    ++free_count;
  }
  void unlink_free(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b];
    else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b];
    else tail = prev[b];
    is_free[b] = 0;
    --free_count;
  }
  void uncache(int32_t b) {
    if (!is_cached[b]) return;
    cache.erase(cached_hash[b]);
    is_cached[b] = 0;
  }
  // a fresh block for new contents: the free list's front, dropped from the cache
  int32_t take() {
    const int32_t b = head;
    unlink_free(b);
    uncache(b);
    ref[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--ref[b] == 0) push_free(b);  // keeps its cache entry until the block is taken again
  }
  // enter a just-filled block of s in the cache (unless an identical prefix is there already)
  void register_full(Sequence& s, int32_t block) {
    const uint64_t h = block_hash(s.prefix_hash, s.tail_tokens.data(), (int32_t)s.tail_tokens.size());
    if (!cache.count(h) && !is_cached[block]) {
      cache.emplace(h, CachedBlock{block, s.prefix_hash, s.tail_tokens});
      cached_hash[block] = h;
      is_cached[block] = 1;
    }
    s.prefix_hash = h;
    s.tail_tokens.clear();
  }
};

namespace {

pkv_status bm_fail(pkv_block_manager* bm, pkv_status st, const char* msg) {
  if (bm) bm->error = msg;
  return st;
}

}  // namespace

extern "C" {

pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  pkv_block_manager* bm = new (std::nothrow) pkv_block_manager();
  if (!bm) return nullptr;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref.assign(num_blocks, 0);
  bm->next.assign(num_blocks, -1);
  bm->prev.assign(num_blocks, -1);
  bm->is_free.assign(num_blocks, 0);
  bm->cached_hash.assign(num_blocks, 0);
  bm->is_cached.assign(num_blocks, 0);
  if (free_order) {
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || bm->is_free[b]) {
        delete bm;
        return nullptr;  // not a permutation of 0..num_blocks-1
      }
      bm->push_free(b);
    }
  } else {
    for (int32_t b = 0; b < num_blocks; ++b) bm->push_free(b);
  }
  return bm;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

const char* pkv_bm_last_error(const pkv_block_manager* bm) { return bm ? bm->error.c_str() : "manager is NULL"; }

int32_t pkv_bm_num_free(const pkv_block_manager* bm) { return bm ? bm->free_count : -1; }

int32_t pkv_bm_ref_count(const pkv_block_manager* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[block];
}

int32_t pkv_bm_num_cached(const pkv_block_manager* bm) { return bm ? (int32_t)bm->cache.size() : -1; }

pkv_status pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq) {
  if (!bm) return PKV_EINVAL;
  if (bm->seqs.count(seq)) return bm_fail(bm, PKV_EINVAL, "sequence id already in use");
  bm->seqs.emplace(seq, Sequence());
  return PKV_OK;
}

pkv_status pkv_bm_add_sequence_cached(pkv_block_manager* bm, int64_t seq, const int32_t* tokens, int32_t num_tokens,
                                      int32_t* cached_tokens) {
  if (!bm || num_tokens < 0 || (num_tokens > 0 && !tokens) || !cached_tokens) return PKV_EINVAL;
  if (bm->seqs.count(seq)) return bm_fail(bm, PKV_EINVAL, "sequence id already in use");
  Sequence s;
  const int32_t bs = bm->block_size;
  // walk the prompt's full blocks while the cache holds them; the last prompt
  // token is never taken from the cache (its query is still to be computed)
  const int32_t reusable = num_tokens > 0 ? (num_tokens - 1) / bs : 0;
  for (int32_t k = 0; k < reusable; ++k) {
    const int32_t* blk_tokens = tokens + (int64_t)k * bs;
    const uint64_t h = block_hash(s.prefix_hash, blk_tokens, bs);
    auto it = bm->cache.find(h);
    if (it == bm->cache.end() || it->second.parent != s.prefix_hash ||
        std::memcmp(it->second.tokens.data(), blk_tokens, sizeof(int32_t) * bs) != 0)
      break;
    const int32_t b = it->second.block;
    if (bm->is_free[b]) bm->unlink_free(b);  // revived from the free list with its contents
    ++bm->ref[b];
    s.blocks.push_back(b);
    s.length += bs;
    s.prefix_hash = h;
  }
  *cached_tokens = s.length;
  bm->seqs.emplace(seq, std::move(s));
  return PKV_OK;
}

pkv_status pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm) return PKV_EINVAL;
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return bm_fail(bm, PKV_EINVAL, "unknown parent sequence");
  if (bm->seqs.count(child)) return bm_fail(bm, PKV_EINVAL, "child sequence id already in use");
  Sequence c = it->second;  // same blocks, length and prefix state
  for (int32_t b : c.blocks) ++bm->ref[b];
  bm->seqs.emplace(child, std::move(c));
  return PKV_OK;
}

pkv_status pkv_bm_append_tokens(pkv_block_manager* bm, int64_t seq, int32_t num_tokens, const int32_t* token_ids,
                                int32_t* slots) {
  if (!bm || num_tokens < 0 || (num_tokens > 0 && !slots)) return PKV_EINVAL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return bm_fail(bm, PKV_EINVAL, "unknown sequence");
  Sequence& s = it->second;
  const int32_t bs = bm->block_size;
  // blocks this call takes: new blocks at multiples of the block size, plus a
  // copy when the first write lands in a shared, partly filled last block
  int64_t need = 0;
  if (num_tokens > 0) {
    const int32_t row = s.length % bs;
    if (row != 0 && bm->ref[s.blocks.back()] > 1) ++need;
    const int64_t room = row == 0 ? 0 : bs - row;
    if (num_tokens > room) need += (num_tokens - room + bs - 1) / bs;
  }
  if (need > bm->free_count) return bm_fail(bm, PKV_ENOSPACE, "block pool exhausted: the sequence needs a new block");
  if ((int64_t)s.length + num_tokens > INT32_MAX) return bm_fail(bm, PKV_EINVAL, "sequence too long");
  if (!token_ids) s.token_tracked = false;
  for (int32_t i = 0; i < num_tokens; ++i) {
    const int32_t row = s.length % bs;
    if (row == 0) {
      s.blocks.push_back(bm->take());
    } else if (bm->ref[s.blocks.back()] > 1) {  // copy-on-write
      const int32_t src = s.blocks.back();
      const int32_t dst = bm->take();
      --bm->ref[src];
      s.blocks.back() = dst;
      bm->copies.emplace_back(src, dst);
    }
    slots[i] = s.blocks.back() * bs + row;
    ++s.length;
    if (s.token_tracked) {
      s.tail_tokens.push_back(token_ids[i]);
      if (s.length % bs == 0) bm->register_full(s, s.blocks.back());
    }
  }
  return PKV_OK;
}

int32_t pkv_bm_take_copies(pkv_block_manager* bm, int32_t* pairs, int32_t max_pairs) {
  if (!bm) return -1;
  const int32_t n = (int32_t)bm->copies.size();
  if (!pairs) return n;
  if (max_pairs < n) return -1;
  for (int32_t i = 0; i < n; ++i) {
    pairs[2 * i] = bm->copies[i].first;
    pairs[2 * i + 1] = bm->copies[i].second;
  }
  bm->copies.clear();
  return n;
}

pkv_status pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq) {
  if (!bm) return PKV_EINVAL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return bm_fail(bm, PKV_EINVAL, "unknown sequence");
  for (int32_t b : it->second.blocks) bm->release(b);
  bm->seqs.erase(it);
  return PKV_OK;
}

int32_t pkv_bm_sequence_length(const pkv_block_manager* bm, int64_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : it->second.length;
}

int32_t pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq, int32_t* table, int32_t max_blocks) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return -1;
  const int32_t n = (int32_t)it->second.blocks.size();
  if (table) {
    if (max_blocks < n) return -1;
    std::memcpy(table, it->second.blocks.data(), sizeof(int32_t) * n);
  }
  return n;
}

pkv_status pkv_bm_export_batch(pkv_block_manager* bm, const int64_t* seqs, int32_t num_seqs, int32_t max_blocks_per_seq,
                               int32_t pad, int32_t* block_tables, int32_t* context_lens) {
  if (!bm || num_seqs < 0 || max_blocks_per_seq <= 0 || (num_seqs > 0 && (!seqs || !block_tables || !context_lens)))
    return PKV_EINVAL;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return bm_fail(bm, PKV_EINVAL, "unknown sequence in the batch");
    if ((int32_t)it->second.blocks.size() > max_blocks_per_seq)
      return bm_fail(bm, PKV_EINVAL, "a sequence has more blocks than max_blocks_per_seq");
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Sequence& s = bm->seqs.find(seqs[i])->second;
    int32_t* row = block_tables + (int64_t)i * max_blocks_per_seq;
    const int32_t n = (int32_t)s.blocks.size();
    std::memcpy(row, s.blocks.data(), sizeof(int32_t) * n);
    for (int32_t j = n; j < max_blocks_per_seq; ++j) row[j] = pad;
    context_lens[i] = s.length;
  }
  return PKV_OK;
}

}  // extern "C"
