// Host block manager behind the C ABI (pkv_bm_*).
//
// [SMTS] "Sub-Millisecond Token Scheduling: Inside Disaggregated KV-Cache
// Paging for Frontier LLMs", section "Paged KV-Cache with Radix Tree Prefix
// Cache": physical blocks carry a reference count; a slot allocation pops a
// block from the free pool, increments its count and appends it to the
// sequence's block list; an empty pool is an error that calls for preemption.
// Sequences sharing a prefix reference the same blocks through copy-on-write
// pointers. The allocation rules below fix what the page leaves open; they
// are stated in pkv.h.
//
// Prefix cache ([LLMI] "LLM inference: prefill, decode, KV cache", "8. Design
// Alternatives": a hash prefix cache over paged blocks and an LRU radix tree
// over paged blocks): a radix tree whose nodes are full blocks keyed under
// their parent by their token ids. match_prefix shares the longest cached
// chain with a new sequence; cache_prefix registers a sequence's blocks; a
// cached block released to count 0 stays (evictable) and revives on a match;
// an empty free pool evicts the least recently used unreferenced leaf.
#include <cstdint>
#include <new>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pkv.h"

struct pkv_bm {
  int32_t block_size;
  std::vector<int32_t> free_pool;                       // top of stack = back()
  std::vector<int32_t> ref;                             // per physical block
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t len = 0;
    bool swapped = false;                               // blocks live on the host
  };
  std::unordered_map<int64_t, Seq> seqs;

  // ---- prefix cache
  struct Key {
    int32_t parent;                    // -1: the root
    std::vector<int32_t> tokens;       // block_size token ids
    bool operator==(const Key& o) const { return parent == o.parent && tokens == o.tokens; }
  };
  struct KeyHash {
    size_t operator()(const Key& k) const {
      uint64_t h = 1469598103934665603ull ^ static_cast<uint32_t>(k.parent);
      for (int32_t t : k.tokens) h = (h ^ static_cast<uint32_t>(t)) * 1099511628211ull;
      return static_cast<size_t>(h);
    }
  };
  static constexpr int32_t kNotCached = -2;
  std::unordered_map<Key, int32_t, KeyHash> children;
  std::vector<int32_t> cached_parent;  // per block: kNotCached, -1 (root) or parent block
  std::vector<Key> cached_key;
  std::vector<int32_t> n_children;     // cached children of a cached block
  std::vector<uint64_t> stamp;         // last use
  uint64_t clock = 0;
  int32_t n_cached = 0;
  std::set<std::pair<uint64_t, int32_t>> evictable;   // (stamp, block) of idle cached leaves

  bool cached(int32_t b) const { return cached_parent[b] != kNotCached; }
  bool idle_leaf(int32_t b) const { return cached(b) && ref[b] == 0 && n_children[b] == 0; }
  // keeps `evictable` equal to the idle cached leaves; call after any change
  // to a block's count, children, stamp or cache membership
  void update(int32_t b) {
    evictable.erase({stamp[b], b});
    if (idle_leaf(b)) evictable.insert({stamp[b], b});
  }
  void tick(int32_t b) {
    evictable.erase({stamp[b], b});
    stamp[b] = ++clock;
    update(b);
  }
  void uncache(int32_t b) {
    evictable.erase({stamp[b], b});
    children.erase(cached_key[b]);
    const int32_t parent = cached_parent[b];
    cached_parent[b] = kNotCached;
    cached_key[b] = Key{};
    n_children[b] = 0;
    n_cached -= 1;
    if (parent >= 0) {
      n_children[parent] -= 1;
      update(parent);
    }
  }

  bool pop(int32_t* blk) {
    if (free_pool.empty()) {
      if (evictable.empty()) return false;
      *blk = evictable.begin()->second;          // least recently used idle leaf
      uncache(*blk);
      ref[*blk] += 1;
      return true;
    }
    *blk = free_pool.back();
    free_pool.pop_back();
    ref[*blk] += 1;
    return true;
  }

  void release(int32_t b) {
    ref[b] -= 1;
    if (ref[b] == 0) {
      if (cached(b))
        tick(b);                                 // stays cached, now evictable
      else
        free_pool.push_back(b);
    }
  }

  // blocks that repeated leaf evictions could free (swap-in admission)
  int64_t reclaimable() const {
    std::vector<int32_t> kids(n_children);
    std::vector<int32_t> stack;
    for (const auto& e : evictable) stack.push_back(e.second);
    int64_t n = 0;
    while (!stack.empty()) {
      const int32_t b = stack.back();
      stack.pop_back();
      n += 1;
      const int32_t parent = cached_parent[b];
      if (parent >= 0 && --kids[parent] == 0 && ref[parent] == 0) stack.push_back(parent);
    }
    return n;
  }
};

extern "C" {

pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size, pkv_bm** out) {
  if (!out || num_blocks < 0 || block_size <= 0) return PKV_ERR_INVALID_ARG;
  pkv_bm* bm = new (std::nothrow) pkv_bm();
  if (!bm) return PKV_ERR_INVALID_ARG;
  bm->block_size = block_size;
  bm->free_pool.resize(num_blocks);
  for (int32_t i = 0; i < num_blocks; ++i) bm->free_pool[i] = i;
  bm->ref.assign(num_blocks, 0);
  bm->cached_parent.assign(num_blocks, pkv_bm::kNotCached);
  bm->cached_key.resize(num_blocks);
  bm->n_children.assign(num_blocks, 0);
  bm->stamp.assign(num_blocks, 0);
  *out = bm;
  return PKV_OK;
}

void pkv_bm_destroy(pkv_bm* bm) { delete bm; }

pkv_status pkv_bm_append_slot(pkv_bm* bm, int64_t seq, int64_t* slot, int32_t* cow_src,
                              int32_t* cow_dst) {
  if (!bm || !slot || !cow_src || !cow_dst) return PKV_ERR_INVALID_ARG;
  auto found = bm->seqs.find(seq);
  if (found != bm->seqs.end() && found->second.swapped) return PKV_ERR_INVALID_ARG;
  const bool created = found == bm->seqs.end();
  auto& s = bm->seqs[seq];
  const int64_t pos = s.len;
  const int32_t bs = bm->block_size;
  int32_t src = -1, dst = -1;
  if (pos % bs == 0) {
    int32_t blk;
    if (!bm->pop(&blk)) {
      if (created) bm->seqs.erase(seq);                 // exhaustion changes nothing
      return PKV_ERR_OUT_OF_BLOCKS;
    }
    s.blocks.push_back(blk);
  } else {
    const int32_t last = s.blocks.back();
    if (bm->ref[last] > 1) {
      int32_t fresh;
      if (!bm->pop(&fresh)) return PKV_ERR_OUT_OF_BLOCKS;
      bm->ref[last] -= 1;                               // still >= 1: stays referenced
      s.blocks.back() = fresh;
      src = last;
      dst = fresh;
    }
  }
  s.len = pos + 1;
  *slot = static_cast<int64_t>(s.blocks.back()) * bs + pos % bs;
  *cow_src = src;
  *cow_dst = dst;
  return PKV_OK;
}

pkv_status pkv_bm_fork(pkv_bm* bm, int64_t parent, int64_t child) {
  if (!bm) return PKV_ERR_INVALID_ARG;
  auto p = bm->seqs.find(parent);
  if (p == bm->seqs.end() || p->second.swapped || bm->seqs.count(child))
    return PKV_ERR_INVALID_ARG;
  pkv_bm::Seq copy = p->second;
  for (int32_t blk : copy.blocks) bm->ref[blk] += 1;
  bm->seqs.emplace(child, std::move(copy));
  return PKV_OK;
}

pkv_status pkv_bm_free(pkv_bm* bm, int64_t seq) {
  if (!bm) return PKV_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PKV_ERR_INVALID_ARG;
  for (int32_t blk : it->second.blocks) bm->release(blk);
  bm->seqs.erase(it);
  return PKV_OK;
}

pkv_status pkv_bm_export_table(const pkv_bm* bm, const int64_t* seqs, int32_t B,
                               int32_t max_blocks, int32_t* host_table) {
  if (!bm || B < 0 || max_blocks < 0 || (B > 0 && (!seqs || !host_table)))
    return PKV_ERR_INVALID_ARG;
  for (int32_t b = 0; b < B; ++b) {
    auto it = bm->seqs.find(seqs[b]);
    const std::vector<int32_t>* blocks = it == bm->seqs.end() ? nullptr : &it->second.blocks;
    const int32_t n = blocks ? static_cast<int32_t>(blocks->size()) : 0;
    if (n > max_blocks) return PKV_ERR_INVALID_ARG;
    if (it != bm->seqs.end() && it->second.swapped) return PKV_ERR_INVALID_ARG;
  }
  for (int32_t b = 0; b < B; ++b) {
    auto it = bm->seqs.find(seqs[b]);
    int32_t* row = host_table + static_cast<int64_t>(b) * max_blocks;
    int32_t n = 0;
    if (it != bm->seqs.end()) {
      for (int32_t blk : it->second.blocks) row[n++] = blk;
    }
    for (; n < max_blocks; ++n) row[n] = 0;
  }
  return PKV_OK;
}

pkv_status pkv_bm_swap_out(pkv_bm* bm, int64_t seq, int32_t* blocks_out, int32_t capacity,
                           int32_t* n_blocks) {
  if (!bm || !n_blocks) return PKV_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end() || it->second.swapped) return PKV_ERR_INVALID_ARG;
  auto& s = it->second;
  const int32_t n = static_cast<int32_t>(s.blocks.size());
  *n_blocks = n;
  if (!blocks_out) return PKV_OK;                       // size query, no change
  if (capacity < n) return PKV_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) {
    blocks_out[i] = s.blocks[i];
    bm->release(s.blocks[i]);
  }
  s.blocks.clear();
  s.swapped = true;
  return PKV_OK;
}

pkv_status pkv_bm_swap_in(pkv_bm* bm, int64_t seq, int32_t* blocks_out, int32_t capacity,
                          int32_t* n_blocks) {
  if (!bm || !n_blocks) return PKV_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end() || !it->second.swapped) return PKV_ERR_INVALID_ARG;
  auto& s = it->second;
  const int64_t need = (s.len + bm->block_size - 1) / bm->block_size;
  *n_blocks = static_cast<int32_t>(need);
  if (!blocks_out) return PKV_OK;                       // size query, no change
  if (capacity < need) return PKV_ERR_INVALID_ARG;
  if (static_cast<int64_t>(bm->free_pool.size()) < need &&
      static_cast<int64_t>(bm->free_pool.size()) + bm->reclaimable() < need)
    return PKV_ERR_OUT_OF_BLOCKS;
  for (int64_t i = 0; i < need; ++i) {
    int32_t blk;
    bm->pop(&blk);
    s.blocks.push_back(blk);
    blocks_out[i] = blk;
  }
  s.swapped = false;
  return PKV_OK;
}

pkv_status pkv_bm_match_prefix(pkv_bm* bm, int64_t seq, const int32_t* tokens, int64_t n_tokens,
                               int64_t* matched_tokens) {
  if (!bm || !matched_tokens || n_tokens < 0 || (n_tokens > 0 && !tokens))
    return PKV_ERR_INVALID_ARG;
  if (bm->seqs.count(seq)) return PKV_ERR_INVALID_ARG;
  const int32_t bs = bm->block_size;
  std::vector<int32_t> blocks;
  int32_t parent = -1;
  for (int64_t i = 0; i + 1 <= n_tokens / bs; ++i) {
    pkv_bm::Key key{parent, std::vector<int32_t>(tokens + i * bs, tokens + (i + 1) * bs)};
    auto hit = bm->children.find(key);
    if (hit == bm->children.end()) break;
    blocks.push_back(hit->second);
    parent = hit->second;
  }
  for (int32_t b : blocks) {
    bm->ref[b] += 1;
    bm->tick(b);
  }
  pkv_bm::Seq s;
  s.blocks = blocks;
  s.len = static_cast<int64_t>(blocks.size()) * bs;
  bm->seqs.emplace(seq, std::move(s));
  *matched_tokens = static_cast<int64_t>(blocks.size()) * bs;
  return PKV_OK;
}

pkv_status pkv_bm_cache_prefix(pkv_bm* bm, int64_t seq, const int32_t* tokens,
                               int64_t n_tokens) {
  if (!bm || n_tokens < 0 || (n_tokens > 0 && !tokens)) return PKV_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end() || it->second.swapped) return PKV_ERR_INVALID_ARG;
  const auto& s = it->second;
  const int32_t bs = bm->block_size;
  const int64_t n = n_tokens / bs;
  if (n > static_cast<int64_t>(s.blocks.size()) || n * bs > s.len) return PKV_ERR_INVALID_ARG;
  int32_t parent = -1;
  for (int64_t i = 0; i < n; ++i) {
    pkv_bm::Key key{parent, std::vector<int32_t>(tokens + i * bs, tokens + (i + 1) * bs)};
    const int32_t blk = s.blocks[i];
    auto have = bm->children.find(key);
    if (have == bm->children.end()) {
      if (bm->cached(blk)) break;                     // cached under another key
      bm->children.emplace(key, blk);
      bm->cached_parent[blk] = parent;
      bm->cached_key[blk] = std::move(key);
      bm->n_children[blk] = 0;
      bm->n_cached += 1;
      if (parent >= 0) {
        bm->n_children[parent] += 1;
        bm->update(parent);
      }
    } else if (have->second != blk) {
      break;                                          // the prefix is cached by other blocks
    }
    bm->tick(blk);
    parent = blk;
  }
  return PKV_OK;
}

int32_t pkv_bm_num_cached(const pkv_bm* bm) { return bm ? bm->n_cached : -1; }

int32_t pkv_bm_num_evictable(const pkv_bm* bm) {
  return bm ? static_cast<int32_t>(bm->evictable.size()) : -1;
}

int32_t pkv_bm_is_swapped(const pkv_bm* bm, int64_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : (it->second.swapped ? 1 : 0);
}

int64_t pkv_bm_seq_len(const pkv_bm* bm, int64_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : it->second.len;
}

int32_t pkv_bm_num_free(const pkv_bm* bm) {
  return bm ? static_cast<int32_t>(bm->free_pool.size()) : -1;
}

pkv_status pkv_bm_check(const pkv_bm* bm) {
  if (!bm) return PKV_ERR_INVALID_ARG;
  const int32_t nb = static_cast<int32_t>(bm->ref.size());
  const int64_t bs = bm->block_size;
  constexpr pkv_status kBad = PKV_ERR_INVALID_ARG;
  // free pool: distinct pool blocks, unreferenced and not cached
  std::vector<char> in_free(nb, 0);
  for (int32_t b : bm->free_pool) {
    if (b < 0 || b >= nb || in_free[b] || bm->ref[b] != 0 || bm->cached(b)) return kBad;
    in_free[b] = 1;
  }
  // counts: each block's count is its number of occurrences in resident
  // sequences; a sequence's blocks cover its length exactly
  std::vector<int64_t> uses(nb, 0);
  for (const auto& kv : bm->seqs) {
    const auto& sq = kv.second;
    if (sq.len < 0) return kBad;
    if (sq.swapped) {
      if (!sq.blocks.empty()) return kBad;
      continue;
    }
    if (static_cast<int64_t>(sq.blocks.size()) != (sq.len + bs - 1) / bs) return kBad;
    for (int32_t b : sq.blocks) {
      if (b < 0 || b >= nb) return kBad;
      uses[b] += 1;
    }
  }
  // every block is free, referenced, or cached and idle: exactly one
  for (int32_t b = 0; b < nb; ++b) {
    if (bm->ref[b] < 0 || bm->ref[b] != uses[b]) return kBad;
    if (bm->ref[b] == 0 && !in_free[b] && !bm->cached(b)) return kBad;
  }
  // radix cache: keys and parents agree with the child map, child counts
  // are exact, and the evictable set is the idle cached leaves
  std::vector<int32_t> kids(nb, 0);
  int32_t n_cached = 0, n_idle_leaves = 0;
  for (int32_t b = 0; b < nb; ++b) {
    if (!bm->cached(b)) continue;
    n_cached += 1;
    const int32_t parent = bm->cached_parent[b];
    if (parent < -1 || parent >= nb || (parent >= 0 && !bm->cached(parent))) return kBad;
    if (bm->cached_key[b].parent != parent ||
        static_cast<int64_t>(bm->cached_key[b].tokens.size()) != bs)
      return kBad;
    auto it = bm->children.find(bm->cached_key[b]);
    if (it == bm->children.end() || it->second != b) return kBad;
    if (parent >= 0) kids[parent] += 1;
  }
  if (n_cached != bm->n_cached || static_cast<int32_t>(bm->children.size()) != n_cached)
    return kBad;
  for (int32_t b = 0; b < nb; ++b) {
    if (bm->cached(b) && kids[b] != bm->n_children[b]) return kBad;
    if (bm->idle_leaf(b)) {
      n_idle_leaves += 1;
      if (!bm->evictable.count({bm->stamp[b], b})) return kBad;
    }
  }
  if (static_cast<int32_t>(bm->evictable.size()) != n_idle_leaves) return kBad;
  return PKV_OK;
}

int32_t pkv_bm_ref_count(const pkv_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= static_cast<int32_t>(bm->ref.size())) return -1;
  return bm->ref[block];
}

}  // extern "C"
