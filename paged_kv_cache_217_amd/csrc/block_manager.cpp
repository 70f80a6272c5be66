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
#include <cstdint>
#include <new>
#include <unordered_map>
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

  bool pop(int32_t* blk) {
    if (free_pool.empty()) return false;
    *blk = free_pool.back();
    free_pool.pop_back();
    ref[*blk] += 1;
    return true;
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
  *out = bm;
  return PKV_OK;
}

void pkv_bm_destroy(pkv_bm* bm) { delete bm; }

pkv_status pkv_bm_append_slot(pkv_bm* bm, int64_t seq, int64_t* slot, int32_t* cow_src,
                              int32_t* cow_dst) {
  if (!bm || !slot || !cow_src || !cow_dst) return PKV_ERR_INVALID_ARG;
  auto found = bm->seqs.find(seq);
  if (found != bm->seqs.end() && found->second.swapped) return PKV_ERR_INVALID_ARG;
  auto& s = bm->seqs[seq];
  const int64_t pos = s.len;
  const int32_t bs = bm->block_size;
  int32_t src = -1, dst = -1;
  if (pos % bs == 0) {
    int32_t blk;
    if (!bm->pop(&blk)) {
      if (s.blocks.empty() && s.len == 0) bm->seqs.erase(seq);  // leave no trace
      return PKV_ERR_OUT_OF_BLOCKS;
    }
    s.blocks.push_back(blk);
  } else {
    const int32_t last = s.blocks.back();
    if (bm->ref[last] > 1) {
      int32_t fresh;
      if (!bm->pop(&fresh)) return PKV_ERR_OUT_OF_BLOCKS;
      bm->ref[last] -= 1;
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
  for (int32_t blk : it->second.blocks) {
    bm->ref[blk] -= 1;
    if (bm->ref[blk] == 0) bm->free_pool.push_back(blk);
  }
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
    const int32_t blk = s.blocks[i];
    blocks_out[i] = blk;
    bm->ref[blk] -= 1;
    if (bm->ref[blk] == 0) bm->free_pool.push_back(blk);
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
  if (static_cast<int64_t>(bm->free_pool.size()) < need) return PKV_ERR_OUT_OF_BLOCKS;
  for (int64_t i = 0; i < need; ++i) {
    int32_t blk;
    bm->pop(&blk);
    s.blocks.push_back(blk);
    blocks_out[i] = blk;
  }
  s.swapped = false;
  return PKV_OK;
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

int32_t pkv_bm_ref_count(const pkv_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= static_cast<int32_t>(bm->ref.size())) return -1;
  return bm->ref[block];
}

}  // extern "C"
