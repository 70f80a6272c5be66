// Host-only driver for the block manager, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_sanitizers.py: random append /
// fork / free / swap / prefix-cache sequences with invariant checks after
// every operation.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "pkv.h"

static int fail(const char* what) {
  std::fprintf(stderr, "invariant violated: %s\n", what);
  return 1;
}

int main() {
  std::mt19937 rng(217);
  for (int trial = 0; trial < 50; ++trial) {
    const int nb = 4 + static_cast<int>(rng() % 60);
    const int bs = 1 << (rng() % 5);
    pkv_bm* bm = nullptr;
    if (pkv_bm_create(nb, bs, &bm) != PKV_OK) return fail("create");
    std::vector<int64_t> live, swapped;
    int64_t next = 0;
    std::vector<std::vector<int32_t>> prompts(5);
    for (auto& p : prompts) {
      p.resize(1 + rng() % (3 * bs + 2));
      for (auto& t : p) t = static_cast<int32_t>(rng() % 3);
    }
    std::vector<int32_t> blocks(nb);
    for (int step = 0; step < 2000; ++step) {
      const unsigned op = rng() % 100;
      if (op < 65 || live.empty()) {
        const bool fresh = live.empty() || rng() % 5 == 0;
        const int64_t seq = fresh ? next++ : live[rng() % live.size()];
        int64_t slot;
        int32_t src, dst;
        const pkv_status st = pkv_bm_append_slot(bm, seq, &slot, &src, &dst);
        if (st == PKV_OK) {
          if (fresh) live.push_back(seq);
          if (slot < 0 || slot >= static_cast<int64_t>(nb) * bs) return fail("slot range");
          if ((src < 0) != (dst < 0)) return fail("cow pair");
        } else if (st != PKV_ERR_OUT_OF_BLOCKS) {
          return fail("append status");
        }
      } else if (op < 72) {
        const int64_t child = next++;
        if (pkv_bm_fork(bm, live[rng() % live.size()], child) != PKV_OK) return fail("fork");
        live.push_back(child);
      } else if (op < 80) {
        // a prompt: match the cached prefix, append the rest, register it
        const auto& p = prompts[rng() % prompts.size()];
        const int64_t seq = next++;
        int64_t matched = -1;
        if (pkv_bm_match_prefix(bm, seq, p.data(), static_cast<int64_t>(p.size()), &matched) !=
                PKV_OK ||
            matched < 0 || matched > static_cast<int64_t>(p.size()) || matched % bs != 0)
          return fail("match_prefix");
        live.push_back(seq);
        bool ok = true;
        for (int64_t i = matched; i < static_cast<int64_t>(p.size()) && ok; ++i) {
          int64_t slot;
          int32_t src, dst;
          const pkv_status st = pkv_bm_append_slot(bm, seq, &slot, &src, &dst);
          if (st == PKV_ERR_OUT_OF_BLOCKS) ok = false;
          else if (st != PKV_OK) return fail("prompt append");
        }
        if (ok && pkv_bm_cache_prefix(bm, seq, p.data(), static_cast<int64_t>(p.size())) !=
                      PKV_OK)
          return fail("cache_prefix");
      } else if (op < 86) {
        const size_t i = rng() % live.size();
        int32_t n = 0;
        if (pkv_bm_swap_out(bm, live[i], blocks.data(), nb, &n) != PKV_OK) return fail("swap_out");
        swapped.push_back(live[i]);
        live.erase(live.begin() + static_cast<long>(i));
      } else if (op < 90 && !swapped.empty()) {
        const size_t i = rng() % swapped.size();
        int32_t n = 0;
        const pkv_status st = pkv_bm_swap_in(bm, swapped[i], blocks.data(), nb, &n);
        if (st == PKV_OK) {
          live.push_back(swapped[i]);
          swapped.erase(swapped.begin() + static_cast<long>(i));
        } else if (st != PKV_ERR_OUT_OF_BLOCKS) {
          return fail("swap_in status");
        }
      } else {
        const size_t i = rng() % live.size();
        if (pkv_bm_free(bm, live[i]) != PKV_OK) return fail("free");
        live.erase(live.begin() + static_cast<long>(i));
      }
      if (pkv_bm_check(bm) != PKV_OK) return fail("pkv_bm_check");
      // every block is free, referenced or cached and idle; counts never negative
      int referenced = 0;
      for (int b = 0; b < nb; ++b) {
        const int r = pkv_bm_ref_count(bm, b);
        if (r < 0) return fail("negative ref count");
        referenced += r > 0;
      }
      const int free_now = pkv_bm_num_free(bm);
      if (referenced + free_now > nb) return fail("free + referenced > pool");
      if (referenced + free_now + pkv_bm_num_cached(bm) < nb) return fail("blocks lost");
      if (pkv_bm_num_evictable(bm) > pkv_bm_num_cached(bm)) return fail("evictable > cached");
    }
    int32_t table[64 * 64];
    int max_blocks = nb;
    if (!live.empty() && live.size() <= 64 && max_blocks <= 64 &&
        pkv_bm_export_table(bm, live.data(), static_cast<int32_t>(live.size()), max_blocks,
                            table) != PKV_OK)
      return fail("export");
    for (int64_t s : live) pkv_bm_free(bm, s);
    for (int64_t s : swapped) pkv_bm_free(bm, s);
    if (pkv_bm_num_free(bm) + pkv_bm_num_cached(bm) != nb)
      return fail("pool not whole after freeing everything");
    pkv_bm_destroy(bm);
  }
  std::printf("block manager: ok\n");
  return 0;
}
