// Stress driver for the host block pool, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_pool_sanitizers.py (CPU only).
//
// Random operations (create, create from a prompt with prefix lookups, fork,
// free, appends with and without token ids, truncation, swaps of whole sharing
// groups, tables, stats, error cases) on pools of several block sizes; after
// every operation pkv_pool_validate must pass and the counters must agree with
// what the driver tracks.  Exit code 0 means no invariant broke; the
// sanitizers abort on any memory or undefined-behaviour error.

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <set>
#include <vector>

#include "pkv.h"

#define CHECK(cond)                                                              \
  do {                                                                           \
    if (!(cond)) {                                                               \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);   \
      std::exit(1);                                                              \
    }                                                                            \
  } while (0)

int main(int argc, char** argv) {
  const int trials = argc > 1 ? std::atoi(argv[1]) : 200;
  std::mt19937 rng(12345);
  auto pick = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  int64_t ops = 0;
  for (int trial = 0; trial < trials; ++trial) {
    const int B = std::vector<int>{1, 2, 4, 16, 32}[pick(0, 4)];
    const int nb = pick(1, 80);
    std::vector<int32_t> order(nb);
    for (int i = 0; i < nb; ++i) order[i] = i;
    std::shuffle(order.begin(), order.end(), rng);
    pkv_pool* pool = nullptr;
    CHECK(pkv_pool_create(nb, B, order.data(), &pool) == PKV_OK);
    CHECK(pkv_pool_set_host_blocks(pool, pick(0, 40)) == PKV_OK);
    std::set<int32_t> live;
    std::vector<int32_t> stem(static_cast<size_t>(pick(1, 3 * B + 2)));
    for (auto& t : stem) t = pick(0, 2);
    for (int step = 0; step < 150; ++step, ++ops) {
      const int op = pick(0, 9);
      std::vector<int32_t> lv(live.begin(), live.end());
      if (op == 0 || lv.empty()) {
        int32_t sid;
        CHECK(pkv_seq_create(pool, &sid) == PKV_OK);
        live.insert(sid);
      } else if (op == 1) {
        std::vector<int32_t> prompt = stem;
        for (int i = pick(0, 5); i > 0; --i) prompt.push_back(pick(0, 2));
        int32_t sid, hit;
        CHECK(pkv_seq_create_prefixed(pool, prompt.data(), static_cast<int32_t>(prompt.size()), &sid, &hit) == PKV_OK);
        CHECK(hit % B == 0 && hit <= static_cast<int32_t>(prompt.size()));
        live.insert(sid);
        const int32_t rest = static_cast<int32_t>(prompt.size()) - hit;
        std::vector<int64_t> slots(rest + 1);
        std::vector<int32_t> pairs(2);
        int32_t ncow = 0;
        const pkv_status st = pkv_append_tokens(pool, &sid, &rest, 1, prompt.data() + hit, slots.data(),
                                                static_cast<int64_t>(slots.size()), pairs.data(), 1, &ncow);
        CHECK(st == PKV_OK || st == PKV_ERR_OUT_OF_BLOCKS || st == PKV_ERR_SWAPPED);
      } else if (op == 2 || op == 3) {
        const int k = pick(1, static_cast<int>(lv.size()));
        std::shuffle(lv.begin(), lv.end(), rng);
        std::vector<int32_t> seqs(lv.begin(), lv.begin() + k), counts(k);
        int64_t total = 0;
        for (auto& c : counts) total += (c = pick(0, 2 * B + 1));
        std::vector<int32_t> tok(static_cast<size_t>(total) + 1);
        for (auto& t : tok) t = pick(0, 2);
        std::vector<int64_t> slots(static_cast<size_t>(total) + 1);
        std::vector<int32_t> pairs(2 * static_cast<size_t>(k));
        int32_t ncow = 0;
        const pkv_status st = pkv_append_tokens(pool, seqs.data(), counts.data(), k, op == 2 ? tok.data() : nullptr,
                                                slots.data(), static_cast<int64_t>(slots.size()), pairs.data(), k,
                                                &ncow);
        CHECK(st == PKV_OK || st == PKV_ERR_OUT_OF_BLOCKS || st == PKV_ERR_SWAPPED);
        if (st == PKV_OK) {
          std::set<int64_t> distinct(slots.begin(), slots.begin() + total);
          CHECK(static_cast<int64_t>(distinct.size()) == total);
          for (int64_t i = 0; i < total; ++i) CHECK(slots[i] >= 0 && slots[i] < static_cast<int64_t>(nb) * B);
        }
      } else if (op == 4) {
        int32_t child;
        const pkv_status st = pkv_seq_fork(pool, lv[pick(0, static_cast<int>(lv.size()) - 1)], &child);
        CHECK(st == PKV_OK || st == PKV_ERR_SWAPPED);
        if (st == PKV_OK) live.insert(child);
      } else if (op == 5) {
        const int32_t sid = lv[pick(0, static_cast<int>(lv.size()) - 1)];
        CHECK(pkv_seq_free(pool, sid) == PKV_OK);
        live.erase(sid);
        CHECK(pkv_seq_free(pool, sid) == PKV_ERR_NO_SUCH_SEQ);  // double free is refused
      } else if (op == 6) {
        const int32_t sid = lv[pick(0, static_cast<int>(lv.size()) - 1)];
        int32_t len, nblk;
        CHECK(pkv_seq_info(pool, sid, &len, &nblk) == PKV_OK);
        const pkv_status st = pkv_seq_truncate(pool, sid, pick(0, len));
        CHECK(st == PKV_OK || st == PKV_ERR_SWAPPED);
        CHECK(pkv_seq_truncate(pool, sid, len + 1) == PKV_ERR_INVALID_ARG || st == PKV_ERR_SWAPPED);
      } else if (op == 7) {
        // swap one sequence's whole sharing group (every live sequence holding one of its blocks, transitively)
        const int32_t sid = lv[pick(0, static_cast<int>(lv.size()) - 1)];
        std::set<int32_t> group{sid};
        bool grew = true;
        while (grew) {
          grew = false;
          std::set<int32_t> blocks;
          for (int32_t g : group) {
            int32_t n = 0, host = 0;
            pkv_seq_table(pool, g, nullptr, 0, &n, &host);
            std::vector<int32_t> t(static_cast<size_t>(n) + 1);
            CHECK(pkv_seq_table(pool, g, t.data(), n, &n, &host) == PKV_OK);
            blocks.insert(t.begin(), t.begin() + n);
          }
          for (int32_t other : lv) {
            if (group.count(other)) continue;
            int32_t n = 0, host = 0, mine = 0;
            pkv_seq_table(pool, sid, nullptr, 0, &n, &mine);
            pkv_seq_table(pool, other, nullptr, 0, &n, &host);
            if (host != mine) continue;
            std::vector<int32_t> t(static_cast<size_t>(n) + 1);
            CHECK(pkv_seq_table(pool, other, t.data(), n, &n, &host) == PKV_OK);
            for (int i = 0; i < n; ++i)
              if (blocks.count(t[i])) {
                group.insert(other);
                grew = true;
                break;
              }
          }
        }
        std::vector<int32_t> g(group.begin(), group.end()), pairs(2 * static_cast<size_t>(nb + 64));
        int32_t n = 0, on_host = 0, np = 0;
        pkv_seq_table(pool, sid, nullptr, 0, &n, &on_host);
        const pkv_status st = on_host ? pkv_swap_in(pool, g.data(), static_cast<int32_t>(g.size()), pairs.data(), nb + 64, &np)
                                      : pkv_swap_out(pool, g.data(), static_cast<int32_t>(g.size()), pairs.data(), nb + 64, &np);
        CHECK(st == PKV_OK || st == PKV_ERR_OUT_OF_BLOCKS || st == PKV_ERR_INVALID_ARG);
      } else if (op == 8) {
        std::vector<int32_t> dev;
        for (int32_t sid : lv) {
          int32_t n = 0, host = 0;
          pkv_seq_table(pool, sid, nullptr, 0, &n, &host);
          if (!host) dev.push_back(sid);
        }
        const int32_t mb = nb + 1;
        std::vector<int32_t> tables(dev.size() * mb + 1), lens(dev.size() + 1);
        CHECK(pkv_block_tables(pool, dev.data(), static_cast<int32_t>(dev.size()), mb, tables.data(), lens.data()) == PKV_OK);
      } else {
        // argument errors leave the pool as it was
        int32_t dup[2] = {lv[0], lv[0]}, ones[2] = {1, 1}, ncow = 0;
        int64_t slots[4];
        int32_t pairs[4];
        CHECK(pkv_append_tokens(pool, dup, ones, 2, nullptr, slots, 4, pairs, 2, &ncow) == PKV_ERR_INVALID_ARG);
        int32_t unknown = 1 << 30;
        CHECK(pkv_append_tokens(pool, &unknown, ones, 1, nullptr, slots, 4, pairs, 2, &ncow) == PKV_ERR_NO_SUCH_SEQ);
        CHECK(pkv_seq_truncate(pool, -1, 0) == PKV_ERR_NO_SUCH_SEQ);
        CHECK(pkv_seq_create_prefixed(pool, nullptr, 3, &unknown, &ncow) == PKV_ERR_INVALID_ARG);
      }
      CHECK(pkv_pool_validate(pool) == PKV_OK);
      pkv_stats st;
      CHECK(pkv_pool_stats(pool, &st) == PKV_OK);
      CHECK(st.num_seqs == static_cast<int64_t>(live.size()));
      CHECK(st.free_blocks + st.used_blocks == nb);
      CHECK(st.cached_free_blocks <= st.cached_blocks && st.cached_blocks <= nb);
      std::vector<uint64_t> keys(static_cast<size_t>(st.cached_blocks) + 1);
      std::vector<int32_t> kb(static_cast<size_t>(st.cached_blocks) + 1);
      int32_t nk = 0;
      CHECK(pkv_pool_cached_blocks(pool, keys.data(), kb.data(), static_cast<int32_t>(st.cached_blocks), &nk) == PKV_OK);
      CHECK(nk == st.cached_blocks);
    }
    pkv_pool_destroy(pool);
  }
  std::printf("ok: %lld operations\n", static_cast<long long>(ops));
  return 0;
}
