// Random operations on the block manager's C ABI, for a sanitizer build of the
// host code (no GPU): every call's outputs are checked for range, and the
// process exits non-zero on the first inconsistency.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <set>
#include <vector>

#include "pkv.h"

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      return 1;                                                    \
    }                                                              \
  } while (0)

int main(int argc, char** argv) {
  const int seed = argc > 1 ? atoi(argv[1]) : 1;
  const int n_ops = argc > 2 ? atoi(argv[2]) : 20000;
  std::mt19937 rng(seed);
  auto pick = [&](int n) { return (int)(rng() % (unsigned)n); };
  const int n_blocks = 64 + pick(200), n_host = pick(100);
  pkv_block_manager* bm = pkv_bm_create(n_blocks, n_host, pick(4) != 0);
  CHECK(bm);
  std::vector<int64_t> live;
  std::set<int64_t> swapped;
  int64_t next_id = 0;
  std::vector<int32_t> toks, pairs((size_t)(n_blocks + n_host + 8) * 2), table(4096);
  std::vector<int64_t> slots;
  for (int op = 0; op < n_ops; ++op) {
    const int r = pick(100);
    if (r < 25 || live.empty()) {
      const int n = pick(120);
      toks.resize((size_t)n);
      const int vocab = 1 + pick(8);
      for (auto& t : toks) t = pick(vocab);
      slots.resize((size_t)n + 1);
      int32_t cow[2];
      int n_cow = -1, n_cached = -1;
      const int rc = pkv_bm_add_sequence(bm, next_id, toks.data(), n, slots.data(), cow, &n_cow,
                                         &n_cached);
      CHECK(rc == PKV_OK || rc == PKV_ERR_NO_BLOCKS);
      if (rc == PKV_OK) {
        CHECK(n_cached >= 0 && n_cached <= n && (n_cow == 0 || n_cow == 1));
        for (int i = 0; i < n; ++i)
          CHECK(i < n_cached ? slots[(size_t)i] == -1
                             : slots[(size_t)i] >= 0 && slots[(size_t)i] < (int64_t)n_blocks * 16);
        live.push_back(next_id);
      }
      ++next_id;
    } else if (r < 50) {
      const int64_t id = live[(size_t)pick((int)live.size())];
      if (swapped.count(id)) continue;
      const int n = 1 + pick(6);
      toks.assign((size_t)n, pick(8));
      slots.resize((size_t)n);
      int32_t cow[2];
      int n_cow = -1;
      const int rc = pkv_bm_append(bm, id, toks.data(), n, slots.data(), cow, &n_cow);
      CHECK(rc == PKV_OK || rc == PKV_ERR_NO_BLOCKS);
      if (rc == PKV_OK)
        for (int i = 0; i < n; ++i)
          CHECK(slots[(size_t)i] >= 0 && slots[(size_t)i] < (int64_t)n_blocks * 16);
    } else if (r < 60) {
      std::vector<int64_t> ids;
      for (int64_t id : live)
        if (!swapped.count(id) && pick(2)) ids.push_back(id);
      const int n = (int)ids.size();
      toks.assign((size_t)n, pick(8));
      slots.resize((size_t)n + 1);
      std::vector<int32_t> cow((size_t)n * 2 + 2);
      int n_cow = -1;
      const int rc = pkv_bm_append_batch(bm, n, ids.data(), toks.data(), slots.data(), cow.data(),
                                         &n_cow);
      CHECK(rc == PKV_OK || rc == PKV_ERR_NO_BLOCKS);
      if (rc == PKV_OK) CHECK(n_cow >= 0 && n_cow <= n);
    } else if (r < 68) {
      const int64_t id = live[(size_t)pick((int)live.size())];
      if (swapped.count(id)) continue;
      CHECK(pkv_bm_fork(bm, id, next_id) == PKV_OK);
      live.push_back(next_id++);
    } else if (r < 80) {
      const size_t k = (size_t)pick((int)live.size());
      CHECK(pkv_bm_free(bm, live[k]) == PKV_OK);
      swapped.erase(live[k]);
      live.erase(live.begin() + (long)k);
    } else if (r < 90) {
      const int64_t id = live[(size_t)pick((int)live.size())];
      int n_pairs = -1;
      const bool out = !swapped.count(id);
      const int rc = out ? pkv_bm_swap_out(bm, id, pairs.data(), (int)pairs.size() / 2, &n_pairs)
                         : pkv_bm_swap_in(bm, id, pairs.data(), (int)pairs.size() / 2, &n_pairs);
      CHECK(rc == PKV_OK || rc == PKV_ERR_NO_BLOCKS || rc == PKV_ERR_INVALID_ARG);
      if (rc == PKV_OK) {
        for (int i = 0; i < n_pairs; ++i) {
          const int32_t d = pairs[2 * (size_t)i], h = pairs[2 * (size_t)i + 1];
          CHECK(out ? (d >= 0 && d < n_blocks && h >= 0 && h < n_host)
                    : (d >= 0 && d < n_host && h >= 0 && h < n_blocks));
        }
        if (out) swapped.insert(id);
        else swapped.erase(id);
      }
    } else {
      const int64_t id = live[(size_t)pick((int)live.size())];
      int nb = -1, len = -1;
      const int rc = pkv_bm_block_table(bm, id, table.data(), (int)table.size(), &nb, &len);
      CHECK(rc == PKV_OK || (rc == PKV_ERR_INVALID_ARG && swapped.count(id)));
      if (rc == PKV_OK) {
        CHECK(nb == (len + 15) / 16);
        for (int j = 0; j < nb; ++j) CHECK(table[(size_t)j] >= 0 && table[(size_t)j] < n_blocks);
      }
    }
    pkv_bm_stats st;
    CHECK(pkv_bm_get_stats(bm, &st) == PKV_OK);
    CHECK(st.free_blocks >= 0 && st.free_blocks <= n_blocks);
    CHECK(st.host_free_blocks >= 0 && st.host_free_blocks <= n_host);
    CHECK(st.cached_free_blocks <= st.free_blocks && st.cached_blocks <= n_blocks);
    CHECK(st.n_sequences == (int32_t)live.size());
  }
  for (int64_t id : live) CHECK(pkv_bm_free(bm, id) == PKV_OK);
  pkv_bm_stats st;
  CHECK(pkv_bm_get_stats(bm, &st) == PKV_OK);
  CHECK(st.free_blocks == n_blocks && st.host_free_blocks == n_host);
  pkv_bm_destroy(bm);
  printf("ok %d ops\n", n_ops);
  return 0;
}
