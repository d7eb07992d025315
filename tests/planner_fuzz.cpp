// Random and adversarial page tables through the host planner, built with
// AddressSanitizer and UBSan by tests/test_planner.py.  Checks that every
// query token's visible keys are covered exactly once and that bad tables
// are rejected with a status instead of crashing.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "mla.h"

static int fails = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      std::printf("CHECK failed line %d: %s\n", __LINE__, #c);     \
      ++fails;                                                     \
    }                                                              \
  } while (0)

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 100;
  std::mt19937 rng(12345);
  for (int it = 0; it < iters; ++it) {
    const int B = rng() % 12;
    const int P = 1 + rng() % 70;
    const int heads = 1 + rng() % 128;
    const int workers = 1 + rng() % 300;
    const bool causal = rng() & 1;
    std::vector<int> qo(B + 1, 0), kv(B + 1, 0), last(B, 0), lens(B), qs(B);
    for (int b = 0; b < B; ++b) {
      lens[b] = (rng() % 5 == 0) ? 0 : rng() % 3000;
      qs[b] = (rng() % 3 == 0) ? rng() % 300 : 1;
      const int n = (lens[b] + P - 1) / P;
      kv[b + 1] = kv[b] + n;
      qo[b + 1] = qo[b] + qs[b];
      last[b] = n ? lens[b] - (n - 1) * P : 0;
    }
    const int nnz = kv[B];
    const int pages = nnz + 3;
    std::vector<int> idx(nnz + 1);
    for (int i = 0; i < nnz; ++i) idx[i] = rng() % pages;
    mla_schedule_t s = nullptr;
    mla_status st = mla_schedule_build(&s, qo.data(), kv.data(), idx.data(), last.data(), B,
                                       causal, P, pages, heads, workers);
    CHECK(st == MLA_OK);
    if (st != MLA_OK) {
      std::printf("%s\n", mla_last_error());
      continue;
    }
    int32_t w = 0;
    int64_t n_items = 0, n_merges = 0, n_slots = 0;
    mla_schedule_sizes(s, &w, &n_items, &n_merges, &n_slots);
    std::vector<int32_t> wi(w + 2), items(n_items * 8 + 8), merges(n_merges * 4 + 4);
    mla_schedule_copy(s, wi.data(), items.data(), merges.data());
    mla_schedule_destroy(s);
    CHECK(w == workers && wi[0] == 0 && wi[w] <= wi[w + 1] && wi[w + 1] == n_items);
    for (int k = 0; k < w; ++k) CHECK(wi[k] <= wi[k + 1]);
    for (int64_t i = wi[w]; i < n_items; ++i) CHECK(items[i * 8 + 4] == -1 && items[i * 8 + 2] == 0);
    const int T = qo[B];
    std::vector<long long> covered(T, 0);
    std::vector<int> slot_used(n_slots, 0);
    for (int64_t i = 0; i < n_items; ++i) {
      const int32_t* e = &items[i * 8];
      const int t = e[0], row = e[1], kb = e[2], ke = e[3], slot = e[4];
      CHECK(t >= 0 && t < T && row >= 0 && row < B);
      CHECK(qo[row] <= t && t < qo[row + 1]);
      const int i_q = t - qo[row];
      long long vis = lens[row];
      if (causal) {
        vis = (long long)i_q + lens[row] - qs[row] + 1;
        if (vis < 0) vis = 0;
        if (vis > lens[row]) vis = lens[row];
      }
      CHECK(kb % 32 == 0 && kb <= ke && ke <= vis);
      covered[t] += ke - kb;
      if (slot >= 0) {
        CHECK(slot < n_slots);
        if (slot < n_slots) ++slot_used[slot];
      }
    }
    for (int t = 0; t < T; ++t) {
      int b = 0;
      while (qo[b + 1] <= t) ++b;
      const int i_q = t - qo[b];
      long long vis = lens[b];
      if (causal) {
        vis = (long long)i_q + lens[b] - qs[b] + 1;
        if (vis < 0) vis = 0;
        if (vis > lens[b]) vis = lens[b];
      }
      CHECK(covered[t] == vis);
    }
    for (int64_t sl = 0; sl < n_slots; ++sl) CHECK(slot_used[sl] == 1);
  }
  // Adversarial tables must be rejected, never crash.
  {
    int qo[3] = {0, 1, 3}, kv[3] = {0, 2, 1}, idx[3] = {0, 1, 2}, last[2] = {3, 4};
    mla_schedule_t s = nullptr;
    CHECK(mla_schedule_build(&s, qo, kv, idx, last, 2, 1, 4, 4, 16, 8) == MLA_E_INVALID);
    int kv2[3] = {0, 2, 3}, idx2[3] = {0, 7, 2};
    CHECK(mla_schedule_build(&s, qo, kv2, idx2, last, 2, 1, 4, 4, 16, 8) == MLA_E_INVALID);
    int last2[2] = {0, 4};
    CHECK(mla_schedule_build(&s, qo, kv2, idx, last2, 2, 1, 4, 4, 16, 8) == MLA_E_INVALID);
    CHECK(mla_schedule_build(&s, qo, kv2, idx, last, 2, 1, 4, 4, 0, 8) == MLA_E_UNSUPPORTED);
    CHECK(mla_schedule_build(&s, qo, kv2, idx, last, -1, 1, 4, 4, 16, 8) == MLA_E_INVALID);
    CHECK(mla_schedule_build(nullptr, qo, kv2, idx, last, 2, 1, 4, 4, 16, 8) == MLA_E_INVALID);
  }
  if (fails) {
    std::printf("%d failures\n", fails);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
