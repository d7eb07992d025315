// Host planner: page-table validation and split-KV work balancing.
//
// The documentation describes planning on the host from CPU index tensors
// (page "mstar.engine.resources.attn.flashinfer_mla", FlashInferMLAWrapper.plan,
// whose index inputs can be host tensors) and a per-row key length built from
// paged_kv_indptr and paged_kv_last_page_len.  The split of long key ranges
// into chunks, and their balance over compute units, is this library's own
// design: the work is laid out as one stream of (token, key tile) units and
// cut into num_workers contiguous pieces of near-equal cost; a token whose
// keys straddle a cut is split into partial results that a merge kernel
// combines through their log-sum-exp.
#include "planner.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>

namespace mla {

namespace {
thread_local std::string g_last_error;

struct TokenWork {
  int32_t token;
  int32_t row;
  int32_t visible;  // keys the token sees (a prefix of its row's keys)
  int32_t tiles;    // ceil(visible / kTileKeys)
};

// Cost of one work item in units of one key tile (32 latent rows, 36 KiB),
// fitted to per-workgroup timings on MI355X: at 128 heads a tile costs about
// 3.3-3.8K cycles and an item's fixed part (query load, pipeline fill and
// drain, output) 24-28K, i.e. seven tiles; a partial output (bf16 rows of all
// heads) takes the workgroup no longer to write than a final one, and the
// split's one-tile charge stands for its share of the merge kernel.
struct CostModel {
  double item;
  double split;
  explicit CostModel(int heads)
      : item(1.0 + 6.0 * heads / 128.0), split(0.25 + 0.75 * heads / 128.0) {}
};

constexpr int kMinPieceTiles = 2;

// The shared pool.  The compute units of one device do not run at one speed:
// under the sustained MFMA load of a prefill the XCDs' clocks differ by up to
// 10%, so workgroups with equal static loads end that far apart.  A batch of
// many query tokens keeps its smallest whole-token items (up to kPoolShare of
// the work, none larger than 1/kPoolItemDiv of a worker's share) out of the
// static lists; workgroups take them, largest first, as their own lists run
// out.  Pool items are never split, so who runs them changes no result.
constexpr double kPoolShare = 0.10;
constexpr int kPoolItemDiv = 8;
constexpr int kPoolMinTokensPerWorker = 4;

// Greedy contiguous fill of `budget` cost per worker; *max_load receives
// the largest worker cost (above the budget only where the last worker had
// to take the rest).  kEmit = false only computes that cost (the budget
// search calls it many times per plan); kEmit = true also records the items.
// Items come out in worker order: those of worker k are
// (*items)[(*first)[k] .. (*first)[k + 1]).
template <bool kEmit>
void fill(const std::vector<TokenWork>& toks, const CostModel& cm, double budget,
          int32_t num_workers, std::vector<WorkItem>* items, std::vector<int32_t>* first,
          double* max_load) {
  if (kEmit) {
    items->clear();
    first->assign(num_workers + 1, 0);
  }
  int k = 0;
  double cur = 0.0;  // cost on worker k
  double peak = 0.0;  // largest cost of the workers before k
  auto next_worker = [&] {
    peak = std::max(peak, cur);
    cur = 0.0;
    ++k;
    if (kEmit) (*first)[k] = static_cast<int32_t>(items->size());
  };
  auto emit = [&](const WorkItem& w) {
    if (kEmit) items->push_back(w);
  };
  for (const TokenWork& tw : toks) {
    if (tw.tiles == 0) {
      emit(WorkItem{tw.token, tw.row, 0, 0, -1, 0, {0, 0}});
      cur += cm.item;
      if (cur >= budget && k < num_workers - 1) next_worker();
      continue;
    }
    int a = 0;
    bool split = false;
    while (a < tw.tiles) {
      const int rem = tw.tiles - a;
      const double free = budget - cur;
      const bool last = k == num_workers - 1;
      // The whole remainder as one item, if it is not too long and fits.
      if (rem <= kMaxItemTiles &&
          (rem + cm.item + (split ? cm.split : 0.0) <= free + kMinPieceTiles || last)) {
        emit(WorkItem{tw.token, tw.row, a * kTileKeys, tw.visible, split ? 0 : -1, 0, {0, 0}});
        cur += rem + cm.item + (split ? cm.split : 0.0);
        a = tw.tiles;
        break;
      }
      // Otherwise a piece: at most kMaxItemTiles, and when it is cut for the
      // budget, leave at least kMinPieceTiles for the rest.
      int cap = rem > kMaxItemTiles ? kMaxItemTiles : rem - kMinPieceTiles;
      int take = last ? cap : std::min(cap, static_cast<int>(free - cm.item - cm.split));
      if (take >= kMinPieceTiles) {
        emit(WorkItem{tw.token, tw.row, a * kTileKeys, (a + take) * kTileKeys, 0, 0, {0, 0}});
        cur += take + cm.item + cm.split;
        a += take;
        split = true;
        if (!last && cur >= budget - kMinPieceTiles) next_worker();  // this worker is full
        continue;
      }
      next_worker();  // no room left on this worker (never the last one here)
    }
    if (cur >= budget && k < num_workers - 1) next_worker();
  }
  *max_load = std::max(peak, cur);
  if (kEmit)
    for (int j = k + 1; j <= num_workers; ++j) (*first)[j] = static_cast<int32_t>(items->size());
}

}  // namespace

void set_last_error(const std::string& msg) { g_last_error = msg; }
void clear_last_error() { g_last_error.clear(); }

static mla_status fail(mla_status s, const std::string& msg) {
  set_last_error(msg);
  return s;
}

mla_status build_schedule(const PlanArgs& a, Schedule* out) {
  char buf[256];
  if (a.batch < 0) return fail(MLA_E_INVALID, "batch must be >= 0");
  if (a.page_size < 1) return fail(MLA_E_INVALID, "page_size must be >= 1");
  if (a.num_heads < 1 || a.num_heads > kMaxHeads)
    return fail(MLA_E_UNSUPPORTED, "num_heads must be in [1, 128]");
  if (a.num_workers < 1) return fail(MLA_E_INVALID, "num_workers must be >= 1");
  if (a.batch > 0 && (!a.qo_indptr || !a.kv_indptr || !a.kv_last_page_len))
    return fail(MLA_E_INVALID, "NULL index array");
  if (a.num_cache_pages < 0) return fail(MLA_E_INVALID, "num_cache_pages must be >= 0");
  // The kernels address a cache row (page * page_size + slot) in 32 bits;
  // 2^31 bf16 rows are 2.5 TB, more than one device holds.
  if (a.num_cache_pages > (int64_t(INT32_MAX) + 1) / a.page_size)
    return fail(MLA_E_UNSUPPORTED, "num_cache_pages * page_size exceeds 2^31 cache rows");

  const int32_t B = a.batch;
  if (B > 0 && (a.qo_indptr[0] != 0 || a.kv_indptr[0] != 0))
    return fail(MLA_E_INVALID, "qo_indptr[0] and kv_indptr[0] must be 0");
  for (int32_t b = 0; b < B; ++b) {
    if (a.qo_indptr[b + 1] < a.qo_indptr[b]) {
      std::snprintf(buf, sizeof buf, "qo_indptr decreases at row %d", b);
      return fail(MLA_E_INVALID, buf);
    }
    if (a.kv_indptr[b + 1] < a.kv_indptr[b]) {
      std::snprintf(buf, sizeof buf, "kv_indptr decreases at row %d", b);
      return fail(MLA_E_INVALID, buf);
    }
    const int32_t n = a.kv_indptr[b + 1] - a.kv_indptr[b];
    const int32_t last = a.kv_last_page_len[b];
    if (n > 0 && (last < 1 || last > a.page_size)) {
      std::snprintf(buf, sizeof buf, "kv_last_page_len[%d]=%d outside [1, %d]", b, last,
                    a.page_size);
      return fail(MLA_E_INVALID, buf);
    }
    const int64_t L = n > 0 ? int64_t(n - 1) * a.page_size + last : 0;
    if (L > INT32_MAX / 2) {
      std::snprintf(buf, sizeof buf, "row %d has too many keys", b);
      return fail(MLA_E_INVALID, buf);
    }
  }
  const int64_t nnz = B > 0 ? a.kv_indptr[B] : 0;
  if (nnz > 0 && !a.kv_indices) return fail(MLA_E_INVALID, "NULL kv_indices");
  for (int64_t i = 0; i < nnz; ++i) {
    const int32_t p = a.kv_indices[i];
    if (p < 0 || p >= a.num_cache_pages) {
      std::snprintf(buf, sizeof buf, "kv_indices[%lld]=%d outside [0, %lld)", (long long)i, p,
                    (long long)a.num_cache_pages);
      return fail(MLA_E_INVALID, buf);
    }
  }
  const int64_t T = B > 0 ? a.qo_indptr[B] : 0;

  std::vector<TokenWork> toks;
  toks.reserve(static_cast<size_t>(T));
  for (int32_t b = 0; b < B; ++b) {
    const int32_t n = a.kv_indptr[b + 1] - a.kv_indptr[b];
    const int64_t L = n > 0 ? int64_t(n - 1) * a.page_size + a.kv_last_page_len[b] : 0;
    const int32_t Q = a.qo_indptr[b + 1] - a.qo_indptr[b];
    for (int32_t i = 0; i < Q; ++i) {
      int64_t vis = L;
      if (a.causal) vis = std::min<int64_t>(L, std::max<int64_t>(0, int64_t(i) + L - Q + 1));
      const int32_t v = static_cast<int32_t>(vis);
      toks.push_back(TokenWork{a.qo_indptr[b] + i, b, v, (v + kTileKeys - 1) / kTileKeys});
    }
  }

  // KV append targets: the step's tokens are the last keys of their rows.
  std::vector<int32_t> append_rows(static_cast<size_t>(T), 0);
  std::string append_error;
  for (int32_t b = 0; b < B && append_error.empty(); ++b) {
    const int32_t n = a.kv_indptr[b + 1] - a.kv_indptr[b];
    const int64_t L = n > 0 ? int64_t(n - 1) * a.page_size + a.kv_last_page_len[b] : 0;
    const int32_t Q = a.qo_indptr[b + 1] - a.qo_indptr[b];
    if (Q > L) {
      std::snprintf(buf, sizeof buf, "row %d has %d query tokens but %lld keys: nowhere to append",
                    b, Q, (long long)L);
      append_error = buf;
      break;
    }
    for (int32_t i = 0; i < Q; ++i) {
      const int64_t j = L - Q + i;
      const int64_t page = a.kv_indices[a.kv_indptr[b] + j / a.page_size];
      const int64_t r = page * a.page_size + j % a.page_size;
      if (r > INT32_MAX) {
        append_error = "cache rows beyond 2^31 are not addressable by the append";
        break;
      }
      append_rows[a.qo_indptr[b] + i] = static_cast<int32_t>(r);
    }
  }

  const CostModel cm(a.num_heads);
  double total = 0.0;
  for (const TokenWork& tw : toks) total += tw.tiles + cm.item;
  const int32_t W = a.num_workers;

  // The pool: smallest whole-token items first, up to kPoolShare of the
  // work; then ordered largest first.  The static lists take the rest, in
  // token order.
  std::vector<TokenWork> pool;
  if (static_cast<int64_t>(toks.size()) >= int64_t(kPoolMinTokensPerWorker) * W) {
    const double cap = total / W / kPoolItemDiv;
    std::vector<int32_t> order;
    order.reserve(toks.size());
    for (int32_t i = 0; i < static_cast<int32_t>(toks.size()); ++i)
      if (toks[i].tiles + cm.item <= cap && toks[i].tiles <= kMaxItemTiles) order.push_back(i);
    std::stable_sort(order.begin(), order.end(),
                     [&](int32_t x, int32_t y) { return toks[x].tiles < toks[y].tiles; });
    std::vector<char> in_pool(toks.size(), 0);
    double pooled = 0.0;
    for (const int32_t i : order) {
      const double c = toks[i].tiles + cm.item;
      if (pooled + c > kPoolShare * total) break;
      pooled += c;
      in_pool[i] = 1;
    }
    if (pooled > 0.0) {
      std::vector<TokenWork> rest;
      rest.reserve(toks.size());
      for (size_t i = 0; i < toks.size(); ++i) (in_pool[i] ? pool : rest).push_back(toks[i]);
      std::stable_sort(pool.begin(), pool.end(),
                       [](const TokenWork& x, const TokenWork& y) { return x.tiles > y.tiles; });
      toks.swap(rest);
      total -= pooled;
    }
  }
  // Smallest per-worker budget whose greedy fill fits on W workers (split
  // costs are only known after a fill, so search for it).
  std::vector<WorkItem> items;
  std::vector<int32_t> first;
  double max_load = 0.0;
  double lo = std::max(total / W, 4.0 + cm.item);
  double hi = lo;
  auto fits = [&](double budget) {
    fill<false>(toks, cm, budget, W, nullptr, nullptr, &max_load);
    return max_load <= budget + kMinPieceTiles;
  };
  while (!fits(hi)) hi *= 1.25;
  for (int iter = 0; iter < 24 && hi - lo > 0.5; ++iter) {
    const double mid = 0.5 * (lo + hi);
    if (fits(mid)) hi = mid; else lo = mid;
  }
  items.reserve(toks.size() + pool.size() + 2 * static_cast<size_t>(W));
  fill<true>(toks, cm, hi, W, &items, &first, &max_load);
  const size_t n_static = items.size();
  for (const TokenWork& tw : pool)
    items.push_back(WorkItem{tw.token, tw.row, 0, tw.visible, -1, 0, {0, 0}});

  // Partial slots: tokens that ended up in more than one item.
  std::vector<int32_t> pieces(static_cast<size_t>(T), 0);
  for (const WorkItem& it : items) ++pieces[it.token];
  std::vector<int32_t> first_slot(static_cast<size_t>(T), -1);
  std::vector<int32_t> next_slot(static_cast<size_t>(T), 0);
  Schedule s;
  int64_t slots = 0;
  for (int64_t t = 0; t < T; ++t) {
    if (pieces[t] > 1) {
      first_slot[t] = static_cast<int32_t>(slots);
      s.merges.push_back(MergeItem{static_cast<int32_t>(t), static_cast<int32_t>(slots), pieces[t], 0});
      slots += pieces[t];
    }
  }
  for (WorkItem& it : items) {
    it.page_base = a.kv_indptr[it.row];
    if (pieces[it.token] > 1) {
      it.slot = first_slot[it.token] + next_slot[it.token]++;
    } else {
      it.slot = -1;
    }
  }

  // Launch order: workgroups are dispatched round-robin over the 8 XCDs of
  // the device (each with its own L2), so consecutive logical workers (which
  // hold neighbouring tokens of the same row, and thus the same keys) are
  // placed on the same XCD.
  constexpr int kXcds = 8;
  std::vector<int32_t> logical_of(W);
  if (W % kXcds == 0) {
    const int per = W / kXcds;
    for (int p = 0; p < W; ++p) logical_of[p] = (p % kXcds) * per + p / kXcds;
  } else {
    for (int p = 0; p < W; ++p) logical_of[p] = p;
  }
  s.worker_indptr.assign(W + 2, 0);
  for (int p = 0; p < W; ++p) {
    const int l = logical_of[p];
    s.worker_indptr[p + 1] = s.worker_indptr[p] + (first[l + 1] - first[l]);
    s.items.insert(s.items.end(), items.begin() + first[l], items.begin() + first[l + 1]);
  }
  s.items.insert(s.items.end(), items.begin() + n_static, items.end());
  s.worker_indptr[W + 1] = static_cast<int32_t>(s.items.size());
  s.append_rows = std::move(append_rows);
  s.append_error = std::move(append_error);
  s.num_workers = W;
  s.batch = B;
  s.num_tokens = T;
  s.num_slots = slots;
  s.nnz = nnz;
  *out = std::move(s);
  return MLA_OK;
}

mla_status check_append(const Schedule& s) {
  if (!s.append_error.empty()) return fail(MLA_E_INVALID, s.append_error);
  std::vector<int32_t> rows(s.append_rows);
  std::sort(rows.begin(), rows.end());
  const auto dup = std::adjacent_find(rows.begin(), rows.end());
  if (dup != rows.end()) {
    char buf[128];
    std::snprintf(buf, sizeof buf, "two query tokens append into cache row %d", *dup);
    return fail(MLA_E_INVALID, buf);
  }
  return MLA_OK;
}

}  // namespace mla

// ---------------------------------------------------------------------------
// C ABI: host-only schedule, status strings, last error.
// ---------------------------------------------------------------------------

struct mla_schedule_s {
  mla::Schedule s;
};

extern "C" {

const char* mla_status_str(mla_status status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_E_INVALID: return "invalid argument";
    case MLA_E_UNSUPPORTED: return "unsupported shape";
    case MLA_E_STATE: return "invalid call order";
    case MLA_E_HIP: return "HIP runtime error";
    case MLA_E_NOMEM: return "out of memory";
  }
  return "unknown status";
}

const char* mla_last_error(void) { return mla::g_last_error.c_str(); }

mla_status mla_schedule_build(mla_schedule_t* out, const int32_t* qo_indptr,
                              const int32_t* kv_indptr, const int32_t* kv_indices,
                              const int32_t* kv_last_page_len, int32_t batch, int32_t causal,
                              int32_t page_size, int64_t num_cache_pages, int32_t num_heads,
                              int32_t num_workers) {
  mla::clear_last_error();
  if (!out) return mla::fail(MLA_E_INVALID, "NULL output handle");
  mla::PlanArgs a{qo_indptr, kv_indptr, kv_indices, kv_last_page_len, batch, causal != 0,
                  page_size, num_cache_pages, num_heads, num_workers};
  auto* h = new (std::nothrow) mla_schedule_s;
  if (!h) return mla::fail(MLA_E_NOMEM, "host allocation failed");
  mla_status st;
  try {
    st = mla::build_schedule(a, &h->s);
  } catch (const std::bad_alloc&) {
    st = mla::fail(MLA_E_NOMEM, "host allocation failed");
  }
  if (st != MLA_OK) {
    delete h;
    return st;
  }
  *out = h;
  return MLA_OK;
}

void mla_schedule_sizes(mla_schedule_t s, int32_t* num_workers, int64_t* num_items,
                        int64_t* num_merges, int64_t* num_slots) {
  if (!s) return;
  if (num_workers) *num_workers = s->s.num_workers;
  if (num_items) *num_items = static_cast<int64_t>(s->s.items.size());
  if (num_merges) *num_merges = static_cast<int64_t>(s->s.merges.size());
  if (num_slots) *num_slots = s->s.num_slots;
}

void mla_schedule_copy(mla_schedule_t s, int32_t* worker_indptr, int32_t* items,
                       int32_t* merges) {
  if (!s) return;
  if (worker_indptr)
    std::memcpy(worker_indptr, s->s.worker_indptr.data(),
                s->s.worker_indptr.size() * sizeof(int32_t));
  if (items && !s->s.items.empty())
    std::memcpy(items, s->s.items.data(), s->s.items.size() * sizeof(mla::WorkItem));
  if (merges && !s->s.merges.empty())
    std::memcpy(merges, s->s.merges.data(), s->s.merges.size() * sizeof(mla::MergeItem));
}

mla_status mla_schedule_append_rows(mla_schedule_t s, int32_t* rows) {
  mla::clear_last_error();
  if (!s) return mla::fail(MLA_E_INVALID, "NULL schedule");
  const mla_status st = mla::check_append(s->s);
  if (st != MLA_OK) return st;
  if (rows && !s->s.append_rows.empty())
    std::memcpy(rows, s->s.append_rows.data(), s->s.append_rows.size() * sizeof(int32_t));
  return MLA_OK;
}

void mla_schedule_destroy(mla_schedule_t s) { delete s; }

}  // extern "C"
