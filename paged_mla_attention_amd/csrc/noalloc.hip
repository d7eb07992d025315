// mla_run_noalloc: paged latent attention in one call that allocates
// nothing, for callers that cannot call hipMalloc (code under HIP graph
// capture, tight serving loops, harnesses that forbid it).
//
// It computes what mla_plan + mla_run compute, with the page table in device
// memory.  Everything beyond the caller's inputs and outputs lives in one
// fixed file-scope device array, `scratch`: the schedule (work items, split
// merges, per-worker ranges), the planning temporaries and the split-KV
// partial results.  Three kernels run on the caller's stream:
//   1. na_plan_kernel (one workgroup) validates the page table on the device
//      and cuts the (token, key tile) stream into one contiguous share of
//      equal cost per worker; a token whose tiles straddle a share boundary
//      becomes several items whose partial results are merged;
//   2. the attention kernel of mla_run, reading that schedule;
//   3. the split-KV merge kernel of mla_run.
//
// `scratch` is one array per GPU, shared by every call on that GPU: calls
// that overlap on one GPU (on different streams, or from several threads
// without ordering) race on it.  Calls ordered on one stream do not.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <mutex>

#include "kernels.h"
#include "planner.h"

namespace mla {
namespace {

constexpr int kNaMaxWorkers = 1024;
constexpr int kNaMaxBatch = 8192;
constexpr int kNaMaxTokens = 8192;
constexpr int kNaMaxItems = 16384;
constexpr size_t kNaPartBytes = size_t(80) << 20;  // split-KV partials
constexpr int kNaMaxDevices = 64;

constexpr size_t na_align(size_t x) { return (x + 255) / 256 * 256; }
// Byte offsets of the sections of `scratch`.
constexpr size_t kOffHdr = 0;  // int32 [0] unused, [1] merge count, [2] status (1: table rejected)
constexpr size_t kOffWi = 256;                                             // int32 [W + 2]
constexpr size_t kOffItems = kOffWi + na_align(4 * (kNaMaxWorkers + 2));   // WorkItem [items]
constexpr size_t kOffMerges = kOffItems + na_align(sizeof(WorkItem) * kNaMaxItems);
constexpr size_t kOffTokRow = kOffMerges + na_align(sizeof(MergeItem) * kNaMaxTokens);
constexpr size_t kOffTokTiles = kOffTokRow + na_align(4 * kNaMaxTokens);
constexpr size_t kOffTokVis = kOffTokTiles + na_align(4 * kNaMaxTokens);
constexpr size_t kOffTokCost = kOffTokVis + na_align(4 * kNaMaxTokens);    // int64
constexpr size_t kOffTokItems = kOffTokCost + na_align(8 * kNaMaxTokens);  // int64 (scanned)
constexpr size_t kOffTokSlots = kOffTokItems + na_align(8 * kNaMaxTokens);
constexpr size_t kOffTokMerge = kOffTokSlots + na_align(8 * kNaMaxTokens);
constexpr size_t kOffPart = kOffTokMerge + na_align(8 * kNaMaxTokens);
constexpr size_t kScratchBytes = kOffPart + kNaPartBytes;

}  // namespace

// The workspace of mla_run_noalloc (one copy per GPU, for the process's life).
// Host code never names it as an address: it uses the per-device pointer
// hipGetSymbolAddress returns.
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

// Cost units of the split: a key tile costs kTileCost, a work item's fixed
// part (query load, pipeline fill, output) about 1 + 6 H / 128 tiles.
constexpr int kTileCost = 8;

struct NaPlanArgs {
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* last;
  int32_t batch;
  int32_t num_tokens;
  int64_t num_kv_indices;
  int64_t num_cache_pages;
  int32_t page_size;
  int32_t causal;
  int32_t max_kv_len;
  int32_t num_workers;
  int32_t item_cost;
  int32_t cap_slots;
  char* ws;  // device address of `scratch`
};

constexpr int kPlanThreads = 1024;

// Exclusive prefix sum of v[0 .. n) in place (one workgroup of kPlanThreads);
// returns the total to every thread.
__device__ int64_t block_exclusive_scan(int64_t* v, int n, int64_t* sh) {
  const int tid = threadIdx.x;
  int64_t carry = 0;
  for (int base = 0; base < n; base += kPlanThreads) {
    const int i = base + tid;
    const int64_t x = i < n ? v[i] : 0;
    sh[tid] = x;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
      const int64_t add = tid >= off ? sh[tid - off] : 0;
      __syncthreads();
      sh[tid] += add;
      __syncthreads();
    }
    if (i < n) v[i] = carry + sh[tid] - x;
    const int64_t chunk = sh[kPlanThreads - 1];
    __syncthreads();
    carry += chunk;
  }
  return carry;
}

// The tiles of a token (cost position `start`, `tiles` tiles after its
// fixed part) fall to workers by the centre of each tile: worker
// floor(centre / beta).  Calls f(worker, first tile, end tile) for each
// non-empty worker range, in order.
template <typename F>
__device__ void for_each_range(int64_t start, int tiles, int item_cost, double beta, int W, F&& f) {
  auto worker_of = [&](int j) {
    const double c = static_cast<double>(start + item_cost) + kTileCost * (j + 0.5);
    const int w = static_cast<int>(floor(c / beta));
    return w < 0 ? 0 : (w >= W ? W - 1 : w);
  };
  int j0 = 0;
  int w = worker_of(0);
  while (j0 < tiles) {
    // last tile of worker w: binary search over [j0, tiles)
    int lo = j0, hi = tiles - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (worker_of(mid) <= w) lo = mid; else hi = mid - 1;
    }
    f(w, j0, lo + 1);
    j0 = lo + 1;
    if (j0 < tiles) w = worker_of(j0);
  }
}

__global__ __launch_bounds__(kPlanThreads) void na_plan_kernel(NaPlanArgs a) {
  __shared__ int64_t sh[kPlanThreads];
  __shared__ int counts[kNaMaxWorkers];
  __shared__ int lfirst[kNaMaxWorkers];
  __shared__ int bad;
  const int tid = threadIdx.x;
  const int B = a.batch, T = a.num_tokens, W = a.num_workers, P = a.page_size;
  char* ws = a.ws;
  int32_t* hdr = reinterpret_cast<int32_t*>(ws + kOffHdr);
  int32_t* wi = reinterpret_cast<int32_t*>(ws + kOffWi);
  WorkItem* items = reinterpret_cast<WorkItem*>(ws + kOffItems);
  MergeItem* merges = reinterpret_cast<MergeItem*>(ws + kOffMerges);
  int32_t* tok_row = reinterpret_cast<int32_t*>(ws + kOffTokRow);
  int32_t* tok_tiles = reinterpret_cast<int32_t*>(ws + kOffTokTiles);
  int32_t* tok_vis = reinterpret_cast<int32_t*>(ws + kOffTokVis);
  int64_t* tok_cost = reinterpret_cast<int64_t*>(ws + kOffTokCost);
  int64_t* tok_items = reinterpret_cast<int64_t*>(ws + kOffTokItems);
  int64_t* tok_slots = reinterpret_cast<int64_t*>(ws + kOffTokSlots);
  int64_t* tok_merge = reinterpret_cast<int64_t*>(ws + kOffTokMerge);

  // 1. The page-table rules mla_plan checks, on the device.
  if (tid == 0) bad = 0;
  __syncthreads();
  if (tid == 0 && (a.qo_indptr[0] != 0 || a.kv_indptr[0] != 0 || a.qo_indptr[B] != T ||
                   a.kv_indptr[B] > a.num_kv_indices))
    bad = 1;
  for (int b = tid; b < B; b += kPlanThreads) {
    const int32_t q0 = a.qo_indptr[b], q1 = a.qo_indptr[b + 1];
    const int32_t k0 = a.kv_indptr[b], k1 = a.kv_indptr[b + 1];
    const int32_t n = k1 - k0, last = a.last[b];
    const int64_t L = n > 0 ? int64_t(n - 1) * P + last : 0;
    if (q1 < q0 || k1 < k0 || (n > 0 && (last < 1 || last > P)) || L > a.max_kv_len) bad = 1;
  }
  __syncthreads();
  if (!bad) {
    const int64_t nnz = a.kv_indptr[B];
    for (int64_t i = tid; i < nnz; i += kPlanThreads) {
      const int32_t pg = a.kv_indices[i];
      if (pg < 0 || pg >= a.num_cache_pages) bad = 1;
    }
  }
  __syncthreads();

  // 2. Per token: its row, visible keys, tiles and cost.  A rejected table
  // is planned as one empty item per token (zero output, -inf LSE).
  for (int t = tid; t < T; t += kPlanThreads) {
    int row = 0, vis = 0;
    if (!bad) {
      int lo = 0, hi = B - 1;  // last row with qo_indptr[row] <= t
      while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (a.qo_indptr[mid] <= t) lo = mid; else hi = mid - 1;
      }
      row = lo;
      const int32_t n = a.kv_indptr[row + 1] - a.kv_indptr[row];
      const int64_t L = n > 0 ? int64_t(n - 1) * P + a.last[row] : 0;
      const int64_t Q = a.qo_indptr[row + 1] - a.qo_indptr[row];
      const int64_t i = t - a.qo_indptr[row];
      int64_t v = L;
      if (a.causal) v = min(L, max(int64_t(0), i + L - Q + 1));
      vis = static_cast<int>(v);
    }
    const int tiles = (vis + kTileKeys - 1) / kTileKeys;
    tok_row[t] = row;
    tok_vis[t] = vis;
    tok_tiles[t] = tiles;
    tok_cost[t] = a.item_cost + int64_t(kTileCost) * tiles;
  }
  __syncthreads();
  const int64_t total = block_exclusive_scan(tok_cost, T, sh);  // -> cost position of each token
  // Cost per worker; at least a few tiles past an item's fixed part, so a
  // small batch is not cut into one-tile pieces (its later workers idle).
  const double beta = fmax(static_cast<double>(total) / W, 4.0 * kTileCost + a.item_cost);

  // 3. Items per token: one per worker range, cut again at kMaxItemTiles.
  for (int t = tid; t < T; t += kPlanThreads) {
    int64_t n = 0;
    if (tok_tiles[t] == 0) {
      n = 1;
    } else {
      for_each_range(tok_cost[t], tok_tiles[t], a.item_cost, beta, W, [&](int, int j0, int j1) {
        n += (j1 - j0 + kMaxItemTiles - 1) / kMaxItemTiles;
      });
    }
    tok_items[t] = n;
    tok_slots[t] = n > 1 ? n : 0;
    tok_merge[t] = n > 1 ? 1 : 0;
  }
  __syncthreads();
  const int64_t n_items = block_exclusive_scan(tok_items, T, sh);
  const int64_t n_slots = block_exclusive_scan(tok_slots, T, sh);
  const int64_t n_merges = block_exclusive_scan(tok_merge, T, sh);
  if (n_items > kNaMaxItems || n_slots > a.cap_slots) {
    // (sizes the host check rules out for a table within its max_kv_len)
    if (tid == 0) bad = 1;
  }
  __syncthreads();
  if (bad) {
    // One empty item per token, spread evenly over the workers.
    for (int p = tid; p <= W; p += kPlanThreads)
      wi[p] = static_cast<int32_t>((static_cast<int64_t>(T) * p) / W);
    if (tid == 0) wi[W + 1] = T;  // (no shared pool)
    for (int t = tid; t < T; t += kPlanThreads)
      items[t] = WorkItem{t, 0, 0, 0, -1, 0, {0, 0}};
    if (tid == 0) {
      hdr[1] = 0;
      hdr[2] = 1;
    }
    return;
  }

  // 4. Items per logical worker, then the workers' order in the launch:
  // workgroups go round-robin over the 8 XCDs, so logical worker l runs as
  // workgroup p(l) = 8 (l % (W/8)) + l / (W/8), which keeps consecutive
  // logical workers (neighbouring tokens of a row) on one XCD's L2.
  for (int k = tid; k < W; k += kPlanThreads) counts[k] = 0;
  __syncthreads();
  for (int t = tid; t < T; t += kPlanThreads) {
    if (tok_tiles[t] == 0) {
      const double c = static_cast<double>(tok_cost[t]) + 0.5 * a.item_cost;
      int w = static_cast<int>(floor(c / beta));
      w = w < 0 ? 0 : (w >= W ? W - 1 : w);
      atomicAdd(&counts[w], 1);
    } else {
      for_each_range(tok_cost[t], tok_tiles[t], a.item_cost, beta, W, [&](int w, int j0, int j1) {
        atomicAdd(&counts[w], (j1 - j0 + kMaxItemTiles - 1) / kMaxItemTiles);
      });
    }
  }
  __syncthreads();
  const bool xcd = W % 8 == 0;
  const int per = W / 8;
  auto phys_of = [&](int l) { return xcd ? 8 * (l % per) + l / per : l; };
  auto logical_of = [&](int p) { return xcd ? (p % 8) * per + p / 8 : p; };
  // lfirst: first global item of each logical worker; wi: per workgroup
  if (tid == 0) {
    int acc = 0;
    for (int k = 0; k < W; ++k) {
      lfirst[k] = acc;
      acc += counts[k];
    }
    acc = 0;
    for (int p = 0; p < W; ++p) {
      wi[p] = acc;
      acc += counts[logical_of(p)];
    }
    wi[W] = acc;
    wi[W + 1] = acc;  // (no shared pool)
    hdr[1] = static_cast<int32_t>(n_merges);
    hdr[2] = 0;
  }
  __syncthreads();

  // 5. The items, at their workgroup's place, and the merge entries.
  for (int t = tid; t < T; t += kPlanThreads) {
    const int row = tok_row[t];
    const int32_t base = a.kv_indptr[row];
    int64_t i = tok_items[t];
    const int64_t n = (t + 1 < T ? tok_items[t + 1] : n_items) - i;
    const int32_t slot0 = n > 1 ? static_cast<int32_t>(tok_slots[t]) : -1;
    int piece = 0;
    auto put = [&](int w, int kb, int ke) {
      const int64_t dst = wi[phys_of(w)] + (i - lfirst[w]);
      items[dst] = WorkItem{t, row, kb, ke, slot0 >= 0 ? slot0 + piece : -1, base, {0, 0}};
      ++i;
      ++piece;
    };
    if (tok_tiles[t] == 0) {
      const double c = static_cast<double>(tok_cost[t]) + 0.5 * a.item_cost;
      int w = static_cast<int>(floor(c / beta));
      w = w < 0 ? 0 : (w >= W ? W - 1 : w);
      put(w, 0, 0);
    } else {
      const int vis = tok_vis[t];
      for_each_range(tok_cost[t], tok_tiles[t], a.item_cost, beta, W, [&](int w, int j0, int j1) {
        for (int j = j0; j < j1; j += kMaxItemTiles) {
          const int je = min(j1, j + kMaxItemTiles);
          put(w, j * kTileKeys, min(vis, je * kTileKeys));
        }
      });
    }
    if (n > 1)
      merges[tok_merge[t]] = MergeItem{t, slot0, static_cast<int32_t>(n), 0};
  }
}

struct DeviceScratch {
  char* ptr = nullptr;
  int workers = 0;
};
DeviceScratch g_dev[kNaMaxDevices];
std::mutex g_dev_mu;

mla_status na_fail(mla_status s, const char* msg) {
  set_last_error(msg);
  return s;
}

}  // namespace

}  // namespace mla

extern "C" mla_status mla_run_noalloc(const int32_t* qo_indptr, const int32_t* kv_indptr,
                                      const int32_t* kv_indices, const int32_t* kv_last_page_len,
                                      int32_t batch, int64_t num_tokens, int64_t num_kv_indices,
                                      int32_t causal, float sm_scale, int64_t num_cache_pages,
                                      int32_t max_kv_len, int32_t num_heads, int32_t page_size,
                                      const void* q_nope, const void* q_pe, const void* kv_cache,
                                      void* out, float* lse, mla_stream_t stream_) {
  using namespace mla;
  clear_last_error();
  char buf[256];
  if (num_heads < 1 || num_heads > kMaxHeads)
    return na_fail(MLA_E_UNSUPPORTED, "num_heads must be in [1, 128]");
  if (page_size < 1) return na_fail(MLA_E_INVALID, "page_size must be >= 1");
  if (!(std::isfinite(sm_scale) && sm_scale > 0.f))
    return na_fail(MLA_E_INVALID, "sm_scale must be finite and positive");
  if (batch < 0 || num_tokens < 0 || num_kv_indices < 0 || num_cache_pages < 0 || max_kv_len < 0)
    return na_fail(MLA_E_INVALID, "negative size");
  // (cache rows, page * page_size + slot, are addressed in 32 bits)
  if (num_cache_pages > (int64_t(INT32_MAX) + 1) / page_size)
    return na_fail(MLA_E_UNSUPPORTED, "num_cache_pages * page_size exceeds 2^31 cache rows");
  if (batch > kNaMaxBatch || num_tokens > kNaMaxTokens) {
    std::snprintf(buf, sizeof buf,
                  "mla_run_noalloc takes at most %d rows and %d query tokens (got %d, %lld)",
                  kNaMaxBatch, kNaMaxTokens, batch, static_cast<long long>(num_tokens));
    return na_fail(MLA_E_INVALID, buf);
  }
  if (num_tokens == 0) return MLA_OK;
  if (batch == 0) return na_fail(MLA_E_INVALID, "query tokens without rows");
  if (!qo_indptr || !kv_indptr || !kv_last_page_len || !q_nope || !q_pe || !out)
    return na_fail(MLA_E_INVALID, "NULL pointer");
  if (num_kv_indices > 0 && (!kv_indices || !kv_cache))
    return na_fail(MLA_E_INVALID, "NULL kv_indices or kv_cache");

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return na_fail(MLA_E_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kNaMaxDevices) return na_fail(MLA_E_UNSUPPORTED, "device index too large");
  DeviceScratch ds;
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (!g_dev[dev].ptr) {
      // Once per device, with that device current: the device address of
      // this GPU's copy of `scratch`.
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) {
        std::snprintf(buf, sizeof buf, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        return na_fail(MLA_E_HIP, buf);
      }
      int cus = 0;
      e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (e != hipSuccess) return na_fail(MLA_E_HIP, hipGetErrorString(e));
      g_dev[dev].workers = cus < 1 ? 1 : (cus > kNaMaxWorkers ? kNaMaxWorkers : cus);
      g_dev[dev].ptr = static_cast<char*>(p);
    }
    ds = g_dev[dev];
  }
  const int W = ds.workers;
  // Worst case of the schedule for rows of at most max_kv_len keys: every
  // share boundary splits one token in two, and a token with more than
  // kMaxItemTiles tiles is cut at every kMaxItemTiles.
  const int64_t max_tiles = (int64_t(max_kv_len) + kTileKeys - 1) / kTileKeys;
  const int64_t long_cuts = max_tiles > kMaxItemTiles ? (max_tiles - 1) / kMaxItemTiles : 0;
  const int64_t worst_items = num_tokens * (1 + long_cuts) + W;
  const int64_t worst_slots = 2 * int64_t(W) + num_tokens * (long_cuts > 0 ? 1 + long_cuts : 0);
  const int64_t slot_bytes = int64_t(num_heads) * (kLoraRank * 2 + 4);
  const int64_t cap_slots = static_cast<int64_t>(kNaPartBytes) / slot_bytes;
  if (worst_items > kNaMaxItems || worst_slots > cap_slots) {
    std::snprintf(buf, sizeof buf,
                  "mla_run_noalloc: %lld tokens with up to %d keys need up to %lld work items and "
                  "%lld partial slots; its fixed workspace holds %d items and %lld slots at %d heads",
                  static_cast<long long>(num_tokens), max_kv_len, static_cast<long long>(worst_items),
                  static_cast<long long>(worst_slots), kNaMaxItems, static_cast<long long>(cap_slots),
                  num_heads);
    return na_fail(MLA_E_INVALID, buf);
  }

  hipStream_t stream = static_cast<hipStream_t>(stream_);
  char* ws = ds.ptr;
  NaPlanArgs pa{};
  pa.qo_indptr = qo_indptr;
  pa.kv_indptr = kv_indptr;
  pa.kv_indices = kv_indices;
  pa.last = kv_last_page_len;
  pa.batch = batch;
  pa.num_tokens = static_cast<int32_t>(num_tokens);
  pa.num_kv_indices = num_kv_indices;
  pa.num_cache_pages = num_cache_pages;
  pa.page_size = page_size;
  pa.causal = causal != 0;
  pa.max_kv_len = max_kv_len;
  pa.num_workers = W;
  pa.item_cost = static_cast<int32_t>(std::lround(kTileCost * (1.0 + 6.0 * num_heads / 128.0)));
  pa.cap_slots = static_cast<int32_t>(cap_slots);
  pa.ws = ws;
  hipLaunchKernelGGL(na_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, pa);
  e = hipGetLastError();
  if (e != hipSuccess) return na_fail(MLA_E_HIP, hipGetErrorString(e));

  const int64_t slots_h = cap_slots * num_heads;
  AttnArgs a{};
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.kv_cache = static_cast<const uint16_t*>(kv_cache);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.part_o = reinterpret_cast<uint16_t*>(ws + kOffPart);
  a.part_lse = reinterpret_cast<float*>(ws + kOffPart + slots_h * kLoraRank * 2);
  a.worker_indptr = reinterpret_cast<const int32_t*>(ws + kOffWi);
  a.items = reinterpret_cast<const WorkItem*>(ws + kOffItems);
  a.kv_indptr = kv_indptr;
  a.kv_indices = kv_indices;
  a.num_heads = num_heads;
  a.page_size = page_size;
  a.scale_log2 = sm_scale * 1.44269504088896340736f;
  a.out_scale = 1.f;
  e = launch_attention(a, W, stream);
  if (e != hipSuccess) return na_fail(MLA_E_HIP, hipGetErrorString(e));

  SplitMergeArgs m{};
  m.part_o = a.part_o;
  m.part_lse = a.part_lse;
  m.merges = reinterpret_cast<const MergeItem*>(ws + kOffMerges);
  m.out = a.out;
  m.lse = lse;
  m.num_heads = num_heads;
  // (the grid covers the most merges the schedule can hold, each of at least
  // two slots; the live count is the plan kernel's)
  m.num_merges = static_cast<int32_t>(std::min<int64_t>(num_tokens, worst_slots / 2));
  m.num_merges_ptr = reinterpret_cast<const int32_t*>(ws + kOffHdr) + 1;
  e = launch_split_merge(m, stream);
  if (e != hipSuccess) return na_fail(MLA_E_HIP, hipGetErrorString(e));
  return MLA_OK;
}
