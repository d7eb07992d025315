// C ABI of the library (include/mla.h): plan objects, the host-to-device
// schedule copy with its staging fence, and the kernel launches.
//
// The staging fences follow the hazard the m-star page
// "mstar.engine.resources.attn.flashinfer_mla" describes under
// FlashInferMLAManager.force_double_buffer: a plan that stages into a reused
// host buffer without blocking must not overwrite that buffer before its
// previous contents have been consumed.  Plans alternate between two pinned
// host slots.  A small schedule (at most two items per worker, as in
// decode) is read by the kernels straight from its pinned slot, which saves
// the upload that would otherwise sit between two steps' kernels; a larger
// one, and every schedule of a plan with reserved capacity, is copied to
// the device buffer on the plan's stream.  Before refilling a slot, a plan
// waits for the last copy from it (an event) and the last run that read it
// (flags the attention workgroups store).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <thread>
#include <vector>

#include "host_wait.h"
#include "kernels.h"
#include "planner.h"

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

mla_status hip_fail(hipError_t e, const char* what) {
  char buf[256];
  std::snprintf(buf, sizeof buf, "%s: %s", what, hipGetErrorString(e));
  mla::set_last_error(buf);
  return e == hipErrorOutOfMemory ? MLA_E_NOMEM : MLA_E_HIP;
}

mla_status fail(mla_status s, const char* msg) {
  mla::set_last_error(msg);
  return s;
}

// Makes `dev` current for the scope and restores the caller's device.
struct DeviceGuard {
  int prev = -1;
  hipError_t err = hipSuccess;
  explicit DeviceGuard(int dev) {
    err = hipGetDevice(&prev);
    if (err == hipSuccess && prev != dev) err = hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

}  // namespace

struct mla_plan_s {
  int device = 0;
  int num_heads = 0;
  int page_size = 0;
  int num_workers = 0;
  int cus = 0;  // compute units of the device

  bool planned = false;
  // The last successful plan's inputs (the plan cache key of the page
  // "mstar.engine.resources.attn.base", PlanCacheKey: an unchanged plan need
  // not be rebuilt).  An identical mla_plan keeps the schedule, its staging
  // slot and its device copy as they are.
  struct Key {
    int32_t batch = -1, causal = 0;
    float sm_scale = 0.f;
    int64_t num_cache_pages = 0;
    std::vector<int32_t> qo, kvp, idx, last;
  } key;
  float scale_log2 = 0.f;
  mla::Schedule sched;

  // Pinned host staging slots and the device mirror: [reserved-plan header]
  // | worker_indptr | items | merges | kv_indptr | kv_indices | append rows
  // | [first items | first page lists, for host-slot schedules], each
  // section 256-byte aligned.
  struct HostSlot {
    char* h_stage = nullptr;
    size_t cap = 0;
    hipEvent_t done = nullptr;  // after the last copy from / run reading the slot
    bool pending = false;
    // Runs that read the schedule straight from this slot: each attention
    // workgroup stores the run's sequence number here when done with it.
    int32_t* flags = nullptr;   // pinned [num_workers]
    int32_t wait_seq = 0;       // > 0: wait for every flag to reach it
  };
  HostSlot slot[2];
  int cur = 0;              // slot of the current plan
  bool direct = false;      // the kernels read the schedule from the host slot
  char* d_stage = nullptr;
  size_t d_stage_cap = 0;
  size_t off_wi = 0, off_items = 0, off_merges = 0, off_kv_indptr = 0, off_kv_indices = 0,
         off_append = 0;
  int append_checked = 0;  // 0: not yet, 1: no slot collision, -1: rejected
  int32_t run_seq = 0;     // sequence number of the last mla_run
  // Reserved capacity (mla_plan_reserve): every section at a fixed offset of
  // the device buffer, the per-plan scalars in a header (scale_log2,
  // num_merges), so kernels captured once read whatever batch was planned
  // last.
  bool reserved = false;
  int32_t cap_batch = 0;
  int64_t cap_tokens = 0, cap_nnz = 0, cap_items = 0, cap_merges = 0;
  size_t off_first = 0, off_fpages = 0;  // host-slot schedules, page size a multiple of 32
  bool first_fast = false;

  // Split-KV partials: bf16 o [slots, H, 512] (normalised by the piece's own
  // denominator), then fp32 lse [slots, H].
  float* d_part = nullptr;
  size_t part_cap = 0;  // 4-byte words
  // Shared-pool counters (next item, workgroups done): zeroed once here,
  // left at zero by every run's last workgroup.
  int32_t* d_pool = nullptr;

};

namespace {

// Whether a plan call repeats the last successful one exactly.
bool same_key(const mla_plan_s::Key& k, const int32_t* qo, const int32_t* kvp, const int32_t* idx,
              const int32_t* last, int32_t batch, int32_t causal, float sm_scale,
              int64_t num_cache_pages) {
  if (k.batch != batch || k.causal != (causal != 0) || num_cache_pages != k.num_cache_pages ||
      std::memcmp(&k.sm_scale, &sm_scale, sizeof(float)) != 0)
    return false;
  if (batch == 0) return true;
  if (!qo || !kvp || !last) return false;
  const auto eq = [](const std::vector<int32_t>& v, const int32_t* a, size_t n) {
    return v.size() == n && (n == 0 || (a && std::memcmp(v.data(), a, n * sizeof(int32_t)) == 0));
  };
  return eq(k.qo, qo, batch + 1) && eq(k.kvp, kvp, batch + 1) && eq(k.last, last, batch) &&
         kvp[batch] >= 0 && eq(k.idx, idx, static_cast<size_t>(kvp[batch]));
}

// Waits until every attention workgroup of the run that last read `sl` from
// the host has stored its sequence number (or a later one), for at most
// kSlotWaitTimeoutS.  On time-out the slot stays marked as in use and the
// call fails with MLA_E_HIP.
mla_status wait_flags(const mla_plan_s* p, mla_plan_s::HostSlot& sl) {
  int late = -1;
  if (!mla::wait_for_flags(sl.flags, p->num_workers, sl.wait_seq, mla::kSlotWaitTimeoutS, &late)) {
    char buf[256];
    std::snprintf(buf, sizeof buf,
                  "run %d reading staging slot %d has not finished after %.0f s (workgroup %d)",
                  static_cast<int>(sl.wait_seq), static_cast<int>(&sl - p->slot), mla::kSlotWaitTimeoutS,
                  late);
    mla::set_last_error(buf);
    return MLA_E_HIP;
  }
  sl.wait_seq = 0;
  return MLA_OK;
}

void release(mla_plan_s* p) {
  for (auto& sl : p->slot) {
    if (sl.pending) (void)hipEventSynchronize(sl.done);
    // A slot that a run may still read is leaked rather than freed under it.
    const bool busy = sl.wait_seq > 0 && wait_flags(p, sl) != MLA_OK;
    if (sl.done) (void)hipEventDestroy(sl.done);
    if (sl.h_stage && !busy) (void)hipHostFree(sl.h_stage);
    if (sl.flags && !busy) (void)hipHostFree(sl.flags);
  }
  if (p->d_stage) (void)hipFree(p->d_stage);
  if (p->d_part) (void)hipFree(p->d_part);
  if (p->d_pool) (void)hipFree(p->d_pool);
  delete p;
}

}  // namespace

extern "C" {

mla_status mla_plan_create(mla_plan_t* out, int32_t device, int32_t num_heads,
                           int32_t kv_lora_rank, int32_t qk_rope_head_dim, int32_t page_size) {
  mla::clear_last_error();
  if (!out) return fail(MLA_E_INVALID, "NULL output handle");
  *out = nullptr;
  if (kv_lora_rank != mla::kLoraRank || qk_rope_head_dim != mla::kRopeDim)
    return fail(MLA_E_UNSUPPORTED, "only kv_lora_rank 512 with qk_rope_head_dim 64 is supported");
  if (num_heads < 1 || num_heads > mla::kMaxHeads)
    return fail(MLA_E_UNSUPPORTED, "num_heads must be in [1, 128]");
  if (page_size < 1) return fail(MLA_E_INVALID, "page_size must be >= 1");
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
  if (device < 0 || device >= count) return fail(MLA_E_INVALID, "device index out of range");
  DeviceGuard g(device);
  if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  auto* p = new (std::nothrow) mla_plan_s;
  if (!p) return fail(MLA_E_NOMEM, "host allocation failed");
  p->device = device;
  p->num_heads = num_heads;
  p->page_size = page_size;
  p->cus = cus > 0 ? cus : 1;
  // One-wave kernels (at most 32 heads) run two workgroups per compute
  // unit, so the planner balances over twice the units.
  p->num_workers = p->cus * (num_heads <= 32 ? 2 : 1);
  for (auto& sl : p->slot) {
    e = hipEventCreateWithFlags(&sl.done, hipEventDisableTiming);
    if (e != hipSuccess) {
      release(p);
      return hip_fail(e, "hipEventCreate");
    }
    e = hipHostMalloc(reinterpret_cast<void**>(&sl.flags), p->num_workers * sizeof(int32_t),
                      hipHostMallocCoherent);
    if (e != hipSuccess) {
      release(p);
      return hip_fail(e, "hipHostMalloc(flags)");
    }
    std::memset(sl.flags, 0, p->num_workers * sizeof(int32_t));
  }
  e = hipMalloc(reinterpret_cast<void**>(&p->d_pool), 4 * sizeof(int32_t));
  if (e == hipSuccess) e = hipMemset(p->d_pool, 0, 4 * sizeof(int32_t));
  if (e == hipSuccess) e = hipDeviceSynchronize();  // (zero before any stream's first run)
  if (e != hipSuccess) {
    release(p);
    return hip_fail(e, "pool counters");
  }
  *out = p;
  return MLA_OK;
}

mla_status mla_plan_reserve(mla_plan_t p, int32_t max_batch, int64_t max_tokens,
                            int64_t max_kv_indices) {
  mla::clear_last_error();
  if (!p) return fail(MLA_E_INVALID, "NULL plan");
  if (max_batch < 1 || max_tokens < 1 || max_kv_indices < 0)
    return fail(MLA_E_INVALID, "reserved sizes must be positive");
  DeviceGuard g(p->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
  const int64_t W = p->num_workers;
  // Items: every token's visible keys (at most a row's keys, at most
  // max_kv_indices pages) cut into pieces of at most kMaxItemTiles tiles, and
  // at most two more per worker where the balance cuts a token.
  const int64_t max_keys = max_kv_indices * p->page_size;
  const int64_t item_keys = int64_t(mla::kTileKeys) * mla::kMaxItemTiles;
  const int64_t per_token = 1 + (max_keys > 0 ? (max_keys - 1) / item_keys : 0);
  if (per_token > (int64_t(1) << 40) / max_tokens)
    return fail(MLA_E_INVALID, "reserved sizes too large");
  const int64_t cap_items = max_tokens * per_token + 2 * W + 8;
  const int64_t cap_merges = std::min<int64_t>(max_tokens, cap_items);
  const size_t total =
      kAlign + align_up((W + 1) * sizeof(int32_t)) + align_up(cap_items * sizeof(mla::WorkItem)) +
      align_up(cap_merges * sizeof(mla::MergeItem)) + align_up((max_batch + 1) * sizeof(int32_t)) +
      align_up((max_kv_indices + mla::kTileKeys) * sizeof(int32_t)) +
      align_up(max_tokens * sizeof(int32_t));
  const size_t part_floats = static_cast<size_t>(cap_items) * p->num_heads * (mla::kLoraRank / 2 + 1);
  // Nothing of an earlier plan may still run while the buffers change.
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
  for (auto& sl : p->slot) {
    if (sl.wait_seq > 0) {
      const mla_status st = wait_flags(p, sl);
      if (st != MLA_OK) return st;
    }
    sl.pending = false;
    if (total > sl.cap) {
      if (sl.h_stage) (void)hipHostFree(sl.h_stage);
      sl.h_stage = nullptr;
      sl.cap = 0;
      e = hipHostMalloc(reinterpret_cast<void**>(&sl.h_stage), total, hipHostMallocDefault);
      if (e != hipSuccess) return hip_fail(e, "hipHostMalloc");
      sl.cap = total;
    }
  }
  if (total > p->d_stage_cap) {
    if (p->d_stage) (void)hipFree(p->d_stage);
    p->d_stage = nullptr;
    p->d_stage_cap = 0;
    e = hipMalloc(reinterpret_cast<void**>(&p->d_stage), total);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(schedule)");
    p->d_stage_cap = total;
  }
  if (part_floats > p->part_cap) {
    if (p->d_part) (void)hipFree(p->d_part);
    p->d_part = nullptr;
    p->part_cap = 0;
    e = hipMalloc(reinterpret_cast<void**>(&p->d_part), part_floats * sizeof(float));
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(partials)");
    p->part_cap = part_floats;
  }
  p->reserved = true;
  p->cap_batch = max_batch;
  p->cap_tokens = max_tokens;
  p->cap_nnz = max_kv_indices;
  p->cap_items = cap_items;
  p->cap_merges = cap_merges;
  p->planned = false;  // plan again into the reserved layout
  p->key = mla_plan_s::Key{};
  return MLA_OK;
}

mla_status mla_plan(mla_plan_t p, const int32_t* qo_indptr, const int32_t* kv_indptr,
                    const int32_t* kv_indices, const int32_t* kv_last_page_len, int32_t batch,
                    int32_t causal, float sm_scale, int64_t num_cache_pages,
                    mla_stream_t stream_) {
  mla::clear_last_error();
  if (!p) return fail(MLA_E_INVALID, "NULL plan");
  if (!(std::isfinite(sm_scale) && sm_scale > 0.f))
    return fail(MLA_E_INVALID, "sm_scale must be finite and positive");
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (p->planned && same_key(p->key, qo_indptr, kv_indptr, kv_indices, kv_last_page_len, batch,
                             causal, sm_scale, num_cache_pages))
    return MLA_OK;
  mla::PlanArgs args{qo_indptr, kv_indptr, kv_indices, kv_last_page_len, batch, causal != 0,
                     p->page_size, num_cache_pages, p->num_heads, p->num_workers};
  mla::Schedule s;
  mla_status st;
  try {
    st = mla::build_schedule(args, &s);
  } catch (const std::bad_alloc&) {
    st = fail(MLA_E_NOMEM, "host allocation failed");
  }
  if (st != MLA_OK) return st;

  DeviceGuard g(p->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");

  const size_t n_wi = s.worker_indptr.size() * sizeof(int32_t);
  const size_t n_items = s.items.size() * sizeof(mla::WorkItem);
  const size_t n_merges = s.merges.size() * sizeof(mla::MergeItem);
  const size_t n_kvp = static_cast<size_t>(s.batch + 1) * sizeof(int32_t);
  // kv_indices plus 32 zeroed spare entries (slack past the last row's
  // pages).
  const size_t n_idx = static_cast<size_t>(s.nnz) * sizeof(int32_t);
  const size_t n_idx_pad = n_idx + mla::kTileKeys * sizeof(int32_t);
  const size_t n_app = s.append_rows.size() * sizeof(int32_t);
  if (p->reserved &&
      (s.batch > p->cap_batch || s.num_tokens > p->cap_tokens || s.nnz > p->cap_nnz ||
       static_cast<int64_t>(s.items.size()) > p->cap_items ||
       static_cast<int64_t>(s.merges.size()) > p->cap_merges || s.num_slots > p->cap_items))
    return fail(MLA_E_INVALID, "batch exceeds the plan's reserved capacity");
  // Section sizes: the schedule's own, or the reserved maxima.
  const size_t z_wi = n_wi;
  const size_t z_items = p->reserved ? p->cap_items * sizeof(mla::WorkItem) : n_items;
  const size_t z_merges = p->reserved ? p->cap_merges * sizeof(mla::MergeItem) : n_merges;
  const size_t z_kvp = p->reserved ? (p->cap_batch + 1) * sizeof(int32_t) : n_kvp;
  const size_t z_idx = p->reserved ? (p->cap_nnz + mla::kTileKeys) * sizeof(int32_t) : n_idx_pad;
  const size_t z_app = p->reserved ? p->cap_tokens * sizeof(int32_t) : n_app;
  const size_t off_hdr = 0;  // reserved plans: float scale_log2, int32 num_merges
  const size_t off_wi = p->reserved ? kAlign : 0;
  const size_t off_items = off_wi + align_up(z_wi);
  const size_t off_merges = off_items + align_up(z_items);
  const size_t off_kvp = off_merges + align_up(z_merges);
  const size_t off_idx = off_kvp + align_up(z_kvp);
  const size_t off_app = off_idx + align_up(z_idx);
  // A small schedule is read by the kernels from the host slot; its merge
  // list then goes to the merge kernel as kernel arguments.
  const bool direct = !p->reserved &&
                      s.items.size() <= 2 * static_cast<size_t>(p->num_workers) &&
                      s.merges.size() <= static_cast<size_t>(mla::kInlineMerges) &&
                      s.worker_indptr[s.num_workers] == s.worker_indptr[s.num_workers + 1];
  // Each worker's first item, and its page list (up to kFirstPages pages),
  // at fixed places: the kernel reads them without a dependent read.
  const bool first_fast = direct && p->page_size % mla::kTileKeys == 0;
  const size_t n_first = first_fast ? s.num_workers * sizeof(mla::WorkItem) : 0;
  const size_t n_fpages =
      first_fast ? static_cast<size_t>(s.num_workers) * mla::kFirstPages * sizeof(int32_t) : 0;
  const size_t off_first = off_app + align_up(z_app);
  const size_t off_fpages = off_first + align_up(n_first);
  const size_t total = off_fpages + align_up(n_fpages);

  // This plan's host slot: the last copy from it and the last run that read
  // it must be done before it is refilled.
  hipError_t e;
  const int si = p->cur ^ 1;
  auto& sl = p->slot[si];
  if (sl.pending) {
    e = hipEventSynchronize(sl.done);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    sl.pending = false;
  }
  if (sl.wait_seq > 0) {
    const mla_status st = wait_flags(p, sl);
    if (st != MLA_OK) return st;
  }
  if (total > sl.cap) {
    if (sl.h_stage) (void)hipHostFree(sl.h_stage);
    sl.h_stage = nullptr;
    sl.cap = 0;
    e = hipHostMalloc(reinterpret_cast<void**>(&sl.h_stage), total, hipHostMallocDefault);
    if (e != hipSuccess) return hip_fail(e, "hipHostMalloc");
    sl.cap = total;
  }
  // Partials: bf16 output rows [slots, H, 512] then fp32 LSE [slots, H].
  const size_t part_floats =
      static_cast<size_t>(s.num_slots) * p->num_heads * (mla::kLoraRank / 2 + 1);
  if ((!direct && total > p->d_stage_cap) || part_floats > p->part_cap) {
    // Buffers may still be read by enqueued kernels of an earlier plan.
    e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
    if (!direct && total > p->d_stage_cap) {
      if (p->d_stage) (void)hipFree(p->d_stage);
      p->d_stage = nullptr;
      p->d_stage_cap = 0;
      e = hipMalloc(reinterpret_cast<void**>(&p->d_stage), total);
      if (e != hipSuccess) return hip_fail(e, "hipMalloc(schedule)");
      p->d_stage_cap = total;
    }
    if (part_floats > p->part_cap) {
      if (p->d_part) (void)hipFree(p->d_part);
      p->d_part = nullptr;
      p->part_cap = 0;
      e = hipMalloc(reinterpret_cast<void**>(&p->d_part), part_floats * sizeof(float));
      if (e != hipSuccess) return hip_fail(e, "hipMalloc(partials)");
      p->part_cap = part_floats;
    }
  }
  char* h = sl.h_stage;
  if (p->reserved) {
    const float sl2 = sm_scale * 1.44269504088896340736f;
    const int32_t nm = static_cast<int32_t>(s.merges.size());
    std::memcpy(h + off_hdr, &sl2, sizeof(float));
    std::memcpy(h + off_hdr + sizeof(float), &nm, sizeof(int32_t));
  }
  std::memcpy(h + off_wi, s.worker_indptr.data(), n_wi);
  if (n_items) std::memcpy(h + off_items, s.items.data(), n_items);
  if (n_merges) std::memcpy(h + off_merges, s.merges.data(), n_merges);
  if (s.batch > 0) std::memcpy(h + off_kvp, kv_indptr, n_kvp);
  if (n_idx) std::memcpy(h + off_idx, kv_indices, n_idx);
  if (n_app) std::memcpy(h + off_app, s.append_rows.data(), n_app);
  if (first_fast) {
    auto* fi = reinterpret_cast<mla::WorkItem*>(h + off_first);
    auto* fp = reinterpret_cast<int32_t*>(h + off_fpages);
    for (int w = 0; w < s.num_workers; ++w) {
      int32_t* pages = fp + static_cast<size_t>(w) * mla::kFirstPages;
      const int32_t wb = s.worker_indptr[w], we = s.worker_indptr[w + 1];
      if (wb == we) {
        fi[w] = mla::WorkItem{0, wb, 0, 0, -1, 0, {we, 0}};
        std::memset(pages, 0, mla::kFirstPages * sizeof(int32_t));
        continue;
      }
      mla::WorkItem it = s.items[wb];
      // The worker's item range rides in the fields the kernel does not read
      // (row, pad[0]).  The item's pages; entries past its last page repeat
      // it (the kernel never reads them).  pad[1] = 1: the list is staged.
      it.row = wb;
      it.pad[0] = we;
      const int32_t first_page = it.kv_end > it.kv_begin ? it.kv_begin / p->page_size : 0;
      const int32_t n_pages =
          it.kv_end > it.kv_begin ? (it.kv_end - 1) / p->page_size - first_page + 1 : 0;
      it.pad[1] = n_pages > 0 && n_pages <= mla::kFirstPages ? 1 : 0;
      const int32_t* src = kv_indices + it.page_base + first_page;
      for (int i = 0; i < mla::kFirstPages; ++i)
        pages[i] = it.pad[1] ? src[i < n_pages ? i : n_pages - 1] : 0;
      fi[w] = it;
    }
  }
  std::memset(h + off_idx + n_idx, 0, n_idx_pad - n_idx);
  if (!direct) {
    // (Stream order keeps the copy behind the runs that read the device
    // buffer before.)
    e = hipMemcpyAsync(p->d_stage, h, total, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
    e = hipEventRecord(sl.done, stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    sl.pending = true;
  }
  p->cur = si;
  p->direct = direct;

  p->off_wi = off_wi;
  p->off_items = off_items;
  p->off_merges = off_merges;
  p->off_kv_indptr = off_kvp;
  p->off_kv_indices = off_idx;
  p->off_append = off_app;
  p->off_first = off_first;
  p->off_fpages = off_fpages;
  p->first_fast = first_fast;
  p->append_checked = 0;
  p->scale_log2 = sm_scale * 1.44269504088896340736f;
  p->sched = std::move(s);
  p->planned = true;
  auto& k = p->key;
  k.batch = batch;
  k.causal = causal != 0;
  k.sm_scale = sm_scale;
  k.num_cache_pages = num_cache_pages;
  if (batch > 0) {
    k.qo.assign(qo_indptr, qo_indptr + batch + 1);
    k.kvp.assign(kv_indptr, kv_indptr + batch + 1);
    k.last.assign(kv_last_page_len, kv_last_page_len + batch);
    k.idx.assign(kv_indices, kv_indices + kv_indptr[batch]);
  } else {
    k.qo.clear();
    k.kvp.clear();
    k.last.clear();
    k.idx.clear();
  }
  return MLA_OK;
}

}  // extern "C"

namespace {

// mla_run / mla_run_fp8: kv_cache8 set selects the fp8 cache, whose scale
// multiplies the softmax scale and the normalised output.
mla_status run_impl(mla_plan_t p, const void* q_nope, const void* q_pe, const void* kv_cache,
                    const void* kv_cache8, float kv_scale, void* out, float* lse,
                    mla_stream_t stream_) {
  mla::clear_last_error();
  if (!p) return fail(MLA_E_INVALID, "NULL plan");
  if (!p->planned) return fail(MLA_E_STATE, "mla_run before a successful mla_plan");
  const auto& s = p->sched;
  if (s.num_tokens == 0) return MLA_OK;
  if (!q_nope || !q_pe || !out) return fail(MLA_E_INVALID, "NULL q_nope, q_pe or out");
  if (!kv_cache && !kv_cache8 && s.nnz > 0) return fail(MLA_E_INVALID, "NULL kv_cache");
  DeviceGuard g(p->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
  hipStream_t stream = static_cast<hipStream_t>(stream_);

  // (a reserved plan keeps the LSE section at the reserved offset)
  const size_t slots_h =
      static_cast<size_t>(p->reserved ? p->cap_items : s.num_slots) * p->num_heads;
  mla::AttnArgs a{};
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.kv_cache = static_cast<const uint16_t*>(kv_cache);
  a.kv_cache8 = static_cast<const uint8_t*>(kv_cache8);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.part_o = reinterpret_cast<uint16_t*>(p->d_part);
  a.part_lse = p->d_part ? p->d_part + slots_h * (mla::kLoraRank / 2) : nullptr;
  auto& sl = p->slot[p->cur];
  const char* d = p->direct ? sl.h_stage : p->d_stage;
  a.worker_indptr = reinterpret_cast<const int32_t*>(d + p->off_wi);
  a.pool_ctr = p->d_pool;
  if (p->reserved) a.scale_log2_ptr = reinterpret_cast<const float*>(d);
  a.items = reinterpret_cast<const mla::WorkItem*>(d + p->off_items);
  a.kv_indptr = reinterpret_cast<const int32_t*>(d + p->off_kv_indptr);
  a.kv_indices = reinterpret_cast<const int32_t*>(d + p->off_kv_indices);
  a.num_heads = p->num_heads;
  a.page_size = p->page_size;
  a.scale_log2 = p->scale_log2;
  a.out_scale = kv_cache8 ? kv_scale : 1.f;
  a.compact = p->num_heads <= 32 && p->num_workers == 2 * p->cus;
  // A schedule read from the host slot: the attention workgroups report when
  // they are done with it (no event between the kernels; runs of one plan
  // are stream-ordered, so a slot's flags only grow), and the merge list
  // reaches the merge kernel through device memory.
  bool capturing = false;
  if (p->direct) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t ce = hipStreamIsCapturing(stream, &cap);
    if (ce != hipSuccess) return hip_fail(ce, "hipStreamIsCapturing");
    capturing = cap != hipStreamCaptureStatusNone;
    // A captured run is never waited on, and stores no flag either: its
    // replays would store its (older) sequence number after later eager
    // runs had stored theirs, and a wait for those would never end.
    if (!capturing) {
      a.done_flags = sl.flags;
      a.run_seq = ++p->run_seq;
    }
    if (p->first_fast) {
      a.first_items = reinterpret_cast<const mla::WorkItem*>(d + p->off_first);
      a.first_pages = reinterpret_cast<const int32_t*>(d + p->off_fpages);
    }
  }
  hipError_t e = mla::launch_attention(a, s.num_workers, stream);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  // (Under stream capture a replay reads the slot whenever it runs: the
  // caller must not re-plan twice while such a graph may still replay.)
  if (p->direct && !capturing) sl.wait_seq = a.run_seq;
  if (!s.merges.empty() || p->reserved) {
    mla::SplitMergeArgs m{};
    m.part_o = a.part_o;
    m.part_lse = a.part_lse;
    if (p->direct)  // (at most kInlineMerges entries, by the choice of direct)
      std::memcpy(m.inline_merges, s.merges.data(), s.merges.size() * sizeof(mla::MergeItem));
    else
      m.merges = reinterpret_cast<const mla::MergeItem*>(d + p->off_merges);
    m.out = a.out;
    m.lse = lse;
    m.num_heads = p->num_heads;
    m.num_merges = static_cast<int32_t>(s.merges.size());
    for (const mla::MergeItem& mi : s.merges) m.max_pieces = std::max(m.max_pieces, mi.num_slots);
    if (p->reserved) {  // (captured kernels cover the reserved count)
      m.num_merges = static_cast<int32_t>(p->cap_merges);
      m.num_merges_ptr = reinterpret_cast<const int32_t*>(d + sizeof(float));
    }
    e = mla::launch_split_merge(m, stream);
    if (e != hipSuccess) return hip_fail(e, "split-merge launch");
  }
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_run(mla_plan_t p, const void* q_nope, const void* q_pe, const void* kv_cache,
                   void* out, float* lse, mla_stream_t stream) {
  return run_impl(p, q_nope, q_pe, kv_cache, nullptr, 1.f, out, lse, stream);
}

mla_status mla_run_fp8(mla_plan_t p, const void* q_nope, const void* q_pe,
                       const void* kv_cache_fp8, float kv_scale, void* out, float* lse,
                       mla_stream_t stream) {
  if (!(std::isfinite(kv_scale) && kv_scale > 0.f)) {
    mla::clear_last_error();
    return fail(MLA_E_INVALID, "kv_scale must be finite and positive");
  }
  return run_impl(p, q_nope, q_pe, nullptr, kv_cache_fp8, kv_scale, out, lse, stream);
}

}  // extern "C"

namespace {

mla_status append_impl(mla_plan_t p, const void* ckv, const void* kpe, void* kv_cache, bool fp8,
                       float kv_scale, mla_stream_t stream_) {
  mla::clear_last_error();
  if (!p) return fail(MLA_E_INVALID, "NULL plan");
  if (!p->planned) return fail(MLA_E_STATE, "mla_append_kv before a successful mla_plan");
  const auto& s = p->sched;
  if (p->append_checked == 0) p->append_checked = mla::check_append(s) == MLA_OK ? 1 : -1;
  if (p->append_checked < 0) {
    (void)mla::check_append(s);  // (sets the message again)
    return MLA_E_INVALID;
  }
  if (s.num_tokens == 0) return MLA_OK;
  if (!ckv || !kpe || !kv_cache) return fail(MLA_E_INVALID, "NULL ckv, kpe or kv_cache");
  DeviceGuard g(p->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  auto& sl = p->slot[p->cur];
  const char* d = p->direct ? sl.h_stage : p->d_stage;
  // A schedule staged in the host slot hands its few rows over as kernel
  // arguments (nothing reads the slot); otherwise the kernel reads them from
  // the device copy.
  const bool inline_rows = p->direct && s.num_tokens <= mla::kInlineRows;
  mla::AppendRows rows{};
  if (inline_rows)
    std::memcpy(rows.inline_rows, s.append_rows.data(), s.append_rows.size() * sizeof(int32_t));
  else
    rows.rows = reinterpret_cast<const int32_t*>(d + p->off_append);
  hipError_t e =
      fp8 ? mla::launch_append_kv_fp8(static_cast<const uint16_t*>(ckv),
                                      static_cast<const uint16_t*>(kpe), rows,
                                      static_cast<uint8_t*>(kv_cache), kv_scale, s.num_tokens,
                                      stream)
          : mla::launch_append_kv(static_cast<const uint16_t*>(ckv),
                                  static_cast<const uint16_t*>(kpe), rows,
                                  static_cast<uint16_t*>(kv_cache), s.num_tokens, stream);
  if (e != hipSuccess) return hip_fail(e, "append launch");
  if (p->direct && !inline_rows) {
    // The kernel reads the host slot (as mla_run does).
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    if (cap == hipStreamCaptureStatusNone) {
      e = hipEventRecord(sl.done, stream);
      if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
      sl.pending = true;
    }
  }
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_append_kv(mla_plan_t p, const void* ckv, const void* kpe, void* kv_cache,
                         mla_stream_t stream) {
  return append_impl(p, ckv, kpe, kv_cache, false, 1.f, stream);
}

mla_status mla_append_kv_fp8(mla_plan_t p, const void* ckv, const void* kpe, void* kv_cache_fp8,
                             float kv_scale, mla_stream_t stream) {
  if (!(std::isfinite(kv_scale) && kv_scale > 0.f)) {
    mla::clear_last_error();
    return fail(MLA_E_INVALID, "kv_scale must be finite and positive");
  }
  return append_impl(p, ckv, kpe, kv_cache_fp8, true, kv_scale, stream);
}

static mla_status projection(hipError_t (*launch)(const uint16_t*, const uint16_t*, uint16_t*,
                                                   int64_t, int, hipStream_t),
                             const char* what, const void* x, const void* w, void* out,
                             int64_t num_tokens, int32_t num_heads, mla_stream_t stream) {
  mla::clear_last_error();
  if (num_tokens < 0 || num_heads < 1 || num_heads > 65535)
    return fail(MLA_E_INVALID, "bad num_tokens / num_heads");
  if (num_tokens == 0) return MLA_OK;
  if (!x || !w || !out) return fail(MLA_E_INVALID, "NULL pointer");
  const hipError_t e = launch(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w),
                              static_cast<uint16_t*>(out), num_tokens, num_heads,
                              static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, what);
  return MLA_OK;
}

mla_status mla_absorb_query(const void* q_nope, const void* w_uk, void* q_abs, int64_t num_tokens,
                            int32_t num_heads, mla_stream_t stream) {
  return projection(mla::launch_absorb_query, "absorb launch", q_nope, w_uk, q_abs, num_tokens,
                    num_heads, stream);
}

mla_status mla_up_project(const void* o, const void* w_uv, void* v, int64_t num_tokens,
                          int32_t num_heads, mla_stream_t stream) {
  return projection(mla::launch_up_project, "up-projection launch", o, w_uv, v, num_tokens,
                    num_heads, stream);
}

mla_status mla_merge_state(const void* v_a, const float* s_a, const void* v_b, const float* s_b,
                           void* v_out, float* s_out, int64_t num_tokens, int32_t num_heads,
                           mla_stream_t stream) {
  mla::clear_last_error();
  if (num_tokens < 0 || num_heads < 1) return fail(MLA_E_INVALID, "bad num_tokens / num_heads");
  if (num_tokens == 0) return MLA_OK;
  if (!v_a || !s_a || !v_b || !s_b || !v_out || !s_out)
    return fail(MLA_E_INVALID, "NULL pointer");
  hipError_t e = mla::launch_merge_state(
      static_cast<const uint16_t*>(v_a), s_a, static_cast<const uint16_t*>(v_b), s_b,
      static_cast<uint16_t*>(v_out), s_out, num_tokens, num_heads,
      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge_state launch");
  return MLA_OK;
}

void mla_plan_destroy(mla_plan_t p) {
  if (!p) return;
  DeviceGuard g(p->device);
  release(p);
}

mla_status mla_plan_stats(mla_plan_t p, int32_t* num_workers, int64_t* num_items,
                          int64_t* num_split_tokens, int64_t* num_partials) {
  mla::clear_last_error();
  if (!p) return fail(MLA_E_INVALID, "NULL plan");
  if (!p->planned) return fail(MLA_E_STATE, "plan has not been planned");
  if (num_workers) *num_workers = p->sched.num_workers;
  if (num_items) *num_items = static_cast<int64_t>(p->sched.items.size());
  if (num_split_tokens) *num_split_tokens = static_cast<int64_t>(p->sched.merges.size());
  if (num_partials) *num_partials = p->sched.num_slots;
  return MLA_OK;
}

}  // extern "C"
