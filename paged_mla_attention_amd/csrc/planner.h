// Host planner for paged latent attention: validation of the CSR page table
// and the split of every query token's visible keys into work items balanced
// over the device's compute units.  Pure C++ (no HIP), so it also builds and
// runs on a machine without a GPU.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/mla.h"

namespace mla {

// Keys per attention tile.  Chunk boundaries inside a token's key range fall
// on multiples of this, so every work item starts on a tile boundary.
constexpr int kTileKeys = 32;
constexpr int kLoraRank = 512;
constexpr int kRopeDim = 64;
constexpr int kLatentDim = kLoraRank + kRopeDim;
constexpr int kMaxHeads = 128;
// Longest work item in tiles.  The attention kernel stages an item's page
// ids (at most one per tile when a tile never crosses a page) in a fixed LDS
// array of this many entries.
constexpr int kMaxItemTiles = 1024;

struct WorkItem {
  int32_t token;     // query token (row of q_nope / out)
  int32_t row;       // batch row (selects the page list)
  int32_t kv_begin;  // first key (multiple of kTileKeys)
  int32_t kv_end;    // one past the last key
  int32_t slot;      // -1: final output; >= 0: partial slot
  int32_t page_base; // kv_indptr[row]: the row's first entry in kv_indices
  int32_t pad[2];
};
static_assert(sizeof(WorkItem) == 32, "work item is 8 int32");

struct MergeItem {
  int32_t token;
  int32_t first_slot;
  int32_t num_slots;
  int32_t pad;
};
static_assert(sizeof(MergeItem) == 16, "merge item is 4 int32");

struct PlanArgs {
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* kv_last_page_len;
  int32_t batch;
  bool causal;
  int32_t page_size;
  int64_t num_cache_pages;
  int32_t num_heads;
  int32_t num_workers;
};

struct Schedule {
  int32_t num_workers = 0;
  int32_t batch = 0;
  int64_t num_tokens = 0;
  int64_t num_slots = 0;
  int64_t nnz = 0;                     // kv_indptr[batch]
  // [num_workers + 2], launch order: worker w's own items are
  // [worker_indptr[w], worker_indptr[w + 1]); items [worker_indptr[W],
  // worker_indptr[W + 1]) form the shared pool, taken one at a time by
  // whichever workgroup runs out of its own items first.
  std::vector<int32_t> worker_indptr;
  std::vector<WorkItem> items;
  std::vector<MergeItem> merges;
  // KV append: cache row (page * page_size + slot) of each query token's
  // latent (token i of a row with Q tokens and L keys is key L - Q + i), and,
  // if the page table cannot take an append, why.
  std::vector<int32_t> append_rows;
  std::string append_error;
};

// Checks that no two tokens of the schedule append into the same cache slot
// (rows shared between requests may name the same pages).  Returns
// MLA_E_INVALID, with the thread's last-error text set, on a collision or
// when the schedule's append_error is set.
mla_status check_append(const Schedule& s);

// Validates `a` and fills `out`.  On failure returns the status, sets the
// thread's last-error text and leaves `out` untouched.
mla_status build_schedule(const PlanArgs& a, Schedule* out);

// Thread-local error text used by every entry point.
void set_last_error(const std::string& msg);
void clear_last_error();

}  // namespace mla
