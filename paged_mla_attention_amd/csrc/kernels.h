// Kernel launch interfaces shared by the C ABI (capi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "planner.h"

namespace mla {

struct AttnArgs {
  const uint16_t* q_nope;    // bf16 [T, H, 512]
  const uint16_t* q_pe;      // bf16 [T, H, 64]
  const uint16_t* kv_cache;  // bf16 [pages, page_size, 576] (bf16 cache)
  const uint8_t* kv_cache8;  // fp8 e4m3 codes [pages, page_size, 576] (fp8 cache)
  uint16_t* out;             // bf16 [T, H, 512]
  float* lse;                // fp32 [T, H] or nullptr
  uint16_t* part_o;          // bf16 [slots, H, 512], normalised output of each piece
  float* part_lse;           // fp32 [slots, H], natural-log LSE of the piece
  // [workgroups + 2]: workgroup w's own items, then the shared pool's range
  // (worker_indptr[workgroups] .. worker_indptr[workgroups + 1]).
  const int32_t* worker_indptr;
  const WorkItem* items;
  // Device counters of the shared pool, zero between runs: [0] the next pool
  // item to hand out, [1] workgroups done with the pool (the last one resets
  // both).  Used only when the pool is not empty.
  int32_t* pool_ctr;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  int32_t num_heads;
  int32_t page_size;
  float scale_log2;  // sm_scale * log2(e)
  // 1 for a bf16 cache; kv_scale for an fp8 cache, whose codes the kernel
  // reads unscaled: it multiplies the scores (with scale_log2) and the
  // normalised output.
  float out_scale;
  // At most 32 heads: nonzero selects the compact kernels that run two
  // workgroups per compute unit (one wave each; with an fp8 cache, or at
  // most 16 heads, a computing and a producing wave each); the schedule
  // must then have been made for two workers per compute unit.
  int32_t compact;
  const float* scale_log2_ptr;  // non-null: read the scale here (reserved plans)
  // Schedule read from a pinned host slot: each workgroup stores run_seq to
  // done_flags[workgroup] once it has read the slot for the last time (the
  // host waits on these before refilling it).  first_items[w] is worker w's
  // first item with its item range in the fields the kernel does not read
  // ({token, w_begin, kv_begin, kv_end, slot, page_base, w_end, staged}), so
  // that one 32-byte read starts the workgroup; when staged is set, the
  // item's page list is first_pages[w * kFirstPages ...], copied to LDS at
  // kernel entry.  Such a schedule has no shared pool.
  int32_t* done_flags;
  int32_t run_seq;
  const WorkItem* first_items;
  const int32_t* first_pages;
};


// The append kernel's destination rows: a device/host array, or, for a few
// tokens, the values themselves (kernel arguments need no memory read
// ahead of the copy and leave the staging slot unread).
constexpr int kInlineRows = 512;
struct AppendRows {
  const int32_t* rows;  // nullptr: use inline_rows
  int32_t inline_rows[kInlineRows];
};

// Pages of a worker's first item staged per worker in the host slot.
constexpr int kFirstPages = 16;
// Merge entries handed to the merge kernel as kernel arguments (schedules
// read from the host slot).
constexpr int kInlineMerges = 192;

struct SplitMergeArgs {
  const uint16_t* part_o;
  const float* part_lse;
  const MergeItem* merges;  // nullptr: inline_merges
  MergeItem inline_merges[kInlineMerges];
  uint16_t* out;
  float* lse;
  int32_t num_heads;
  int32_t num_merges;             // entries (the grid covers this many)
  const int32_t* num_merges_ptr;  // non-null: the live count, <= num_merges (reserved plans)
  int32_t max_pieces;             // most pieces of one token, 0 if not known on the host
};

// Attention over every planned work item: one workgroup per worker.  An
// fp8 cache (a.kv_cache8 set) is read as E4M3 codes whose values the
// arguments' scale factors carry.
hipError_t launch_attention(const AttnArgs& a, int num_workers, hipStream_t stream);

// Combines the partial results of tokens whose keys were split.
hipError_t launch_split_merge(const SplitMergeArgs& a, hipStream_t stream);

// KV append: latent row of token t ([ckv[t] | kpe[t]]) to cache row rows[t].
hipError_t launch_append_kv(const uint16_t* ckv, const uint16_t* kpe, const AppendRows& rows,
                            uint16_t* cache, int64_t num_tokens, hipStream_t stream);
// The same into an fp8 cache: each value stored as the E4M3 code nearest to
// fp32(x / kv_scale) (ties to even, saturated at +-448).
hipError_t launch_append_kv_fp8(const uint16_t* ckv, const uint16_t* kpe, const AppendRows& rows,
                                uint8_t* cache, float kv_scale, int64_t num_tokens,
                                hipStream_t stream);

// Per-head projections: out[t, h, :] = x[t, h, :] @ w[h] (bf16, fp32
// accumulation).  Absorption: [T, H, 128] x [H, 128, 512]; up-projection:
// [T, H, 512] x [H, 512, 128].
constexpr int kNopeDim = 128;
constexpr int kValueDim = 128;
hipError_t launch_absorb_query(const uint16_t* q, const uint16_t* w_uk, uint16_t* q_abs, int64_t T,
                               int H, hipStream_t stream);
hipError_t launch_up_project(const uint16_t* o, const uint16_t* w_uv, uint16_t* v, int64_t T,
                             int H, hipStream_t stream);

// Two-segment LSE merge (mla_merge_state).
hipError_t launch_merge_state(const uint16_t* v_a, const float* s_a, const uint16_t* v_b,
                              const float* s_b, uint16_t* v_out, float* s_out,
                              int64_t num_tokens, int32_t num_heads, hipStream_t stream);

}  // namespace mla
