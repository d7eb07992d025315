// Kernel launch interfaces shared by the C ABI (capi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "planner.h"

namespace mla {

struct AttnArgs {
  const uint16_t* q_nope;    // bf16 [T, H, 512]
  const uint16_t* q_pe;      // bf16 [T, H, 64]
  const uint16_t* kv_cache;  // bf16 [pages, page_size, 576]
  uint16_t* out;             // bf16 [T, H, 512]
  float* lse;                // fp32 [T, H] or nullptr
  uint16_t* part_o;          // bf16 [slots, H, 512], normalised output of each piece
  float* part_lse;           // fp32 [slots, H], natural-log LSE of the piece
  const int32_t* worker_indptr;
  const WorkItem* items;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  int32_t num_heads;
  int32_t page_size;
  float scale_log2;  // sm_scale * log2(e)
};

struct SplitMergeArgs {
  const uint16_t* part_o;
  const float* part_lse;
  const MergeItem* merges;
  uint16_t* out;
  float* lse;
  int32_t num_heads;
  int32_t num_merges;
};

// Attention over every planned work item: one workgroup per worker.
hipError_t launch_attention(const AttnArgs& a, int num_workers, hipStream_t stream);

// Combines the partial results of tokens whose keys were split.
hipError_t launch_split_merge(const SplitMergeArgs& a, hipStream_t stream);

// KV append: latent row of token t ([ckv[t] | kpe[t]]) to cache row rows[t].
hipError_t launch_append_kv(const uint16_t* ckv, const uint16_t* kpe, const int32_t* rows,
                            uint16_t* cache, int64_t num_tokens, hipStream_t stream);

// Two-segment LSE merge (mla_merge_state).
hipError_t launch_merge_state(const uint16_t* v_a, const float* s_a, const uint16_t* v_b,
                              const float* s_b, uint16_t* v_out, float* s_out,
                              int64_t num_tokens, int32_t num_heads, hipStream_t stream);

}  // namespace mla
