/*
 * mla.h - paged Multi-head Latent Attention (MLA) for AMD Instinct MI355X
 * (gfx950).  C ABI: plain pointers and sizes, no framework types.
 *
 * What is computed (m-star documentation, page
 * "mstar.engine.resources.attn.flashinfer_mla": module description and
 * FlashInferMLAWrapper.plan / run):
 *
 *   The cache holds one latent row per token, [ckv (512) | kpe (64)] bf16.
 *   For query token t of row b, head h, and each key j the row may see,
 *     s_j = sm_scale * (q_nope[t,h,:] . ckv_j + q_pe[t,h,:] . kpe_j)
 *     out[t,h,:] = sum_j softmax(s)_j * ckv_j          (latent space, 512 wide)
 *     lse[t,h]   = ln sum_j exp(s_j)                   (natural log, fp32)
 *   q_nope is the absorbed query (q_nope @ W_UK, kv_lora_rank wide) and q_pe
 *   the un-rotated rope part; the kernel applies no rotation and no W_UV.
 *
 *   Rows are ragged through a CSR page table (FlashInferMLAWrapper.plan):
 *     qo_indptr[B+1]        query tokens of row b: [qo_indptr[b], qo_indptr[b+1])
 *     kv_indptr[B+1]        pages of row b: kv_indices[kv_indptr[b] .. kv_indptr[b+1])
 *     kv_indices[nnz]       page ids into the cache, in key order
 *     kv_last_page_len[B]   valid slots of the row's last page, 1..page_size
 *   so row b holds L_b = (n_b - 1) * page_size + kv_last_page_len[b] keys
 *   (0 when it names no page).  Key j of the row is slot j % page_size of
 *   page kv_indices[kv_indptr[b] + j / page_size].
 *
 *   Causal (the plan default): a row's query block is aligned to the end of
 *   its keys (page "mstar.engine.resources.attn.ragged.wrappers",
 *   PrefixedPrefillWrapper): query i of Q sees keys j <= i + L - Q.  A query
 *   that sees no key gets out = 0 and lse = -inf.  Non-causal: every query
 *   sees all L keys.
 *
 *   sm_scale is the softmax scale of the original head dim, e.g. 192^-0.5
 *   (FlashInferMLAWrapper parameters).
 *
 * Tensor layouts (all row-major, contiguous, device memory):
 *   q_nope   bf16 [T, H, 512]     q_pe bf16 [T, H, 64]
 *   kv_cache bf16 [num_cache_pages, page_size, 576]  (ckv first, then kpe)
 *   out      bf16 [T, H, 512]     lse  fp32 [T, H]
 * with T = qo_indptr[B] and H = num_heads.
 *
 * Supported shapes: kv_lora_rank 512 and qk_rope_head_dim 64 exactly (the
 * DeepSeek/Kimi latent shape the flashinfer_mla_supports page names); other
 * ranks return MLA_E_UNSUPPORTED, there is no fallback path.  1 <= num_heads
 * <= 128, page_size >= 1.
 *
 * Errors: every entry point returns a status; nothing aborts or throws across
 * the ABI.  mla_last_error() returns a thread-local text for the last failing
 * call on the calling thread.
 *
 * Threading: a plan handle must not be used by two threads at once.
 * Independent handles never interact.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_E_INVALID = 1,     /* bad argument or page table (message says which) */
  MLA_E_UNSUPPORTED = 2, /* shape the kernels do not implement */
  MLA_E_STATE = 3,       /* call order violated, e.g. mla_run before mla_plan */
  MLA_E_HIP = 4,         /* a HIP runtime call failed (message has the HIP error) */
  MLA_E_NOMEM = 5        /* device or pinned host allocation failed */
} mla_status;

/* An opaque plan.  The library owns its pinned staging buffer, its device
 * copy of the schedule and page table, and its split-KV partial workspace. */
typedef struct mla_plan_s* mla_plan_t;

/* A HIP stream (hipStream_t); NULL is the null stream. */
typedef void* mla_stream_t;

/* Create a plan on HIP device `device` for `num_heads` query heads (1..128),
 * latent shape (kv_lora_rank, qk_rope_head_dim) which must be (512, 64), and
 * cache pages of `page_size` tokens.  Constructor arguments follow
 * FlashInferMLAWrapper(num_qo_heads, kv_lora_rank, qk_rope_head_dim,
 * page_size).  The number of workers is the device's compute-unit count.
 * On success *out owns the plan; release it with mla_plan_destroy. */
mla_status mla_plan_create(mla_plan_t* out, int32_t device, int32_t num_heads,
                           int32_t kv_lora_rank, int32_t qk_rope_head_dim,
                           int32_t page_size);

/* Plan one batch (FlashInferMLAWrapper.plan): validate the CSR page table,
 * split each query token's visible keys into chunks balanced over the
 * compute units, and copy the schedule and page table to the device.
 *
 * All four index arrays are HOST int32 memory (the page notes that the KV plan
 * builds them on the host); they are read before the call returns and not
 * kept.  kv_indices must hold at least kv_indptr[batch] entries.  Page ids
 * must lie in [0, num_cache_pages).
 *
 * The schedule is staged in one of two pinned host slots, alternating
 * between plans.  A small schedule (at most two work items per compute
 * unit, as in decode) is read by the kernels straight from that slot; a
 * larger one is copied asynchronously on `stream` to the plan's device
 * buffer.  Before refilling a slot, mla_plan waits for the last copy from it
 * and the last mla_run that read it, so planning step N+1 never races step
 * N.  The first plan, and any plan that outgrows the buffers, synchronises
 * the device while it (re)allocates; later plans of equal or smaller size
 * allocate nothing.  mla_run must be called on `stream` (or a stream
 * ordered after it).
 *
 * A call whose inputs (all four arrays, batch, causal, sm_scale and
 * num_cache_pages) equal those of the plan's last successful call returns at
 * once and keeps that schedule (page "mstar.engine.resources.attn.base",
 * PlanCacheKey: an unchanged plan need not be rebuilt).
 *
 * Errors: MLA_E_INVALID for a malformed table (indptr[0] != 0, decreasing
 * indptr, last_page_len outside [1, page_size] on a row with pages, page id
 * out of range, batch < 0, non-finite or non-positive sm_scale);
 * MLA_E_UNSUPPORTED when num_cache_pages * page_size exceeds 2^31 rows (the
 * kernels address cache rows in 32 bits).  The plan keeps its previous state
 * on error. */
mla_status mla_plan(mla_plan_t plan, const int32_t* qo_indptr, const int32_t* kv_indptr,
                    const int32_t* kv_indices, const int32_t* kv_last_page_len,
                    int32_t batch, int32_t causal, float sm_scale,
                    int64_t num_cache_pages, mla_stream_t stream);

/* Reserve fixed capacity (page "mstar.engine.resources.attn.base":
 * captured_page_capacity and static buffers, so a captured graph stays valid
 * while the batch changes): later plans of at most max_batch rows,
 * max_tokens query tokens and max_kv_indices page ids are laid out at fixed
 * places of the plan's device buffer, copied there on the plan's stream, and
 * every value the kernels need (scale, merge count) is read from that
 * buffer.  An mla_run captured once then runs whatever batch was planned
 * last (q, out and lse must be sized for max_tokens; rows beyond the batch's
 * tokens are untouched; capture after a plan with at least one token).  A
 * plan beyond the capacity fails with MLA_E_INVALID and keeps the previous
 * one.  Synchronises the device and allocates; call it before capturing.
 * After it the plan must be planned again. */
mla_status mla_plan_reserve(mla_plan_t plan, int32_t max_batch, int64_t max_tokens,
                            int64_t max_kv_indices);

/* Run the planned batch (FlashInferMLAWrapper.run): all pointers are device
 * memory with the layouts above; `lse` may be NULL when not wanted.  The call
 * only enqueues kernels on `stream` (no allocation, no synchronisation), so
 * it may be captured in a HIP graph.  A schedule read straight from its host
 * slot is released by the kernels themselves (each workgroup stores the
 * run's sequence number to pinned memory when it is done with the slot; a
 * later mla_plan waits on those); all runs of one plan must therefore be
 * ordered on one stream (they also share the plan's split-KV workspace and
 * the device counters from which the workgroups draw a batch's shared pool
 * of whole-token items, which each run leaves at zero).  The plan must not
 * be re-planned while a captured graph that reads it may still replay.
 *
 * Errors: MLA_E_STATE without a successful mla_plan; MLA_E_INVALID for a NULL
 * required pointer; MLA_E_HIP if a launch fails. */
mla_status mla_run(mla_plan_t plan, const void* q_nope, const void* q_pe,
                   const void* kv_cache, void* out, float* lse, mla_stream_t stream);

/* mla_run over an fp8 latent cache (FlashInferMLAWrapper.plan takes a
 * kv_dtype; the pages name no fp8 format, and this library reads one as):
 * kv_cache_fp8 is [num_cache_pages, page_size, 576] bytes of OCP FP8 E4M3
 * codes (sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals,
 * largest finite 448, no infinities), ckv then kpe, and a cached value is
 * decode(code) * kv_scale for the one fp32 scale of the whole cache.  The
 * result is the attention of mla_run over those values: q, out and lse keep
 * the layouts and dtypes of mla_run.  The codes are converted exactly to
 * bf16 on the GPU and kv_scale is applied in fp32 to the scores and the
 * normalised output.  The same plan serves bf16 and fp8 runs.
 *
 * Errors: those of mla_run, and MLA_E_INVALID for a kv_scale that is not
 * finite and positive. */
mla_status mla_run_fp8(mla_plan_t plan, const void* q_nope, const void* q_pe,
                       const void* kv_cache_fp8, float kv_scale, void* out, float* lse,
                       mla_stream_t stream);

/* Write this step's latent rows into the cache before attention reads it
 * (page "mstar.engine.resources.attn.base", AttentionManager.requires_kv_write:
 * a layer writes the step's K/V through the KV resource, then calls run).
 * Uses the planned page table: the Q query tokens of row b are the row's
 * last Q keys, so token t = qo_indptr[b] + i becomes key j = L_b - Q_b + i
 * and its row [ckv[t,:] | kpe[t,:]] is stored at slot j % page_size of page
 * kv_indices[kv_indptr[b] + j / page_size] (the same end alignment as the
 * causal query block).  Other slots are untouched.
 *   ckv bf16 [T, 512], kpe bf16 [T, 64]: device memory, read;
 *   kv_cache bf16 [num_cache_pages, page_size, 576]: device memory, written
 *   in place (ckv into columns 0..511, kpe into 512..575).
 * Enqueued on `stream` (one kernel; no allocation or synchronisation); call
 * it before mla_run on the same stream.  Like mla_run it reads the plan's
 * schedule, so the same re-planning fence applies.
 *
 * Errors: MLA_E_STATE without a successful mla_plan; MLA_E_INVALID for a NULL
 * pointer (with T > 0), a row with more query tokens than keys, or two tokens
 * that would land in the same cache slot (rows sharing pages); MLA_E_HIP if
 * the launch fails. */
mla_status mla_append_kv(mla_plan_t plan, const void* ckv, const void* kpe, void* kv_cache,
                         mla_stream_t stream);

/* mla_append_kv into an fp8 cache (the layout of mla_run_fp8): each bf16
 * value x becomes the E4M3 code nearest to the fp32 quotient x / kv_scale,
 * ties to the even mantissa, magnitudes beyond 448 saturated to 448, the
 * sign of zero kept.  Same slots, fences and errors as mla_append_kv, plus
 * MLA_E_INVALID for a kv_scale that is not finite and positive. */
mla_status mla_append_kv_fp8(mla_plan_t plan, const void* ckv, const void* kpe,
                             void* kv_cache_fp8, float kv_scale, mla_stream_t stream);

/* The projections either side of the kernel (module description of the
 * flashinfer_mla page: the query entering the kernel is absorbed,
 * q_nope @ W_UK, and the latent output is brought back to the value heads by
 * W_UV), per head h, in bf16 with fp32 accumulation:
 *   mla_absorb_query: q_abs[t,h,:] = q_nope[t,h,:] @ w_uk[h]
 *     q_nope bf16 [T, H, 128], w_uk bf16 [H, 128, 512] (row k of head h holds
 *     the 512 latent weights of nope dim k), q_abs bf16 [T, H, 512];
 *   mla_up_project: v[t,h,:] = o[t,h,:] @ w_uv[h]
 *     o bf16 [T, H, 512] (what mla_run writes), w_uv bf16 [H, 512, 128],
 *     v bf16 [T, H, 128].
 * (128 = the nope and value head dims; the pages state only the 192-wide
 * softmax scale, 192 = 128 + 64.)  Device memory, row-major; the output may
 * not alias the inputs.  Enqueued on `stream`, no allocation or
 * synchronisation.  MLA_E_INVALID for NULL pointers (with T > 0),
 * num_tokens < 0 or num_heads outside [1, 65535]. */
mla_status mla_absorb_query(const void* q_nope, const void* w_uk, void* q_abs, int64_t num_tokens,
                            int32_t num_heads, mla_stream_t stream);
mla_status mla_up_project(const void* o, const void* w_uv, void* v, int64_t num_tokens,
                          int32_t num_heads, mla_stream_t stream);

/* Merge two attention results over disjoint key segments of the same
 * queries through their LSEs (FlashInferMLAManager.run: the LSE is returned
 * for merging with another key segment):
 *   M = max(s_a, s_b);  w_x = exp(s_x - M)
 *   v_out = (w_a v_a + w_b v_b) / (w_a + w_b),  s_out = M + ln(w_a + w_b)
 * and (0, -inf) where both sides are empty (-inf).
 * v_* are bf16 [num_tokens, num_heads, 512], s_* fp32 [num_tokens, num_heads],
 * device memory; arithmetic in fp32.  v_out / s_out may alias v_a / s_a (or
 * v_b / s_b) exactly; partial overlap is not allowed.  Enqueued on `stream`,
 * no allocation or synchronisation. */
mla_status mla_merge_state(const void* v_a, const float* s_a, const void* v_b,
                           const float* s_b, void* v_out, float* s_out,
                           int64_t num_tokens, int32_t num_heads, mla_stream_t stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): mla_plan + mla_run in one
 * call that allocates nothing and reads the page table from DEVICE memory.
 *
 * qo_indptr [batch+1], kv_indptr [batch+1], kv_indices [num_kv_indices] and
 * kv_last_page_len [batch] are device int32 arrays with the layout and rules
 * of mla_plan; num_tokens must equal qo_indptr[batch] and max_kv_len must
 * bound the keys of every row (both host values the caller knows from its
 * tensor shapes and sequence limits).  q_nope, q_pe, kv_cache, out and lse
 * are as for mla_run; `lse` may be NULL.  Runs on the current HIP device.
 *
 * Three kernels are enqueued on `stream` (a planner that validates the page
 * table and splits the work on the device, the attention kernel and the
 * split-KV merge); there is no allocation, no host synchronisation and no
 * memset, so the call may be captured in a HIP graph.  The schedule, its
 * temporaries and the split-KV partials live in one fixed device array of
 * about 81 MiB per GPU, allocated with the library's code object on each GPU
 * it runs on and held until the process ends.  Every call on a GPU shares
 * that array and leaves its contents behind: calls that overlap on one GPU
 * (other streams, other threads) race and must be ordered by the caller.
 *
 * Limits: batch <= 8192 rows, num_tokens <= 8192, and a worst case for rows of
 * max_kv_len keys within the workspace: num_tokens * (1 + c) + 256 work items
 * <= 16384 and 512 + num_tokens * (c ? c + 1 : 0) split partials <=
 * 80 MiB / (num_heads * 1028 B), where c = (ceil(max_kv_len / 32) - 1) / 1024
 * for max_kv_len > 32768 keys, else 0 (at 128 heads: 637 partials).  Calls
 * beyond them fail with MLA_E_INVALID and a message naming the limit.  A
 * page table that breaks the rules of mla_plan (checked on the device,
 * including max_kv_len) yields zero output and -inf LSE for every token.
 *
 * Errors: MLA_E_INVALID for sizes beyond the limits, NULL pointers or a bad
 * scalar; MLA_E_UNSUPPORTED for num_heads outside [1, 128] or
 * num_cache_pages * page_size above 2^31 rows; MLA_E_HIP when the symbol
 * lookup or a launch fails. */
mla_status mla_run_noalloc(const int32_t* qo_indptr, const int32_t* kv_indptr,
                           const int32_t* kv_indices, const int32_t* kv_last_page_len,
                           int32_t batch, int64_t num_tokens, int64_t num_kv_indices,
                           int32_t causal, float sm_scale, int64_t num_cache_pages,
                           int32_t max_kv_len, int32_t num_heads, int32_t page_size,
                           const void* q_nope, const void* q_pe, const void* kv_cache,
                           void* out, float* lse, mla_stream_t stream);

/* Release a plan and everything it owns.  Waits for the plan's pending
 * copy; the caller must make sure no enqueued mla_run on it is still
 * executing.  NULL is ignored. */
void mla_plan_destroy(mla_plan_t plan);

/* Planner introspection for a plan that has been planned: the number of
 * workers (workgroups) the attention kernel launches, work items, query
 * tokens whose keys were split over several items, and partial slots.
 * Any output pointer may be NULL. */
mla_status mla_plan_stats(mla_plan_t plan, int32_t* num_workers, int64_t* num_items,
                          int64_t* num_split_tokens, int64_t* num_partials);

/* Static text for a status code. */
const char* mla_status_str(mla_status status);

/* Detail of the last failing call on this thread ("" if none). */
const char* mla_last_error(void);

/* ------------------------------------------------------------------------
 * Host-only schedule (no device needed).  The same planner mla_plan runs,
 * exposed so its output can be inspected and replayed on the CPU.
 *
 * Work item (8 int32 each): {token, row, kv_begin, kv_end, slot, 0, 0, 0}:
 *   query token `token` of row `row` attends the row's keys
 *   [kv_begin, kv_end); slot = -1 writes the final result, slot >= 0 writes
 *   a partial result (normalised output and LSE) into partial slot `slot`.
 * Merge entry (4 int32 each): {token, first_slot, num_slots, 0}: the token's
 *   result is the LSE merge of partial slots [first_slot, first_slot+num_slots).
 * worker_indptr[num_workers+2]: worker w (workgroup w of the attention
 *   launch) runs items [worker_indptr[w], worker_indptr[w+1]) in order;
 *   items [worker_indptr[num_workers], worker_indptr[num_workers+1]) are a
 *   shared pool of whole-token items (slot -1) that the workgroups take one
 *   at a time, in order, once their own items are done (empty unless the
 *   batch has many query tokens).
 * ------------------------------------------------------------------------ */
typedef struct mla_schedule_s* mla_schedule_t;

mla_status mla_schedule_build(mla_schedule_t* out, const int32_t* qo_indptr,
                              const int32_t* kv_indptr, const int32_t* kv_indices,
                              const int32_t* kv_last_page_len, int32_t batch,
                              int32_t causal, int32_t page_size, int64_t num_cache_pages,
                              int32_t num_heads, int32_t num_workers);

/* Sizes of a built schedule; any pointer may be NULL. */
void mla_schedule_sizes(mla_schedule_t s, int32_t* num_workers, int64_t* num_items,
                        int64_t* num_merges, int64_t* num_slots);

/* Copy the schedule out: worker_indptr [num_workers+2], items [num_items*8],
 * merges [num_merges*4] (host memory, sized from mla_schedule_sizes). */
void mla_schedule_copy(mla_schedule_t s, int32_t* worker_indptr, int32_t* items,
                       int32_t* merges);

/* The cache row (page * page_size + slot) mla_append_kv writes for each of
 * the schedule's T query tokens, into rows [T] (host memory; may be NULL to
 * only validate).  MLA_E_INVALID, with the reason, when the page table cannot
 * take an append (a row with more tokens than keys, or two tokens in one
 * slot). */
mla_status mla_schedule_append_rows(mla_schedule_t s, int32_t* rows);

void mla_schedule_destroy(mla_schedule_t s);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
