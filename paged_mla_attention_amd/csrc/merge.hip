// LSE merges for gfx950.
//
// Both kernels combine attention results over disjoint key segments through
// their natural-log LSEs, which is what the m-star page
// "mstar.engine.resources.attn.flashinfer_mla" returns the LSE for
// (FlashInferMLAManager.run):
//   M = max_k s_k,  w_k = exp(s_k - M),  v = sum w_k v_k / sum w_k,
//   s = M + ln sum w_k,  and (0, -inf) when every segment is empty.
// Both are bandwidth-bound elementwise passes over [tokens, heads, 512].
#include "kernels.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;

__device__ __forceinline__ uint16_t to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ float bf16_lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) {
  return __builtin_bit_cast(float, w & 0xFFFF0000u);
}

// Split-KV partials -> final bf16 output + LSE.  A piece k holds its
// normalised output o_k (bf16) and its LSE s_k.  One wave per (merge item,
// head): lane l owns columns 8l .. 8l+7.  The first batch of partial rows is
// loaded together with the pieces' LSEs (lane k holds s_k), so a token split
// in at most kBatch pieces costs one memory round trip; the weights come
// from the LSE lanes by readlane.  Batches of 4 rows keep the kernel at 8
// waves per SIMD, so a decode batch's (token, head) waves (64 x 128) are all
// resident at once: the latency-bound kernel then costs one round trip of
// its waves, where batches of 8 needed two.  A merge of few (token, head)
// pairs with many pieces each (a long-context decode: 16 x 16 pairs of 32
// pieces) has registers to spare and takes them in larger batches.
template <int kBatch>
__global__ __launch_bounds__(256) void split_merge_kernel(SplitMergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int H = a.num_heads;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int num_merges = a.num_merges_ptr ? *a.num_merges_ptr : a.num_merges;
  if (pair >= num_merges * H) return;
  const int mi = pair / H, h = pair - mi * H;
  const MergeItem m = a.merges ? a.merges[mi] : a.inline_merges[mi];
  const int n = m.num_slots;
  const int64_t base = static_cast<int64_t>(m.first_slot) * H + h;  // slot k: base + k H
  const uint16_t* rows = a.part_o + base * kLoraRank + lane * 8;
  const int64_t row_step = static_cast<int64_t>(H) * kLoraRank;
  // Issued together: the first batch of rows and the LSEs of pieces 0..63.
  u32x4_t r[kBatch];
#pragma unroll
  for (int b = 0; b < kBatch; ++b) {
    const int k = b < n ? b : n - 1;  // (a repeated row gets weight 0)
    r[b] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(rows + k * row_step));
  }
  const float s_lane = lane < n ? a.part_lse[base + static_cast<int64_t>(lane) * H] : -INFINITY;
  float M = s_lane;
  for (int k = lane + 64; k < n; k += 64) M = fmaxf(M, a.part_lse[base + static_cast<int64_t>(k) * H]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (M != -INFINITY) {
    for (int k0 = 0; k0 < n; k0 += kBatch) {
      float s[kBatch];
      if (k0 > 0) {
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          const int k = k0 + b < n ? k0 + b : n - 1;
          r[b] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(rows + k * row_step));
        }
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int k = k0 + b;
        s[b] = k < 64 ? __shfl(s_lane, k < n ? k : 0)
                      : a.part_lse[base + static_cast<int64_t>(k < n ? k : n - 1) * H];
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const float w = (k0 + b >= n || s[b] == -INFINITY) ? 0.f : expf(s[b] - M);
        wsum += w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] += w * bf16_lo(r[b][j]);
          acc[2 * j + 1] += w * bf16_hi(r[b][j]);
        }
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int64_t th = static_cast<int64_t>(m.token) * H + h;
  u32x4_t o;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = to_bf16(acc[2 * j] * inv) | (static_cast<unsigned>(to_bf16(acc[2 * j + 1] * inv)) << 16);
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(a.out + th * kLoraRank + lane * 8));
  if (a.lse && lane == 0) a.lse[th] = wsum > 0.f ? M + logf(wsum) : -INFINITY;
}

// The same merge for few (token, head) pairs with many pieces each (a
// long-context decode: 16 x 16 pairs of 32 pieces), where one wave per pair
// leaves most compute units idle and each busy one with more rows in flight
// than it can keep moving: one workgroup per pair, wave w taking pieces w,
// w + 4, ... (kBatch rows per batch); every wave finds the pair's largest
// LSE from all the pieces' LSEs, so the four partial sums share one scale,
// and wave 0 adds them up through LDS.
template <int kBatch>
__global__ __launch_bounds__(256) void split_merge_wg_kernel(SplitMergeArgs a) {
  __shared__ float part[3][64 * 8 + 64];  // waves 1..3: 8 sums per lane, then the weight sums
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = a.num_heads;
  const int pair = blockIdx.x;
  const int num_merges = a.num_merges_ptr ? *a.num_merges_ptr : a.num_merges;
  if (pair >= num_merges * H) return;  // (uniform over the workgroup)
  const int mi = pair / H, h = pair - mi * H;
  const MergeItem m = a.merges ? a.merges[mi] : a.inline_merges[mi];
  const int n = m.num_slots;
  const int64_t base = static_cast<int64_t>(m.first_slot) * H + h;  // slot k: base + k H
  const uint16_t* rows = a.part_o + base * kLoraRank + lane * 8;
  const int64_t row_step = static_cast<int64_t>(H) * kLoraRank;
  // Issued together: this wave's first batch of rows and the LSEs of pieces 0..63.
  u32x4_t r[kBatch];
#pragma unroll
  for (int b = 0; b < kBatch; ++b) {
    const int k = wave + 4 * b;
    r[b] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4_t*>(rows + (k < n ? k : n - 1) * row_step));
  }
  const float s_lane = lane < n ? a.part_lse[base + static_cast<int64_t>(lane) * H] : -INFINITY;
  float M = s_lane;
  for (int k = lane + 64; k < n; k += 64) M = fmaxf(M, a.part_lse[base + static_cast<int64_t>(k) * H]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (M != -INFINITY) {
    for (int k0 = wave; k0 < n; k0 += 4 * kBatch) {
      if (k0 > wave) {
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          const int k = k0 + 4 * b;
          r[b] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4_t*>(rows + (k < n ? k : n - 1) * row_step));
        }
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int k = k0 + 4 * b;
        const float s = k < 64 ? __shfl(s_lane, k < n ? k : 0)
                               : a.part_lse[base + static_cast<int64_t>(k < n ? k : n - 1) * H];
        const float w = (k >= n || s == -INFINITY) ? 0.f : expf(s - M);
        wsum += w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] += w * bf16_lo(r[b][j]);
          acc[2 * j + 1] += w * bf16_hi(r[b][j]);
        }
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) part[wave - 1][j * 64 + lane] = acc[j];
    part[wave - 1][512 + lane] = wsum;
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += part[w][j * 64 + lane];
    wsum += part[w][512 + lane];
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int64_t th = static_cast<int64_t>(m.token) * H + h;
  u32x4_t o;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = to_bf16(acc[2 * j] * inv) | (static_cast<unsigned>(to_bf16(acc[2 * j + 1] * inv)) << 16);
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(a.out + th * kLoraRank + lane * 8));
  if (a.lse && lane == 0) a.lse[th] = wsum > 0.f ? M + logf(wsum) : -INFINITY;
}

__global__ __launch_bounds__(256) void merge_state_kernel(const uint16_t* v_a,
                                                          const float* s_a,
                                                          const uint16_t* v_b,
                                                          const float* s_b, uint16_t* v_out,
                                                          float* s_out, int64_t pairs) {
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (pair >= pairs) return;
  const int lane = threadIdx.x & 63;
  const float sa = s_a[pair], sb = s_b[pair];
  const float M = fmaxf(sa, sb);
  const int64_t off = pair * kLoraRank + lane * 8;
  // (streamed once: non-temporal loads and store keep them from displacing
  // other data in the caches)
  const u32x4_t va = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(v_a + off));
  const u32x4_t vb = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(v_b + off));
  float wa = 0.f, wb = 0.f;
  if (M != -INFINITY) {
    wa = (sa == -INFINITY) ? 0.f : expf(sa - M);
    wb = (sb == -INFINITY) ? 0.f : expf(sb - M);
  }
  const float z = wa + wb;
  const float inv = z > 0.f ? 1.f / z : 0.f;
  const float ca = wa * inv, cb = wb * inv;
  u32x4_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = ca * bf16_lo(va[j]) + cb * bf16_lo(vb[j]);
    const float hi = ca * bf16_hi(va[j]) + cb * bf16_hi(vb[j]);
    r[j] = to_bf16(lo) | (static_cast<unsigned>(to_bf16(hi)) << 16);
  }
  __builtin_nontemporal_store(r, reinterpret_cast<u32x4_t*>(v_out + off));
  if (lane == 0) s_out[pair] = z > 0.f ? M + logf(z) : -INFINITY;
}

}  // namespace

hipError_t launch_split_merge(const SplitMergeArgs& a, hipStream_t stream) {
  if (a.num_merges <= 0) return hipSuccess;
  const int64_t pairs = static_cast<int64_t>(a.num_merges) * a.num_heads;
  const dim3 grid(static_cast<unsigned>((pairs + 3) / 4));
  // (up to 4096 pairs, 16 waves per compute unit: residency does not limit
  // the round trips there)
  const bool few = pairs <= 4096;
  // (at most 1024 pairs of more than 8 pieces: a workgroup per pair)
  if (pairs <= 1024 && a.max_pieces > 8) {
    const dim3 wg_grid(static_cast<unsigned>(pairs));
    if (a.max_pieces > 16)
      hipLaunchKernelGGL(split_merge_wg_kernel<8>, wg_grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(split_merge_wg_kernel<4>, wg_grid, dim3(256), 0, stream, a);
  } else if (few && a.max_pieces > 16)
    hipLaunchKernelGGL(split_merge_kernel<32>, grid, dim3(256), 0, stream, a);
  else if (few && a.max_pieces > 4)
    hipLaunchKernelGGL(split_merge_kernel<16>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(split_merge_kernel<4>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_merge_state(const uint16_t* v_a, const float* s_a, const uint16_t* v_b,
                              const float* s_b, uint16_t* v_out, float* s_out,
                              int64_t num_tokens, int32_t num_heads, hipStream_t stream) {
  const int64_t pairs = num_tokens * num_heads;
  if (pairs <= 0) return hipSuccess;
  const int64_t blocks = (pairs + 3) / 4;
  hipLaunchKernelGGL(merge_state_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, v_a, s_a, v_b, s_b, v_out, s_out, pairs);
  return hipGetLastError();
}

}  // namespace mla
