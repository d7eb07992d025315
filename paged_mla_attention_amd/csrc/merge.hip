// LSE merges for gfx950.
//
// Both kernels combine attention results over disjoint key segments through
// their natural-log LSEs, the use the m-star page
// "mstar.engine.resources.attn.flashinfer_mla" gives for the returned LSE
// (FlashInferMLAManager.run: "for merging with another key segment"):
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
// normalised output o_k (bf16) and its LSE s_k.  One block of 128 threads
// per (merge entry, head); each thread owns 4 consecutive latent columns.
__global__ __launch_bounds__(128) void split_merge_kernel(SplitMergeArgs a) {
  const int h = blockIdx.x;
  const MergeItem m = a.merges[blockIdx.y];
  const int H = a.num_heads;
  const int c = threadIdx.x * 4;
  float M = -INFINITY;
  for (int k = 0; k < m.num_slots; ++k)
    M = fmaxf(M, a.part_lse[static_cast<int64_t>(m.first_slot + k) * H + h]);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (M != -INFINITY) {
    for (int k = 0; k < m.num_slots; ++k) {
      const int64_t sh = static_cast<int64_t>(m.first_slot + k) * H + h;
      const float s = a.part_lse[sh];
      const float w = (s == -INFINITY) ? 0.f : expf(s - M);
      const u32x2_t r = *reinterpret_cast<const u32x2_t*>(a.part_o + sh * kLoraRank + c);
      const f32x4_t v = {bf16_lo(r[0]), bf16_hi(r[0]), bf16_lo(r[1]), bf16_hi(r[1])};
      acc += w * v;
      wsum += w;
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int64_t th = static_cast<int64_t>(m.token) * H + h;
  u32x2_t o;
  o[0] = to_bf16(acc[0] * inv) | (static_cast<unsigned>(to_bf16(acc[1] * inv)) << 16);
  o[1] = to_bf16(acc[2] * inv) | (static_cast<unsigned>(to_bf16(acc[3] * inv)) << 16);
  *reinterpret_cast<u32x2_t*>(a.out + th * kLoraRank + c) = o;
  if (a.lse && threadIdx.x == 0) a.lse[th] = wsum > 0.f ? M + logf(wsum) : -INFINITY;
}

// Two-segment merge.  One wave per (token, head): lane i owns columns
// 8i .. 8i+7 (16 bytes of each bf16 input).  All lanes read s_a / s_b in the
// same instruction before any lane writes s_out, so s_out may alias s_a.
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
  const u32x4_t va = *reinterpret_cast<const u32x4_t*>(v_a + off);
  const u32x4_t vb = *reinterpret_cast<const u32x4_t*>(v_b + off);
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
  *reinterpret_cast<u32x4_t*>(v_out + off) = r;
  if (lane == 0) s_out[pair] = z > 0.f ? M + logf(z) : -INFINITY;
}

}  // namespace

hipError_t launch_split_merge(const SplitMergeArgs& a, hipStream_t stream) {
  if (a.num_merges <= 0) return hipSuccess;
  hipLaunchKernelGGL(split_merge_kernel, dim3(a.num_heads, a.num_merges), dim3(128), 0, stream,
                     a);
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
