// KV append for gfx950: writes this step's latent rows into the paged cache
// (bf16, or an fp8 cache of E4M3 codes with one dequantisation scale)
// before attention runs over it (page "mstar.engine.resources.attn.base",
// AttentionManager.requires_kv_write: a layer writes the step's K/V through
// the KV resource, then calls run).  The host planner gives every query
// token its cache row (page * page_size + slot of key L - Q + i of its row);
// this kernel is a bandwidth-bound scatter of 1152-byte rows.
#include "kernels.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;

// One wave per token: lanes 0..63 copy the 1024-byte ckv part in 16-byte
// pieces, lanes 0..7 the 128-byte kpe part, to the token's cache row.
__global__ __launch_bounds__(256) void append_kv_kernel(const uint16_t* ckv, const uint16_t* kpe,
                                                        AppendRows rows, uint16_t* cache,
                                                        int64_t num_tokens) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= num_tokens) return;
  const int lane = threadIdx.x & 63;
  const int32_t r = rows.rows ? rows.rows[t] : rows.inline_rows[t];
  uint16_t* dst = cache + static_cast<int64_t>(r) * kLatentDim;
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ckv + t * kLoraRank + lane * 8);
  u32x4_t w{};
  if (lane < kRopeDim / 8) w = *reinterpret_cast<const u32x4_t*>(kpe + t * kRopeDim + lane * 8);
  *reinterpret_cast<u32x4_t*>(dst + lane * 8) = v;
  if (lane < kRopeDim / 8) *reinterpret_cast<u32x4_t*>(dst + kLoraRank + lane * 8) = w;
}

// fp8 cache: one wave per token; lane l quantises 8 ckv values (lanes 0..7
// also 8 kpe values) to E4M3 codes of fp32(x / kv_scale), nearest with ties
// to even (the conversion's rounding), saturated at +-448 by clamping the
// quotient first, and stores them as 8 bytes.
__device__ __forceinline__ uint32_t quant4(const uint16_t* x, float scale) {
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float f = __builtin_bit_cast(float, static_cast<uint32_t>(x[i]) << 16);
    v[i] = fminf(fmaxf(f / scale, -448.f), 448.f);
  }
  const uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0u, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], lo, true);
}

__global__ __launch_bounds__(256) void append_kv_fp8_kernel(const uint16_t* ckv, const uint16_t* kpe,
                                                            AppendRows rows, uint8_t* cache,
                                                            float kv_scale, int64_t num_tokens) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= num_tokens) return;
  const int lane = threadIdx.x & 63;
  const int32_t r = rows.rows ? rows.rows[t] : rows.inline_rows[t];
  uint8_t* dst = cache + static_cast<int64_t>(r) * kLatentDim;
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ckv + t * kLoraRank + lane * 8);
  const uint16_t* xv = reinterpret_cast<const uint16_t*>(&v);
  const u32x2_t q = {quant4(xv, kv_scale), quant4(xv + 4, kv_scale)};
  *reinterpret_cast<u32x2_t*>(dst + lane * 8) = q;
  if (lane < kRopeDim / 8) {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(kpe + t * kRopeDim + lane * 8);
    const uint16_t* xw = reinterpret_cast<const uint16_t*>(&w);
    const u32x2_t qw = {quant4(xw, kv_scale), quant4(xw + 4, kv_scale)};
    *reinterpret_cast<u32x2_t*>(dst + kLoraRank + lane * 8) = qw;
  }
}

}  // namespace

hipError_t launch_append_kv_fp8(const uint16_t* ckv, const uint16_t* kpe, const AppendRows& rows,
                                uint8_t* cache, float kv_scale, int64_t num_tokens,
                                hipStream_t stream) {
  if (!rows.rows && num_tokens > kInlineRows) return hipErrorInvalidValue;
  if (num_tokens <= 0) return hipSuccess;
  const int64_t blocks = (num_tokens + 3) / 4;
  hipLaunchKernelGGL(append_kv_fp8_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, ckv, kpe, rows, cache, kv_scale, num_tokens);
  return hipGetLastError();
}

hipError_t launch_append_kv(const uint16_t* ckv, const uint16_t* kpe, const AppendRows& rows,
                            uint16_t* cache, int64_t num_tokens, hipStream_t stream) {
  if (!rows.rows && num_tokens > kInlineRows) return hipErrorInvalidValue;
  if (num_tokens <= 0) return hipSuccess;
  const int64_t blocks = (num_tokens + 3) / 4;
  hipLaunchKernelGGL(append_kv_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     ckv, kpe, rows, cache, num_tokens);
  return hipGetLastError();
}

}  // namespace mla
