// Paged latent attention kernel for gfx950 (CDNA4), decode and prefill alike.
//
// Computes, for each planned work item (one query token, a range of its
// row's keys), the latent attention of the m-star page
// "mstar.engine.resources.attn.flashinfer_mla" (module description and
// FlashInferMLAWrapper.run): scores (q_nope . ckv + q_pe . kpe) * sm_scale
// over a [ckv | kpe] latent cache read through the CSR page table, softmax,
// and the 512-wide latent output softmax . ckv with its natural-log LSE.
//
// Work decomposition (this library's design, not the pages'):
//   * one workgroup per worker (one per compute unit); it runs the worker's
//     items in order.  An item is one query token with ALL its heads, so a
//     key tile staged in LDS is shared by every head of the token;
//   * wave w owns heads [32w, 32w + 32); a workgroup has ceil(H / 32) waves;
//   * keys are processed in tiles of 32, double-buffered in LDS: while the
//     waves compute on one stage, the next tile is fetched into registers
//     and then written to the other stage;
//   * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 with keys as M and heads as N,
//     so each lane ends up holding 16 scores of ONE head and the softmax
//     statistics are per lane (one cross-lane exchange per tile);
//   * O^T += V^T . P^T on the same MFMA with latent columns as M: the
//     probabilities come straight from the score accumulators (no shuffle),
//     and V^T is read from a transposed, swizzled copy of the tile's ckv
//     columns that the loader writes beside the row-major K tile;
//   * softmax in base 2 against a per-head reference maximum fixed at the
//     item's first tile: p = 2^(x - m_ref) is exact for any reference (output
//     and LSE are normalised with the same value), so the O accumulators are
//     never rescaled inside the key loop.  A later score more than 2^64 above
//     the reference (which would overflow) makes the workgroup redo the item
//     with the largest score seen as the reference;
//   * items covering a token's whole key range write bf16 output + LSE;
//     pieces of a split token write fp32 partials that a merge kernel combines.
#include "kernels.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kWave = 64;
constexpr int kQChunks = kLatentDim / 16;          // 36 k-steps of 16 over 576
constexpr int kKRowBytes = kLatentDim * 2 + 16;    // 1168 B: row pad spreads rows over banks
constexpr int kKBytes = kTileKeys * kKRowBytes;    // 37376
constexpr int kVtRowBytes = kTileKeys * 2;         // 64 B: one ckv column, 32 keys
constexpr int kVtBytes = kLoraRank * kVtRowBytes;  // 32768
constexpr int kStageBytes = kKBytes + kVtBytes;    // 70144
constexpr int kStages = 2;
constexpr int kFlagBytes = 16;                     // per-wave redo flags after the stages
constexpr int kLoadUnits = 256;                    // (column chunk, key octet) pairs per tile
constexpr float kMaxExponent = 64.0f;              // log2 headroom above the reference
constexpr float kLn2 = 0.693147180559945309f;

// The transposed-V row of column c holds 4 chunks of 8 keys; chunk q is
// stored at 16-byte slot q ^ vt_swizzle(c) so that the 8 (and 16) lanes that
// read one chunk of consecutive columns, and the lanes that write 8
// consecutive columns, fall into different LDS banks.
__device__ __forceinline__ int vt_swizzle(int c) { return ((c >> 1) + (c >> 3)) & 3; }

// Key of element i (0..7) of key octet (ks, half) inside a tile.  The P^T
// operand of the P.V product takes score register j = 8 ks + i of lane
// half `half`, which the 32x32 MFMA result layout places at key
// 8 (j / 4) + 4 half + j % 4.
__device__ __forceinline__ int octet_key(int ks, int half, int i) {
  return 16 * ks + 8 * (i >> 2) + 4 * half + (i & 3);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

struct TileRegs {
  u32x4_t ckv[8];  // 8 keys x 16 B of one ckv column chunk
  u32x4_t kpe;     // 16 B of one key's kpe
};

template <int NW>
struct Attn {
  static constexpr int NT = NW * kWave;
  static constexpr int kRounds = (kLoadUnits + NT - 1) / NT;

  const AttnArgs& a;
  char* smem;
  int tid, lane, l32, half, wave, head;
  bool head_ok;
  // current item
  int token, kv_end, slot;
  const int32_t* pages;  // the row's page ids

  __device__ Attn(const AttnArgs& args, char* s) : a(args), smem(s) {
    tid = threadIdx.x;
    lane = tid & 63;
    l32 = lane & 31;
    half = lane >> 5;
    wave = tid >> 6;
    head = wave * 32 + l32;
    head_ok = head < a.num_heads;
  }

  __device__ __forceinline__ const uint16_t* key_row(int key) const {
    const int P = a.page_size;
    const int page = pages[key / P];
    return a.kv_cache + (static_cast<int64_t>(page) * P + key % P) * kLatentDim;
  }

  // Global -> registers for load round r of the tile starting at key `base`.
  __device__ __forceinline__ void fetch(TileRegs& r, int base, int round) const {
    const int u = tid + round * NT;
    if (u >= kLoadUnits) return;
    const int cc = u & 63, oct = u >> 6;
    const int ks = oct >> 1, hf = oct & 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = base + octet_key(ks, hf, i);
      r.ckv[i] = key < kv_end
                     ? *reinterpret_cast<const u32x4_t*>(key_row(key) + cc * 8)
                     : u32x4_t{0u, 0u, 0u, 0u};
    }
    const int kk = u >> 3, ch = u & 7;
    const int key = base + kk;
    r.kpe = key < kv_end ? *reinterpret_cast<const u32x4_t*>(key_row(key) + kLoraRank + ch * 8)
                         : u32x4_t{0u, 0u, 0u, 0u};
  }

  // Registers -> LDS stage: row-major K rows and the transposed V columns.
  __device__ __forceinline__ void store(const TileRegs& r, char* stage, int round) const {
    const int u = tid + round * NT;
    if (u >= kLoadUnits) return;
    const int cc = u & 63, oct = u >> 6;
    const int ks = oct >> 1, hf = oct & 1;
    char* K = stage;
    char* VT = stage + kKBytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<u32x4_t*>(K + octet_key(ks, hf, i) * kKRowBytes + cc * 16) = r.ckv[i];
    }
    const int kk = u >> 3, ch = u & 7;
    *reinterpret_cast<u32x4_t*>(K + kk * kKRowBytes + kLoraRank * 2 + ch * 16) = r.kpe;
    // 8x8 transpose: column e of the 8 key chunks -> 8 keys of column 8cc+e.
    const int q = 2 * ks + hf;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u32x4_t w;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned lo = r.ckv[2 * j][e >> 1];
        const unsigned hi = r.ckv[2 * j + 1][e >> 1];
        w[j] = (e & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
      }
      const int c = cc * 8 + e;
      *reinterpret_cast<u32x4_t*>(VT + c * kVtRowBytes + ((q ^ vt_swizzle(c)) * 16)) = w;
    }
  }

  __device__ void run() {
    const int w_begin = a.worker_indptr[blockIdx.x];
    const int w_end = a.worker_indptr[blockIdx.x + 1];
    const int H = a.num_heads;

    for (int it = w_begin; it < w_end; ++it) {
      const WorkItem item = a.items[it];
      token = item.token;
      kv_end = item.kv_end;
      slot = item.slot;
      pages = a.kv_indices + a.kv_indptr[item.row];
      const int kv_begin = item.kv_begin;

      // Query of this lane's head: 36 chunks of 8 along the 576 latent dims,
      // element layout matching the K operand (dims 16 kk + 8 half + i).
      bf16x8_t q[kQChunks];
      {
        const uint16_t* qn = a.q_nope + (static_cast<int64_t>(token) * H + head) * kLoraRank;
        const uint16_t* qp = a.q_pe + (static_cast<int64_t>(token) * H + head) * kRopeDim;
#pragma unroll
        for (int kk = 0; kk < kQChunks; ++kk) {
          u32x4_t v = {0u, 0u, 0u, 0u};
          if (head_ok) {
            v = kk < kLoraRank / 16
                    ? *reinterpret_cast<const u32x4_t*>(qn + kk * 16 + half * 8)
                    : *reinterpret_cast<const u32x4_t*>(qp + (kk - kLoraRank / 16) * 16 + half * 8);
          }
          q[kk] = __builtin_bit_cast(bf16x8_t, v);
        }
      }

      f32x16_t o[kLoraRank / 32];
      float m_ref = -INFINITY;  // reference max of scaled base-2 scores (per head)
      float m_seen = -INFINITY; // largest score seen (per head)
      float l_run = 0.f;        // this lane's share of the softmax denominator
      const int ntiles = (kv_end - kv_begin + kTileKeys - 1) / kTileKeys;
      for (;;) {
#pragma unroll
        for (int mb = 0; mb < kLoraRank / 32; ++mb)
#pragma unroll
          for (int j = 0; j < 16; ++j) o[mb][j] = 0.f;
        l_run = 0.f;
        if (ntiles == 0) break;
        TileRegs regs;
        for (int r = 0; r < kRounds; ++r) {
          fetch(regs, kv_begin, r);
          store(regs, smem, r);
        }
        __syncthreads();
        for (int t = 0; t < ntiles; ++t) {
          const int base = kv_begin + t * kTileKeys;
          const bool more = t + 1 < ntiles;
          if (more) fetch(regs, base + kTileKeys, 0);
          char* stage = smem + (t & 1) * kStageBytes;
          compute_tile(stage, base, q, o, m_ref, m_seen, l_run);
          if (more) {
            char* next = smem + ((t + 1) & 1) * kStageBytes;
            store(regs, next, 0);
            for (int r = 1; r < kRounds; ++r) {
              fetch(regs, base + kTileKeys, r);
              store(regs, next, r);
            }
          }
          __syncthreads();
        }
        // Redo the item if any head of the workgroup overflowed its reference.
        int* flags = reinterpret_cast<int*>(smem + kStages * kStageBytes);
        const bool redo = __any(m_seen > m_ref + kMaxExponent);
        if (lane == 0) flags[wave] = redo ? 1 : 0;
        __syncthreads();
        int any_redo = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) any_redo |= flags[w];
        __syncthreads();
        if (!any_redo) break;
        m_ref = m_seen;
      }
      const float m_run = m_ref;
      finish(o, m_run, l_run);
    }
  }

  __device__ __forceinline__ void compute_tile(const char* stage, int base,
                                               const bf16x8_t (&q)[kQChunks],
                                               f32x16_t (&o)[kLoraRank / 32], float& m_ref,
                                               float& m_seen, float& l_run) const {
    const char* K = stage;
    const char* VT = stage + kKBytes;
    // S^T[key, head] over the 576 latent dims.
    f32x16_t s;
#pragma unroll
    for (int j = 0; j < 16; ++j) s[j] = 0.f;
    const char* krow = K + l32 * kKRowBytes + half * 16;
#pragma unroll
    for (int kk = 0; kk < kQChunks; ++kk) {
      const bf16x8_t kv = *reinterpret_cast<const bf16x8_t*>(krow + kk * 32);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, q[kk], s, 0, 0, 0);
    }
    // Scale to base 2, mask keys beyond the item's range, tile max.
    float x[16];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = base + 8 * (j >> 2) + 4 * half + (j & 3);
      x[j] = key < kv_end ? s[j] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, x[j]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    m_seen = fmaxf(m_seen, mx);
    if (m_ref == -INFINITY) m_ref = mx;  // first tile of the item: O is still zero
    // Probabilities relative to the reference, as the bf16 B operand.
    bf16x8_t p[2];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float e = __builtin_amdgcn_exp2f(fminf(x[j] - m_ref, kMaxExponent));
      l_run += e;
      p[j >> 3][j & 7] = static_cast<__bf16>(e);
    }
    // O^T[col, head] += V^T[col, key] . P^T[key, head].
#pragma unroll
    for (int mb = 0; mb < kLoraRank / 32; ++mb) {
      const int c = mb * 32 + l32;
      const char* vrow = VT + c * kVtRowBytes;
      const int sw = vt_swizzle(c);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(vrow + (((2 * ks + half) ^ sw) * 16));
        o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, p[ks], o[mb], 0, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void finish(f32x16_t (&o)[kLoraRank / 32], float m_run,
                                         float l_run) const {
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const bool any = l_tot > 0.f;
    const float inv = any ? 1.f / l_tot : 0.f;
    const float lse_v = any ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    if (!head_ok) return;
    const int H = a.num_heads;
    if (slot < 0) {
      uint16_t* dst = a.out + (static_cast<int64_t>(token) * H + head) * kLoraRank;
#pragma unroll
      for (int mb = 0; mb < kLoraRank / 32; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int c = mb * 32 + q4 * 8 + half * 4;
          u32x2_t w;
          w[0] = f32_to_bf16_bits(o[mb][4 * q4 + 0] * inv) |
                 (static_cast<unsigned>(f32_to_bf16_bits(o[mb][4 * q4 + 1] * inv)) << 16);
          w[1] = f32_to_bf16_bits(o[mb][4 * q4 + 2] * inv) |
                 (static_cast<unsigned>(f32_to_bf16_bits(o[mb][4 * q4 + 3] * inv)) << 16);
          *reinterpret_cast<u32x2_t*>(dst + c) = w;
        }
      if (a.lse && half == 0) a.lse[static_cast<int64_t>(token) * H + head] = lse_v;
    } else {
      float* dst = a.part_o + (static_cast<int64_t>(slot) * H + head) * kLoraRank;
#pragma unroll
      for (int mb = 0; mb < kLoraRank / 32; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int c = mb * 32 + q4 * 8 + half * 4;
          f32x4_t w;
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = o[mb][4 * q4 + i] * inv;
          *reinterpret_cast<f32x4_t*>(dst + c) = w;
        }
      if (half == 0) a.part_lse[static_cast<int64_t>(slot) * H + head] = lse_v;
    }
  }
};

template <int NW>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attention_kernel(AttnArgs args) {
  __shared__ __attribute__((aligned(16))) char smem[kStages * kStageBytes + kFlagBytes];
  Attn<NW> k(args, smem);
  k.run();
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int num_workers, hipStream_t stream) {
  if (num_workers <= 0) return hipSuccess;
  const int nw = (a.num_heads + 31) / 32;
  const dim3 grid(num_workers);
  switch (nw) {
    case 1: hipLaunchKernelGGL(attention_kernel<1>, grid, dim3(1 * kWave), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(attention_kernel<2>, grid, dim3(2 * kWave), 0, stream, a); break;
    case 3: hipLaunchKernelGGL(attention_kernel<3>, grid, dim3(3 * kWave), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(attention_kernel<4>, grid, dim3(4 * kWave), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
