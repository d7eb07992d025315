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
//   * keys are processed in tiles of 32.  A tile is copied from HBM straight
//     into LDS by global_load_lds (no staging registers), four tiles deep
//     (4 x 36 KiB of the 160 KiB LDS), with explicit vmcnt waits and a bare
//     s_barrier per tile;
//   * one swizzled LDS layout serves both products: 16-byte chunk (key, dc)
//     (dc = 8-column chunk of the 576 latent columns) sits at
//     (dc/2)*1024 + (dc%2)*512 + (key ^ 4*(dc%2))*16, which the loader
//     writes as 36 DMA instructions of 1 KiB and which keeps both read
//     patterns free of bank conflicts;
//   * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 with keys as M and heads as N
//     (K operand: ds_read_b128 of 32 keys x 16 B), so each lane ends up
//     holding 16 scores of ONE head and the softmax statistics are per lane
//     (one cross-lane exchange per tile);
//   * O^T += V^T . P^T on the same MFMA with latent columns as M: the
//     probabilities come straight from the score accumulators, and the V^T
//     operand is read from the same K tile with ds_read_b64_tr_b16, whose
//     16-lane transpose turns four 8-byte row pieces into one column each;
//   * softmax in base 2 against a per-head reference maximum fixed at the
//     item's first tile: p = 2^(x - m_ref) is exact for any reference (output
//     and LSE are normalised with the same value), so the O accumulators are
//     never rescaled inside the key loop.  A later score more than 2^64 above
//     the reference (which would overflow) makes the workgroup redo the item
//     with the largest score seen as the reference;
//   * page ids come through scalar loads, so no vector load inside the key
//     loop ever forces the in-order vmcnt to drain the DMA queue;
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
typedef short s16x4_t __attribute__((vector_size(8)));
typedef short s16x8_t __attribute__((vector_size(16)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(4))) const int32_t const_i32_t;

constexpr int kWave = 64;
constexpr int kQChunks = kLatentDim / 16;         // 36 k-steps of 16 over 576
constexpr int kDmaPerTile = kLatentDim / 16;      // 36 x 1 KiB (two 16-B chunks x 32 keys)
constexpr int kTileBytes = kDmaPerTile * 1024;    // 36864
constexpr int kStages = 4;
constexpr int kFlagBytes = 16;                    // per-wave redo flags after the stages
constexpr int kFinishRow = 128 + 4;               // floats per head row of the output staging
constexpr int kFinishWaveBytes = (32 * kFinishRow + 32) * 4;  // per-wave staging + 1/l per head
constexpr float kMaxExponent = 64.0f;             // log2 headroom above the reference
constexpr float kLn2 = 0.693147180559945309f;

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector
// memory operations are outstanding and leaves the other counters alone.
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Barrier without the memory fence of __syncthreads (which would wait for
// every outstanding LDS DMA); the empty asm keeps the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int NW>
struct Attn {
  static constexpr int kLoadsPerWave = (kDmaPerTile + NW - 1) / NW;
  static constexpr int kWaitOne = kLoadsPerWave > 63 ? 63 : kLoadsPerWave;
  static constexpr int kWaitTwo = 2 * kLoadsPerWave > 63 ? 63 : 2 * kLoadsPerWave;

  const AttnArgs& a;
  char* smem;
  int lane, l32, half, wave, head;
  bool head_ok;
  int ld_key, ld_off, qk_off, pv_off;  // per-lane LDS / row offsets
  uint32_t lds_base;                   // LDS address of the stages
  // current item
  int token, kv_end, slot;
  int page_base;  // index of the row's first page in kv_indices

  __device__ Attn(const AttnArgs& args, char* s) : a(args), smem(s) {
    const int tid = threadIdx.x;
    lane = tid & 63;
    l32 = lane & 31;
    half = lane >> 5;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    head = wave * 32 + l32;
    head_ok = head < a.num_heads;
    lds_base = static_cast<uint32_t>(reinterpret_cast<size_t>((__attribute__((address_space(3))) char*)smem));
    // loader: lane p fetches key (p%32) ^ 4(p/32), chunk parity p/32
    ld_key = l32 ^ (4 * half);
    ld_off = half * 16;
    // score operand: key l32, chunk 2kk + half
    qk_off = half * 512 + ((l32 ^ (4 * half)) * 16);
    // P.V operand through the 16-lane transpose read: group G = lane/16 is
    // (key half hf, 16-column group cg); source lane s of the group points at
    // key 4hf + s/4 (+8 for the second read), columns 16cg + 4(s%4) .. +3.
    const int G = lane >> 4, sl = lane & 15;
    const int hf = G >> 1, cg = G & 1;
    const int par = (sl >> 1) & 1;  // chunk parity of the source columns
    const int key_l = 4 * hf + (sl >> 2);
    pv_off = cg * 1024 + par * 512 + (sl & 1) * 8 + ((key_l ^ (4 * par)) * 16);
  }

  // Page id of key `key` of the current row, for the lane's own key.  The
  // page table is read with scalar loads only (wave-uniform addresses, made
  // explicit with readfirstlane so no select is folded into a per-lane
  // address): a vector load here would make the in-order vmcnt wait for every
  // DMA in flight.
  __device__ __forceinline__ int lane_page(int base, int key) const {
    const int P = a.page_size;
    const_i32_t* idx = (const_i32_t*)(a.kv_indices) + page_base;
    const int first = base / P;
    if (P % kTileKeys == 0)  // the whole tile is in one page
      return __builtin_amdgcn_readfirstlane(idx[first]);
    const int j = key / P - first;  // 0 .. 31
    int v = __builtin_amdgcn_readfirstlane(idx[first]);
#pragma unroll
    for (int i = 1; i < kTileKeys; ++i) {
      const int pi = __builtin_amdgcn_readfirstlane(idx[first + i]);
      v = (j == i) ? pi : v;
    }
    return v;
  }

  // One 16-byte-per-lane DMA from global memory into LDS at lds_addr + 16 *
  // lane.  Issued through asm so that the compiler, which cannot tell the
  // stages apart, does not make later LDS reads wait for every DMA; the
  // tile pipeline waits on vmcnt itself.  M0 holds the LDS base; one wait
  // state separates its write from the DMA.
  __device__ __forceinline__ static void dma16(const char* src, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds_addr)
                 : "memory", "m0");
  }

  // DMA the 32-key tile starting at key `base` into LDS stage `stage`.  Keys
  // beyond the item's range re-read its last key (finite data, masked later).
  __device__ __forceinline__ void issue_tile(int base, int stage) const {
    int key = base + ld_key;
    key = key < kv_end ? key : kv_end - 1;
    const int P = a.page_size;
    const int page = lane_page(base, key);
    const char* src = reinterpret_cast<const char*>(
        a.kv_cache + (static_cast<int64_t>(page) * P + key % P) * kLatentDim) + ld_off;
    const uint32_t dst = lds_base + stage * kTileBytes;
#pragma unroll
    for (int j = 0; j < kLoadsPerWave; ++j) {
      const int I = wave + j * NW;
      if (NW * kLoadsPerWave == kDmaPerTile || I < kDmaPerTile) dma16(src + I * 32, dst + I * 1024);
    }
  }

  // Wait until this wave's DMAs for the tile `later` tiles before the newest
  // have landed.
  __device__ __forceinline__ void wait_tile(int later) const {
    if (later >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kWaitTwo));
    else if (later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kWaitOne));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }

  __device__ void run() {
    const_i32_t* widx = (const_i32_t*)(a.worker_indptr);
    const int w_begin = widx[blockIdx.x];
    const int w_end = widx[blockIdx.x + 1];
    const int H = a.num_heads;

    for (int it = w_begin; it < w_end; ++it) {
      const_i32_t* item = (const_i32_t*)(a.items) + it * 8;  // WorkItem fields
      token = item[0];
      const int row = item[1];
      const int kv_begin = item[2];
      kv_end = item[3];
      slot = item[4];
      page_base = ((const_i32_t*)(a.kv_indptr))[row];

      // Query of this lane's head: 36 chunks of 8 along the 576 latent dims,
      // element layout matching the K operand (dims 16 kk + 8 half + i).
      bf16x8_t q[kQChunks];
      {
        // Lanes of padding heads read head 0's row and zero it.
        const int hq = head_ok ? head : 0;
        const uint16_t* qn = a.q_nope + (static_cast<int64_t>(token) * H + hq) * kLoraRank;
        const uint16_t* qp = a.q_pe + (static_cast<int64_t>(token) * H + hq) * kRopeDim;
        const unsigned keep = head_ok ? 0xFFFFFFFFu : 0u;
#pragma unroll
        for (int kk = 0; kk < kQChunks; ++kk) {
          u32x4_t v = kk < kLoraRank / 16
                          ? *reinterpret_cast<const u32x4_t*>(qn + kk * 16 + half * 8)
                          : *reinterpret_cast<const u32x4_t*>(qp + (kk - kLoraRank / 16) * 16 + half * 8);
          v &= keep;
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
        // Every wave is done with the previous item's output staging (LDS),
        // and this wave's query loads and earlier stores retire before the
        // DMA queue is counted tile by tile.
        __syncthreads();
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        asm volatile("" ::: "memory");
        for (int t = 0; t < kStages - 1 && t < ntiles; ++t)
          issue_tile(kv_begin + t * kTileKeys, t);
        for (int t = 0; t < ntiles; ++t) {
          const int issued_after = ntiles - 1 - t < kStages - 2 ? ntiles - 1 - t : kStages - 2;
          wait_tile(issued_after);
          lds_barrier();
          if (t + kStages - 1 < ntiles)
            issue_tile(kv_begin + (t + kStages - 1) * kTileKeys, (t + kStages - 1) % kStages);
          compute_tile(smem + (t % kStages) * kTileBytes, kv_begin + t * kTileKeys, q, o, m_ref,
                       m_seen, l_run);
        }
        // Redo the item if any head of the workgroup overflowed its reference.
        int* flags = reinterpret_cast<int*>(smem + kStages * kTileBytes);
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
      finish(o, m_ref, l_run);
    }
  }

  __device__ __forceinline__ void compute_tile(const char* K, int base,
                                               const bf16x8_t (&q)[kQChunks],
                                               f32x16_t (&o)[kLoraRank / 32], float& m_ref,
                                               float& m_seen, float& l_run) const {
    // S^T[key, head] over the 576 latent dims.
    f32x16_t s;
#pragma unroll
    for (int j = 0; j < 16; ++j) s[j] = 0.f;
    // Operands are read kAhead k-steps before their MFMA, so LDS latency
    // overlaps the MFMA pipeline.
    const char* kq = K + qk_off;
    constexpr int kAhead = 3;
    bf16x8_t kbuf[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) kbuf[i] = *reinterpret_cast<const bf16x8_t*>(kq + i * 1024);
#pragma unroll
    for (int kk = 0; kk < kQChunks; ++kk) {
      const bf16x8_t kv = kbuf[kk % kAhead];
      if (kk + kAhead < kQChunks)
        kbuf[kk % kAhead] = *reinterpret_cast<const bf16x8_t*>(kq + (kk + kAhead) * 1024);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, q[kk], s, 0, 0, 0);
    }
    // Keep the reads kAhead steps ahead: the scheduler would otherwise pull
    // each read down next to its MFMA.
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);  // DS reads
#pragma unroll
    for (int kk = 0; kk < kQChunks; ++kk) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      if (kk + kAhead < kQChunks) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one DS read
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
    const char* kv = K + pv_off;
    auto vload = [&](int step) {
      const char* ptr = kv + (step >> 1) * 2048 + (step & 1) * 256;
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(ptr));
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(ptr + 128));
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    constexpr int kSteps = 2 * (kLoraRank / 32);  // (column block, key half) pairs
    bf16x8_t vbuf[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) vbuf[i] = vload(i);
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const bf16x8_t v = vbuf[st % kAhead];
      if (st + kAhead < kSteps) vbuf[st % kAhead] = vload(st + kAhead);
      o[st >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, p[st & 1], o[st >> 1], 0, 0, 0);
    }
  }

  // Writes the item's result.  The accumulators are never touched by VALU
  // code here (that makes the compiler shuttle all 256 of them through
  // VGPRs): a partial piece stores the raw sums and 1/l for the merge kernel;
  // a final item stages the raw sums through this wave's LDS region, then
  // normalises, converts and stores 16 bytes per lane, 4 heads x 256 B
  // contiguous per instruction.  The caller has made the LDS stages free.
  __device__ __forceinline__ void finish(f32x16_t (&o)[kLoraRank / 32], float m_run,
                                         float l_run) const {
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const bool any = l_tot > 0.f;
    const float inv = any ? 1.f / l_tot : 0.f;
    const float lse_v = any ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    const int H = a.num_heads;
    if (slot >= 0) {
      if (head_ok) {
        float* dst = a.part_o + (static_cast<int64_t>(slot) * H + head) * kLoraRank;
#pragma unroll
        for (int mb = 0; mb < kLoraRank / 32; ++mb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4_t w = {o[mb][4 * q4], o[mb][4 * q4 + 1], o[mb][4 * q4 + 2],
                               o[mb][4 * q4 + 3]};
            *reinterpret_cast<f32x4_t*>(dst + mb * 32 + q4 * 8 + half * 4) = w;
          }
        if (half == 0) {
          const int64_t sh = static_cast<int64_t>(slot) * H + head;
          a.part_lse[sh] = lse_v;
          a.part_scale[sh] = inv;
        }
      }
      return;
    }
    float* R = reinterpret_cast<float*>(smem + wave * kFinishWaveBytes);
    float* inv_h = R + 32 * kFinishRow;
    if (half == 0) inv_h[l32] = inv;
    if (a.lse && head_ok && half == 0) a.lse[static_cast<int64_t>(token) * H + head] = lse_v;
#pragma unroll
    for (int round = 0; round < kLoraRank / 128; ++round) {
#pragma unroll
      for (int m4 = 0; m4 < 4; ++m4) {
        const int mb = round * 4 + m4;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4_t w = {o[mb][4 * q4], o[mb][4 * q4 + 1], o[mb][4 * q4 + 2],
                             o[mb][4 * q4 + 3]};
          *reinterpret_cast<f32x4_t*>(R + l32 * kFinishRow + m4 * 32 + q4 * 8 + half * 4) = w;
        }
      }
      // lane: head h = (lane + 64 r) / 16 of the wave, 8 columns cc * 8 of
      // this round's 128.
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int qi = lane + 64 * r;
        const int h = qi >> 4, cc = qi & 15;
        const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(R + h * kFinishRow + cc * 8);
        const f32x4_t v1 = *reinterpret_cast<const f32x4_t*>(R + h * kFinishRow + cc * 8 + 4);
        const float sc = inv_h[h];
        u32x4_t w;
        w[0] = f32_to_bf16_bits(v0[0] * sc) | (static_cast<unsigned>(f32_to_bf16_bits(v0[1] * sc)) << 16);
        w[1] = f32_to_bf16_bits(v0[2] * sc) | (static_cast<unsigned>(f32_to_bf16_bits(v0[3] * sc)) << 16);
        w[2] = f32_to_bf16_bits(v1[0] * sc) | (static_cast<unsigned>(f32_to_bf16_bits(v1[1] * sc)) << 16);
        w[3] = f32_to_bf16_bits(v1[2] * sc) | (static_cast<unsigned>(f32_to_bf16_bits(v1[3] * sc)) << 16);
        const int hg = wave * 32 + h;
        if (hg < H)
          *reinterpret_cast<u32x4_t*>(a.out + (static_cast<int64_t>(token) * H + hg) * kLoraRank +
                                      round * 128 + cc * 8) = w;
      }
    }
  }
};

template <int NW>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attention_kernel(AttnArgs args) {
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kTileBytes + kFlagBytes];
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
