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
//     (dc/2)*1024 + (dc%2)*512 + (key ^ 4*(dc%2) ^ 8*((dc/2)%2))*16, which
//     the loader writes as 36 DMA instructions of 1 KiB and which keeps both
//     read patterns free of bank conflicts on the 64-bank LDS (16 lanes per
//     pass for 16-byte reads, 32 lanes for 8-byte reads);
//   * S^T = K . Q^T on v_mfma_f32_16x16x32_bf16: four independent
//     accumulator chains (2 key blocks x 2 head blocks of 16), so the 18
//     k-steps never wait on a previous MFMA's result.  One exchange of half
//     the scores with lane^16 then leaves each lane with 16 scores of ONE
//     head (lane l: head l%32, keys 16ks + 8(l/32) + e), so the softmax
//     statistics are per lane plus one cross-lane max per tile;
//   * O^T += V^T . P^T on v_mfma_f32_32x32x16_bf16 with latent columns as M
//     and heads as N: the probabilities are the B operand as they stand, and
//     the V^T operand is read from the same K tile with ds_read_b64_tr_b16,
//     whose 16-lane transpose turns four 8-byte row pieces into one column
//     each.  The 16 column blocks are independent accumulators;
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
constexpr int kQSteps = kLatentDim / 32;          // 18 k-steps of 32 over 576
constexpr int kDmaPerTile = kLatentDim / 16;      // 36 x 1 KiB (two 16-B chunks x 32 keys)
constexpr int kTileBytes = kDmaPerTile * 1024;    // 36864
constexpr int kStages = 4;
constexpr int kFlagBytes = 16;                    // per-wave redo flags after the stages
constexpr int kMaxItemPages = 1024;               // page ids staged per item (tile-aligned pages)
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

template <int NW, bool kTileInPage>
struct Attn {
  static constexpr int kLoadsPerWave = (kDmaPerTile + NW - 1) / NW;
  static constexpr int kWaitOne = kLoadsPerWave > 63 ? 63 : kLoadsPerWave;
  static constexpr int kWaitTwo = 2 * kLoadsPerWave > 63 ? 63 : 2 * kLoadsPerWave;

  const AttnArgs& a;
  char* smem;
  int lane, l32, half, wave, head;
  bool head_ok;
  int ld_key, ld_off, qk_off, pv_off0, pv_off1;  // per-lane LDS / row offsets
  uint32_t lds_base;                   // LDS address of the stages
  // current item
  int token, kv_end, slot;
  int page_base;   // index of the row's first page in kv_indices
  int first_page;  // row page index of the item's first key (tile-aligned pages)

  __device__ Attn(const AttnArgs& args, char* s) : a(args), smem(s) {
    const int tid = threadIdx.x;
    lane = tid & 63;
    l32 = lane & 31;
    half = lane >> 5;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    head = wave * 32 + l32;
    head_ok = head < a.num_heads;
    lds_base = static_cast<uint32_t>(reinterpret_cast<size_t>((__attribute__((address_space(3))) char*)smem));
    // loader: lane p of DMA instruction I fetches key (p%32) ^ 4(p/32) ^ 8(I%2),
    // chunk 2I + p/32 (the XOR by 8 is folded in when the DMA is issued)
    ld_key = l32 ^ (4 * half);
    ld_off = half * 16;
    // score operand (16x16x32, A = K): lane (l16 = key in a 16-key block,
    // g4 = lane/16) reads chunk 4ks + g4 of key 16kb + l16 at
    // ks*2048 + kb*256 + qk_off
    {
      const int l16 = lane & 15, g4 = lane >> 4;
      qk_off = (g4 >> 1) * 1024 + (g4 & 1) * 512 +
               ((l16 ^ (4 * (g4 & 1)) ^ (8 * ((g4 >> 1) & 1))) * 16);
    }
    // P.V operand through the 16-lane transpose read: group G = lane/16 is
    // (key half g2, 16-column group cg); source lane s of the group points at
    // key 16ks + 8g2 + 4r + s/4 for read r (0, 1), columns 16cg + 4(s%4) .. +3.
    const int G = lane >> 4, sl = lane & 15;
    const int g2 = G >> 1, cg = G & 1;
    const int par = (sl >> 1) & 1;  // chunk parity of the source columns
    const int pv_base = cg * 1024 + par * 512 + (sl & 1) * 8;
    pv_off0 = pv_base + ((8 * (g2 ^ cg) + 4 * (0 ^ par) + (sl >> 2)) * 16);
    pv_off1 = pv_base + ((8 * (g2 ^ cg) + 4 * (1 ^ par) + (sl >> 2)) * 16);
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
    if (kTileInPage)  // page_size % 32 == 0: the whole tile is in one page
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
  // state separates its write from the DMA.  Volatile asm keeps its order
  // against the barriers (also volatile asm); the stage it writes is not
  // read before the next barrier.
  __device__ __forceinline__ static void dma16(const char* src, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
                 : "m0");
  }

  // The same DMA with a uniform 64-bit base (SGPR pair) and a 32-bit lane
  // offset, for tiles that lie in one page.
  // Both uniform operands pass through readfirstlane so that they are SGPRs
  // even where the compiler cannot prove them uniform.
  __device__ __forceinline__ static void dma16s(uint32_t voff, const char* sbase,
                                                uint32_t lds_addr) {
    const uint64_t b = reinterpret_cast<uint64_t>(sbase);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
    const uint64_t sb = (static_cast<uint64_t>(hi) << 32) | lo;
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sb), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
                 : "m0");
  }

  // Source rows and LDS destination of one tile's DMAs for this lane: even
  // DMA instructions fetch key ld_key, odd ones key ld_key ^ 8.  Keys beyond
  // the item's range re-read its last key (finite data, masked later).
  struct TileDma {
    const char* src_e;  // general pages: per-lane row addresses
    const char* src_o;
    const char* sbase;  // tile in one page: page base (uniform) ...
    uint32_t voff_e;    // ... and the row offsets of the even / odd DMAs' key
    uint32_t voff_o;
    uint32_t dst;
  };

  __device__ __forceinline__ TileDma prep_tile(int base, int stage) const {
    const int P = a.page_size;
    int ke = base + ld_key, ko = base + (ld_key ^ 8);
    ke = ke < kv_end ? ke : kv_end - 1;
    ko = ko < kv_end ? ko : kv_end - 1;
    TileDma d;
    d.dst = lds_base + stage * kTileBytes;
    if (kTileInPage) {  // one page id per tile, staged in LDS for the item
      const int pg = __builtin_amdgcn_readfirstlane(page_lds()[base / P - first_page]);
      d.sbase = reinterpret_cast<const char*>(a.kv_cache + static_cast<int64_t>(pg) * P * kLatentDim);
      d.voff_e = static_cast<uint32_t>((ke % P) * (kLatentDim * 2) + ld_off);
      d.voff_o = static_cast<uint32_t>((ko % P) * (kLatentDim * 2) + ld_off);
      d.src_e = d.src_o = nullptr;
    } else {
      const int pe = lane_page(base, ke), po = lane_page(base, ko);
      d.src_e = reinterpret_cast<const char*>(
          a.kv_cache + (static_cast<int64_t>(pe) * P + ke % P) * kLatentDim) + ld_off;
      d.src_o = reinterpret_cast<const char*>(
          a.kv_cache + (static_cast<int64_t>(po) * P + ko % P) * kLatentDim) + ld_off;
      d.sbase = nullptr;
      d.voff_e = d.voff_o = 0;
    }
    return d;
  }

  // DMA instruction j (0 .. kLoadsPerWave-1) of this wave for a tile.
  __device__ __forceinline__ void issue_one(const TileDma& d, int j) const {
    const int I = wave + j * NW;
    if (NW * kLoadsPerWave == kDmaPerTile || I < kDmaPerTile) {
      if (kTileInPage)  // (with an even number of waves I has this wave's parity)
        dma16s(((I & 1) ? d.voff_o : d.voff_e) + I * 32, d.sbase, d.dst + I * 1024);
      else
        dma16(((I & 1) ? d.src_o : d.src_e) + I * 32, d.dst + I * 1024);
    }
  }

  __device__ __forceinline__ void issue_tile(int base, int stage) const {
    const TileDma d = prep_tile(base, stage);
#pragma unroll
    for (int j = 0; j < kLoadsPerWave; ++j) issue_one(d, j);
  }

  __device__ __forceinline__ int* page_lds() const {
    return reinterpret_cast<int*>(smem + kStages * kTileBytes + kFlagBytes);
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

      // Query as the B operand of the 16x16x32 score MFMAs: for head block
      // hb, lane (l16, g4) holds head 32 wave + 16 hb + l16, dims
      // 32 ks + 8 g4 .. +8.  Padding heads read head 0's row and zero it.
      bf16x8_t q[2][kQSteps];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int h = wave * 32 + hb * 16 + (lane & 15);
        const bool ok = h < H;
        const int hq = ok ? h : 0;
        const uint16_t* qn = a.q_nope + (static_cast<int64_t>(token) * H + hq) * kLoraRank;
        const uint16_t* qp = a.q_pe + (static_cast<int64_t>(token) * H + hq) * kRopeDim;
        const unsigned keep = ok ? 0xFFFFFFFFu : 0u;
        const int dl = 8 * (lane >> 4);
#pragma unroll
        for (int ks = 0; ks < kQSteps; ++ks) {
          u32x4_t v = ks < kLoraRank / 32
                          ? *reinterpret_cast<const u32x4_t*>(qn + ks * 32 + dl)
                          : *reinterpret_cast<const u32x4_t*>(qp + (ks - kLoraRank / 32) * 32 + dl);
          v &= keep;
          q[hb][ks] = __builtin_bit_cast(bf16x8_t, v);
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
        // Every wave is done with the previous item's output staging and
        // page ids (LDS); then this item's page ids are staged, and this
        // wave's query loads and earlier stores retire before the DMA queue
        // is counted tile by tile.
        __syncthreads();
        if (kTileInPage) {
          const int P = a.page_size;
          first_page = kv_begin / P;
          const int n = (kv_end - 1) / P - first_page + 1;  // <= kMaxItemPages
          for (int i = threadIdx.x; i < n; i += NW * kWave)
            page_lds()[i] = a.kv_indices[page_base + first_page + i];
          __syncthreads();
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        asm volatile("" ::: "memory");
#pragma unroll
        for (int t = 0; t < kStages - 1; ++t)
          if (t < ntiles) issue_tile(kv_begin + t * kTileKeys, t);
        bf16x8_t p[2];
        // Steady state (straight-line body): tile t has kStages-2 later
        // tiles in flight; tile t+3 is issued into the stage tile t-1 used.
        const int steady = ntiles - (kStages - 1);
        int t = 0;
        for (; t < steady; ++t) {
          wait_tile(kStages - 2);  // tile t has landed ...
          lds_barrier();           // ... for every wave; tile t-1 is free
          const TileDma dma =
              prep_tile(kv_begin + (t + kStages - 1) * kTileKeys, (t + kStages - 1) % kStages);
          const char* stage = smem + (t % kStages) * kTileBytes;
          float x[2][8];
          scores(stage, q, x);
          softmax<false>(x, kv_begin + t * kTileKeys, m_ref, m_seen, l_run, p);
          pv(stage, p, o, &dma);
        }
        // The last (up to kStages-1) tiles: everything is issued; the very
        // last one may be partial.
        for (; t < ntiles; ++t) {
          wait_tile(0);
          lds_barrier();
          const char* stage = smem + (t % kStages) * kTileBytes;
          float x[2][8];
          scores(stage, q, x);
          softmax<true>(x, kv_begin + t * kTileKeys, m_ref, m_seen, l_run, p);
          pv(stage, p, o);
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

  // S^T of the tile in stage K: four 16x16x32 accumulator chains
  // acc[kb][hb] (keys 16kb.., heads 16hb..), operands read kAhead k-steps
  // early; then the lane^16 exchange.  On return x[ks][e] is the score of
  // key 16ks + 8(lane/32) + e for head lane%32.
  __device__ __forceinline__ void scores(const char* K, const bf16x8_t (&q)[2][kQSteps],
                                         float (&x)[2][8]) const {
    constexpr int kAhead = 2;
    const char* kq = K + qk_off;
    auto kload = [&](int ks, int kb) {
      return *reinterpret_cast<const bf16x8_t*>(kq + ks * 2048 + kb * 256);
    };
    f32x4_t acc[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) acc[kb][hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    bf16x8_t kbuf[kAhead][2];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      kbuf[i][0] = kload(i, 0);
      kbuf[i][1] = kload(i, 1);
    }
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks) {
      const bf16x8_t k0 = kbuf[ks % kAhead][0], k1 = kbuf[ks % kAhead][1];
      if (ks + kAhead < kQSteps) {
        kbuf[ks % kAhead][0] = kload(ks + kAhead, 0);
        kbuf[ks % kAhead][1] = kload(ks + kAhead, 1);
      }
      acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, q[0][ks], acc[0][0], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, q[0][ks], acc[1][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, q[1][ks], acc[0][1], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, q[1][ks], acc[1][1], 0, 0, 0);
    }
    // Keep the reads kAhead k-steps ahead of their MFMAs.
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 0);  // DS reads
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // four MFMAs
      if (ks + kAhead < kQSteps) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    // acc[kb][hb][i] is key 16kb + 4(lane/16) + i of head 16hb + lane%16.
    // Lane l keeps head block hb_t = (l/16)%2 (its head l%32) and trades the
    // other block with lane l^16, whose head it is.
    const int g4 = lane >> 4;
    const bool odd = g4 & 1;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float own = odd ? acc[kb][1][i] : acc[kb][0][i];
        const float give = odd ? acc[kb][0][i] : acc[kb][1][i];
        const float got = __shfl_xor(give, 16);
        x[kb][i] = odd ? got : own;      // keys 16kb + 8(l/32) + i
        x[kb][4 + i] = odd ? own : got;  // keys 16kb + 8(l/32) + 4 + i
      }
    }
  }

  // Softmax of one tile's scores against the item's reference maximum:
  // p = 2^(s * scale_log2 - m_ref) as the bf16 P^T operand (x[ks][e] is key
  // 16ks + 8 half + e of the lane's head).
  template <bool kMask>
  __device__ __forceinline__ void softmax(float (&x)[2][8], int base, float& m_ref,
                                          float& m_seen, float& l_run, bf16x8_t (&p)[2]) const {
    float mx = -INFINITY;
    if (!kMask || base + kTileKeys <= kv_end) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, x[ks][e]);
    } else {  // the item's last tile: mask keys beyond its range
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = base + 16 * ks + 8 * half + e;
          x[ks][e] = key < kv_end ? x[ks][e] : -INFINITY;
          mx = fmaxf(mx, x[ks][e]);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * a.scale_log2;
    m_seen = fmaxf(m_seen, mx);
    if (m_ref == -INFINITY) m_ref = mx;  // first tile of the item: O is still zero
    const float neg_ref = -m_ref;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = __builtin_amdgcn_exp2f(
            fminf(__builtin_fmaf(x[ks][e], a.scale_log2, neg_ref), kMaxExponent));
        l_run += v;
        p[ks][e] = static_cast<__bf16>(v);
      }
  }

  // O^T += V^T . P^T for the tile in stage K: 32 MFMAs over 16 independent
  // accumulators (key half outermost, so consecutive MFMAs never depend on
  // each other); operands read kAhead steps early.  With `dma`, the next
  // tile's DMAs go out one every third MFMA, so their issue overlaps the
  // MFMA pipe instead of stalling the wave in one burst.
  __device__ __forceinline__ void pv(const char* K, const bf16x8_t (&p)[2],
                                     f32x16_t (&o)[kLoraRank / 32],
                                     const TileDma* dma = nullptr) const {
    constexpr int kAhead = 3;
    constexpr int kSteps = 2 * (kLoraRank / 32);
    const char* kv0 = K + pv_off0;
    const char* kv1 = K + pv_off1;
    auto vload = [&](int st) {  // column block st % 16, key half st / 16
      const int off = (st & 15) * 2048 + (st >> 4) * 256;
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(kv0 + off));
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(kv1 + off));
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8_t vbuf[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) vbuf[i] = vload(i);
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const bf16x8_t v = vbuf[st % kAhead];
      if (st + kAhead < kSteps) vbuf[st % kAhead] = vload(st + kAhead);
      o[st & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, p[st >> 4], o[st & 15], 0, 0, 0);
      if (dma && (st % 3) == 2 && st / 3 < kLoadsPerWave) issue_one(*dma, st / 3);
    }
    if (dma) {  // waves of fewer than 4 per workgroup issue more DMAs per tile
#pragma unroll
      for (int j = kSteps / 3; j < kLoadsPerWave; ++j) issue_one(*dma, j);
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

template <int NW, bool kTileInPage>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attention_kernel(AttnArgs args) {
  __shared__ __attribute__((aligned(1024)))
  char smem[kStages * kTileBytes + kFlagBytes + kMaxItemPages * 4];
  Attn<NW, kTileInPage> k(args, smem);
  k.run();
}

template <int NW>
hipError_t launch_nw(const AttnArgs& a, int num_workers, hipStream_t stream) {
  if (a.page_size % kTileKeys == 0)
    hipLaunchKernelGGL((attention_kernel<NW, true>), dim3(num_workers), dim3(NW * kWave), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((attention_kernel<NW, false>), dim3(num_workers), dim3(NW * kWave), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int num_workers, hipStream_t stream) {
  if (num_workers <= 0) return hipSuccess;
  switch ((a.num_heads + 31) / 32) {
    case 1: return launch_nw<1>(a, num_workers, stream);
    case 2: return launch_nw<2>(a, num_workers, stream);
    case 3: return launch_nw<3>(a, num_workers, stream);
    case 4: return launch_nw<4>(a, num_workers, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mla
