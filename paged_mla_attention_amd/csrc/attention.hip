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
//   * NW = 1, 2 or 4 waves hold 32 NW head slots.  For the scores wave w owns
//     heads [32w, 32w + 32) (its query rows stay in registers); for P . V it
//     owns latent columns [512w/NW, 512(w+1)/NW) of EVERY head, taking the
//     other waves' probabilities from LDS.  Splitting P . V by columns cuts
//     each wave's transposed V reads by NW (a wave issues one transposing
//     LDS read per ~24 cycles, which bounded a split by heads);
//   * keys are processed in tiles of 32.  A tile is copied from HBM straight
//     into LDS by global_load_lds (no staging registers) into four 36 KiB
//     stages, with explicit vmcnt waits and one bare s_barrier per tile;
//   * one swizzled LDS layout serves both products: 16-byte chunk (key, dc)
//     (dc = 8-column chunk of the 576 latent columns) sits at
//     (dc/2)*1024 + (dc%2)*512 + (key ^ 4*(dc%2) ^ 8*((dc/2)%2))*16, which
//     the loader writes as 36 DMA instructions of 1 KiB and which keeps both
//     read patterns free of bank conflicts;
//   * S^T = K . Q^T on v_mfma_f32_16x16x32_bf16: four independent
//     accumulator chains (2 key blocks x 2 head blocks of 16).  One exchange
//     of half the scores with lane^16 leaves each lane with 16 scores of ONE
//     head (lane l: head l%32, keys 16ks + 8(l/32) + e), already laid out as
//     the P^T operand of the 32x32x16 MFMA;
//   * O^T += V^T . P^T on v_mfma_f32_32x32x16_bf16 with latent columns as M
//     and heads as N; V^T is read from the same K tile with
//     ds_read_b64_tr_b16, whose 16-lane transpose turns four 8-byte row
//     pieces into one column each;
//   * software pipeline: iteration t computes S(t), then the softmax of tile
//     t (VALU) next to P . V of tile t-1 (MFMA), and publishes P(t) in one
//     of two LDS buffers.  Tile t+2 is DMA'd during S(t);
//   * softmax in base 2 against a per-head reference maximum fixed at the
//     item's first tile: p = 2^(x - m_ref) is exact for any reference (output
//     and LSE are normalised with the same value), so the O accumulators are
//     never rescaled inside the key loop.  A later score more than 2^64 above
//     the reference (which would overflow) makes the workgroup redo the item
//     with the largest score seen as the reference;
//   * page ids come through scalar loads issued one tile ahead, and the
//     query rows through asm loads with one explicit wait, so nothing inside
//     the key loop makes the in-order vmcnt drain the DMA queue;
//   * items covering a token's whole key range write bf16 output + LSE;
//     pieces of a split token write fp32 partials that a merge kernel combines.
#include <type_traits>
#include <utility>

#include "kernels.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef short s16x4_t __attribute__((vector_size(8)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(4))) const int32_t const_i32_t;

constexpr int kWave = 64;
constexpr int kQSteps = kLatentDim / 32;          // 18 k-steps of 32 over 576
constexpr int kDmaPerTile = kLatentDim / 16;      // 36 x 1 KiB (two 16-B chunks x 32 keys)
constexpr int kTileBytes = kDmaPerTile * 1024;    // 36864
constexpr int kStages = 4;
constexpr int kStageBytes = kStages * kTileBytes;
constexpr int kPGroupBytes = 2 * kWave * 16;      // one wave's P^T operands of a tile
constexpr float kMaxExponent = 64.0f;             // log2 headroom above the reference
// LDS layout of a tile: 16-byte chunk (key, dc) (dc = 8-column chunk of the
// 576 latent columns) at (dc/2)*1024 + (dc%2)*512 + ((key ^ swz(dc))*16)
// with swz(dc) = kSwzA*(dc%2) ^ kSwzB*((dc/2)%2).
constexpr int kSwzA = 4;
constexpr int kSwzB = 8;
constexpr float kLn2 = 0.693147180559945309f;

// s_waitcnt immediates (gfx9 encoding) that wait on one counter and leave
// the others alone.
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kLgkmZero = 0xF | (0x7 << 4) | (0x3 << 14);

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Barrier without the memory fence of __syncthreads (which would wait for
// every outstanding LDS DMA): this wave's LDS accesses have completed, then
// s_barrier.  The empty asm keeps the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kLgkmZero);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Pins an MFMA operand to VGPRs: left alone, the register allocator may
// load operands into AGPRs (MFMA accepts both), where they evict the
// output accumulators.  Applied where the operand is used (the asm waits for
// a pending load of it).
__device__ __forceinline__ void in_vgpr(bf16x8_t& v) { asm("" : "+v"(v)); }

// f(integral_constant<int, I>) for I = 0 .. N-1, in order, fully unrolled
// (the index is a compile-time constant in f).
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// A per-call copy of a lane value the compiler cannot see through: address
// arithmetic derived from it stays where it is used instead of being hoisted
// out of the item loop, where it would occupy (and spill) registers for the
// whole kernel.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

template <int NW, bool kTileInPage>
struct Attn {
  static constexpr int kDimBlocks = (kLoraRank / 32) / NW;  // 32-column blocks of O per wave
  static constexpr int kLoadsPerWave = kDmaPerTile / NW;    // DMA instructions per tile per wave
  static_assert(kDmaPerTile % NW == 0 && (kLoraRank / 32) % NW == 0, "NW must be 1, 2 or 4");
  static_assert(kLoadsPerWave <= 63, "vmcnt holds at most 63");
  static constexpr int kWaitTwo = 2 * kLoadsPerWave > 63 ? 63 : 2 * kLoadsPerWave;
  static constexpr int kPBufBytes = NW * kPGroupBytes;
  static constexpr int kFlagOff = kStageBytes + kPBufBytes;  // per-wave redo flags
  // Page ids of the current item (tiles that never span pages): an item has
  // at most kMaxItemTiles tiles, so at most that many pages.
  static constexpr int kPageOff = kFlagOff + 16;
  static constexpr int kPageLoads = (kMaxItemTiles + NW * kWave - 1) / (NW * kWave);
  static constexpr int kLdsBytes = kPageOff + (kTileInPage ? kMaxItemTiles * 4 : 16);
  // Output staging in the idle stages: per wave, 32 head rows of its columns.
  static constexpr int kFinRow = kDimBlocks * 32 + 4;  // floats (padding staggers banks)
  static constexpr int kFinWaveBytes = 32 * kFinRow * 4;
  static constexpr int kXchgOff = NW * kFinWaveBytes;  // 1/l of every head slot
  static_assert(kXchgOff + 32 * NW * 4 <= kStageBytes, "finish staging fits the stages");

  const AttnArgs& a;
  char* smem;
  int lane, l32, half, wave, head;
  bool head_ok;
  int ld_key, ld_off, qk_off, pv_off0, pv_off1;  // per-lane LDS / row offsets
  uint32_t lds_base;                               // LDS address of the stages
  // current item
  int token, kv_begin, kv_end, slot;
  int page_base;   // index of the row's first page in kv_indices
  int first_page;  // row page index of the item's first key

  __device__ Attn(const AttnArgs& args, char* s) : a(args), smem(s) {
    const int tid = threadIdx.x;
    lane = tid & 63;
    l32 = lane & 31;
    half = lane >> 5;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    head = wave * 32 + l32;
    head_ok = head < a.num_heads;
    lds_base = static_cast<uint32_t>(reinterpret_cast<size_t>((__attribute__((address_space(3))) char*)smem));
    // loader: lane p of DMA instruction I fetches key (p%32) ^ swz(2I + p/32),
    // chunk 2I + p/32 (the XOR by 8 is folded in when the DMA is issued)
    ld_key = l32 ^ (kSwzA * half);
    ld_off = half * 16;
    // score operand (16x16x32, A = K): lane (l16 = key in a 16-key block,
    // g4 = lane/16) reads chunk 4ks + g4 of key 16kb + l16 at
    // ks*2048 + kb*256 + qk_off
    {
      const int l16 = lane & 15, g4 = lane >> 4;
      qk_off = (g4 >> 1) * 1024 + (g4 & 1) * 512 +
               ((l16 ^ (kSwzA * (g4 & 1)) ^ (kSwzB * ((g4 >> 1) & 1))) * 16);
    }
    // P.V operand through the 16-lane transpose read: group G = lane/16 is
    // (key half g2, 16-column group cg); source lane s of the group points at
    // key 16ks + 8g2 + 4r + s/4 for read r (0, 1), columns 16cg + 4(s%4) .. +3.
    const int G = lane >> 4, sl = lane & 15;
    const int g2 = G >> 1, cg = G & 1;
    const int par = (sl >> 1) & 1;  // chunk parity of the source columns
    const int pv_base = cg * 1024 + par * 512 + (sl & 1) * 8;
    const int swz = kSwzA * par ^ kSwzB * cg;
    pv_off0 = pv_base + (((8 * g2 + (sl >> 2)) ^ swz) * 16);
    pv_off1 = pv_base + (((8 * g2 + 4 + (sl >> 2)) ^ swz) * 16);
  }

  __device__ __forceinline__ char* pbuf() const { return smem + kStageBytes; }
  __device__ __forceinline__ const char* stage(int t) const {
    return smem + (t % kStages) * kTileBytes;
  }

  // Page id of tile t of the item, from the item's page list in LDS (as a
  // VGPR value; the caller makes it uniform where it uses it).  LDS reads
  // keep the compiler's lgkmcnt waits exact, where a scalar load in flight
  // would make every LDS wait a full drain.
  __device__ __forceinline__ int tile_page_v(int t) const {
    const int* pl = reinterpret_cast<const int*>(smem + kPageOff);
    return pl[(kv_begin + t * kTileKeys) / a.page_size - first_page];
  }

  // Page id for the lane's own key `key` of the tile starting at `base`
  // when a tile can span pages: 32 scalar loads and a select (a vector load
  // here would make the in-order vmcnt wait for every DMA in flight).
  __device__ __forceinline__ int lane_page(int base, int key) const {
    const int P = a.page_size;
    const_i32_t* idx = (const_i32_t*)(a.kv_indices) + page_base;
    const int first = base / P;
    const int j = key / P - first;  // 0 .. 31
    int v = __builtin_amdgcn_readfirstlane(idx[first]);
#pragma unroll
    for (int i = 1; i < kTileKeys; ++i) {
      const int pi = __builtin_amdgcn_readfirstlane(idx[first + i]);
      v = (j == i) ? pi : v;
    }
    return v;
  }

  // One 16-byte-per-lane DMA from global memory into LDS at
  // m0 + offset + 16 * lane:
  // lane row address (64-bit VGPR pair, `off` form) or a uniform base (SGPR
  // pair) plus a 32-bit lane offset, each with a constant byte offset.
  // Issued through asm so that the compiler, which cannot tell the stages
  // apart, does not make later LDS reads wait for every DMA; the tile
  // pipeline waits on vmcnt itself.  One wait state separates the M0 write
  // from the DMA.  The stage it writes is not read before the next barrier.
  // The uniform operands pass through readfirstlane so that they are SGPRs
  // even where the compiler cannot prove them uniform.
  template <int kOff>
  __device__ __forceinline__ static void dma16(const char* src, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2"
                 :
                 : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "i"(kOff)
                 : "m0");
  }
  template <int kOff>
  __device__ __forceinline__ static void dma16s(uint32_t voff, const char* sbase,
                                                uint32_t lds_addr) {
    const uint64_t b = reinterpret_cast<uint64_t>(sbase);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
    const uint64_t sb = (static_cast<uint64_t>(hi) << 32) | lo;
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3"
                 :
                 : "v"(voff), "s"(sb), "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "i"(kOff)
                 : "m0");
  }

  // One tile's DMAs for this wave.  DMA instruction I = wave + j NW covers
  // 16-byte chunks 2I and 2I+1 (lane halves) of the 32 keys: lane p fetches
  // key (p%32) ^ 4(p/32) ^ 8(I%2) into LDS at 1024 I + 16 p.  The wave's
  // share of the row offset (32 I bytes) splits into a per-wave part folded
  // into the lane address and a constant per instruction.  Keys beyond the
  // item's range re-read its last key (finite data, masked later).
  struct TileDma {
    const char* src_e;  // tiles that may span pages: lane row address for
    const char* src_o;  //   even / odd I (+ 32 wave)
    const char* sbase;  // tile in one page: page base (uniform) ...
    uint32_t voff_e;    // ... and the lane row offsets for even / odd I
    uint32_t voff_o;
    uint32_t dst;       // LDS address of DMA I = wave
  };

  // Tile t of the item; `pg` is the page of its first key (used when tiles
  // never span pages).
  __device__ __forceinline__ TileDma prep_tile(int t, int pg) const {
    const int P = a.page_size;
    const int base = kv_begin + t * kTileKeys;
    int ke = base + ld_key, ko = base + (ld_key ^ kSwzB);
    ke = ke < kv_end ? ke : kv_end - 1;
    ko = ko < kv_end ? ko : kv_end - 1;
    TileDma d;
    d.dst = lds_base + (t % kStages) * kTileBytes + wave * 1024;
    if (kTileInPage) {  // the tile lies in page pg: key k is row k - base + base % P
      const int in_page = base % P;
      d.sbase = reinterpret_cast<const char*>(a.kv_cache + static_cast<int64_t>(pg) * P * kLatentDim);
      d.voff_e = static_cast<uint32_t>((in_page + ke - base) * (kLatentDim * 2) + ld_off + wave * 32);
      d.voff_o = static_cast<uint32_t>((in_page + ko - base) * (kLatentDim * 2) + ld_off + wave * 32);
      d.src_e = d.src_o = nullptr;
    } else {
      const int pe = lane_page(base, ke), po = lane_page(base, ko);
      d.src_e = reinterpret_cast<const char*>(
          a.kv_cache + (static_cast<int64_t>(pe) * P + ke % P) * kLatentDim) + ld_off + wave * 32;
      d.src_o = reinterpret_cast<const char*>(
          a.kv_cache + (static_cast<int64_t>(po) * P + ko % P) * kLatentDim) + ld_off + wave * 32;
      d.sbase = nullptr;
      d.voff_e = d.voff_o = 0;
    }
    return d;
  }

  // DMA instruction I = wave + j NW of this wave for a tile.  With an even
  // number of waves I has the wave's parity; with one wave, j's.
  template <int j>
  __device__ __forceinline__ void issue_one(const TileDma& d) const {
    constexpr int kOff = j * NW * 32;
    // The instruction offset moves the LDS destination as well as the
    // global address, so M0 takes it back off.
    const uint32_t dst = d.dst + j * NW * 1024 - kOff;
    const bool odd = NW == 1 ? (j & 1) : (wave & 1);
    if (kTileInPage)
      dma16s<kOff>(odd ? d.voff_o : d.voff_e, d.sbase, dst);
    else
      dma16<kOff>(odd ? d.src_o : d.src_e, dst);
  }

  template <int j0, int j1>
  __device__ __forceinline__ void issue_range(const TileDma& d) const {
    if constexpr (j0 < j1) {
      issue_one<j0>(d);
      issue_range<j0 + 1, j1>(d);
    }
  }

  __device__ __forceinline__ void issue_tile(int t, int pg) const {
    const TileDma d = prep_tile(t, pg);
    issue_range<0, kLoadsPerWave>(d);
  }

  // Waits for this wave's DMAs except those of the `later` newest tiles.
  __device__ __forceinline__ static void wait_vm(int later) {
    if (later >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kWaitTwo));
    else if (later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadsPerWave));
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
      kv_begin = item[2];
      kv_end = item[3];
      slot = item[4];
      page_base = ((const_i32_t*)(a.kv_indptr))[row];
      const int ntiles = (kv_end - kv_begin + kTileKeys - 1) / kTileKeys;

      f32x16_t o[NW][kDimBlocks];
      float m_ref = -INFINITY;  // reference max of scaled base-2 scores (per head)
      float m_seen = -INFINITY; // largest scaled score seen by this lane
      float l_run = 0.f;        // this lane's share of the softmax denominator
      for (;;) {
#pragma unroll
        for (int g = 0; g < NW; ++g)
#pragma unroll
          for (int db = 0; db < kDimBlocks; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) o[g][db][j] = 0.f;
        l_run = 0.f;
        m_seen = -INFINITY;
        if (ntiles == 0) break;
        if (kTileInPage) {
          // Stage the item's page ids in LDS; the loads go out before the
          // barrier that waits for the previous item's LDS users.
          const int P = a.page_size;
          first_page = kv_begin / P;
          const int n = (kv_end - 1) / P - first_page + 1;  // <= kMaxItemTiles
          int pv[kPageLoads];
#pragma unroll
          for (int k = 0; k < kPageLoads; ++k) {
            const int i = threadIdx.x + k * NW * kWave;
            pv[k] = i < n ? reinterpret_cast<const int32_t*>(a.kv_indices)[page_base + first_page + i] : 0;
          }
          lds_barrier();
          int* pl = reinterpret_cast<int*>(smem + kPageOff);
#pragma unroll
          for (int k = 0; k < kPageLoads; ++k) {
            const int i = threadIdx.x + k * NW * kWave;
            if (i < n) pl[i] = pv[k];
          }
        }
        // Every wave is done with the previous item's (or attempt's) LDS,
        // and the page list is complete.
        lds_barrier();
#pragma unroll
        for (int t = 0; t < kStages - 1; ++t)
          if (t < ntiles)
            issue_tile(t, kTileInPage ? __builtin_amdgcn_readfirstlane(tile_page_v(t)) : 0);
        int pg_next = kTileInPage && ntiles > kStages - 1 ? tile_page_v(kStages - 1) : 0;
        // Query as the B operand of the 16x16x32 score MFMAs: for head block
        // hb, lane (l16, g4) holds head 32 wave + 16 hb + l16, dims
        // 32 ks + 8 g4 .. +8.  Padding heads (beyond H) compute with head 0's
        // row; their results are never stored.  Loaded after the first
        // tiles' DMAs (the memory clobber keeps that order), so the
        // compiler's waits for these loads also cover the DMAs before them.
        asm volatile("" ::: "memory");
        // (A redo attempt loads them again.)
        u32x4_t q[2][kQSteps];
        {
          const int qlane = opaque(lane);
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            const int h = wave * 32 + hb * 16 + (qlane & 15);
            const int hq = h < H ? h : 0;
            const uint16_t* qn = a.q_nope + (static_cast<int64_t>(token) * H + hq) * kLoraRank;
            const uint16_t* qp = a.q_pe + (static_cast<int64_t>(token) * H + hq) * kRopeDim;
            const int dl = 8 * (qlane >> 4);
#pragma unroll
            for (int ks = 0; ks < kQSteps; ++ks)
              q[hb][ks] = ks < kLoraRank / 32
                              ? *reinterpret_cast<const u32x4_t*>(qn + ks * 32 + dl)
                              : *reinterpret_cast<const u32x4_t*>(qp + (ks - kLoraRank / 32) * 32 + dl);
          }
        }
        // Tile t: S(t) (with the DMAs of tile t+3 in between), softmax,
        // P(t) published in LDS, then this wave's columns of P . V for every
        // head.  Barriers: tile t landed for every wave and P . V of t-1
        // done (its stage and the P buffer are free); P(t) complete.  One
        // loop body for every tile (uniform branches for the first tile, the
        // DMAs and the partial last tile) keeps the code and its register
        // allocation single.
        for (int t = 0; t < ntiles; ++t) {
          wait_vm(ntiles - 1 - t);
          lds_barrier();
          const bool dma = t + kStages - 1 < ntiles;
          TileDma d;
          auto prep = [&] {
            d = prep_tile(t + kStages - 1, kTileInPage ? __builtin_amdgcn_readfirstlane(pg_next) : 0);
            if (kTileInPage) {  // the next tile's page id, read a tile ahead
              const int tn = t + kStages < ntiles ? t + kStages : ntiles - 1;
              pg_next = tile_page_v(tn);
            }
          };
          // With several waves, tile t+3's DMA set-up goes under the first
          // k-step's MFMAs (a lone wave, with four times the DMAs, has no
          // registers to spare there).  Its DMAs go under the other k-steps.
          constexpr bool kPrepUnder = NW > 1;
          if (!kPrepUnder && dma) prep();
          float x[2][8];
          scores(stage(t), q, x, [&](auto kc) {
            constexpr int k = decltype(kc)::value;
            if (!dma) return;
            if constexpr (k == 0) {
              if (kPrepUnder) prep();
            } else {
              dma_step<k>(d);
            }
          });
          bf16x8_t p[2];
          softmax(x, kv_begin + t * kTileKeys, t == 0, m_ref, m_seen, l_run, p);
          store_p(p);
          lds_barrier();
          pv(stage(t), o);
        }
        // Redo the item if any head of the workgroup overflowed its reference.
        int* flags = reinterpret_cast<int*>(smem + kFlagOff);
        const bool redo = __any(m_seen > m_ref + kMaxExponent);
        if (lane == 0) flags[wave] = redo ? 1 : 0;
        lds_barrier();
        int any_redo = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) any_redo |= flags[w];
        if (!any_redo) break;
        m_ref = fmaxf(m_seen, __shfl_xor(m_seen, 32));  // the head's largest score
      }
      finish(o, m_ref, l_run);
    }
  }

  __device__ __forceinline__ void store_p(const bf16x8_t (&p)[2]) const {
    char* pb = pbuf();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      *reinterpret_cast<bf16x8_t*>(pb + wave * kPGroupBytes + ks * (kWave * 16) + lane * 16) = p[ks];
  }

  // The DMAs issued under k-step ks = 1 .. 17 of a score pass (k-step 0
  // prepares them), spread evenly.
  template <int ks>
  __device__ __forceinline__ void dma_step(const TileDma& d) const {
    static_assert(ks >= 1 && ks < kQSteps, "DMAs go under k-steps 1 .. 17");
    constexpr int kN = kQSteps - 1;
    issue_range<(ks - 1) * kLoadsPerWave / kN, ks * kLoadsPerWave / kN>(d);
  }

  // S^T of the tile in stage K: four 16x16x32 accumulator chains
  // acc[kb][hb] (keys 16kb.., heads 16hb..), operands read kAhead k-steps
  // early; with dma a later tile's DMAs go out between the k-steps.  Then
  // the lane^16 exchange.  On return x[ks][e] is the score of key
  // 16ks + 8(lane/32) + e for head lane%32.
  template <typename Extra>
  __device__ __forceinline__ void scores(const char* K, const u32x4_t (&q)[2][kQSteps],
                                         float (&x)[2][8], Extra&& extra) const {
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
    static_for<kQSteps>([&](auto kc) {
      constexpr int ks = decltype(kc)::value;
      bf16x8_t k0 = kbuf[ks % kAhead][0], k1 = kbuf[ks % kAhead][1];
      in_vgpr(k0);  // (at the use: the asm waits for the load)
      in_vgpr(k1);
      if constexpr (ks + kAhead < kQSteps) {
        kbuf[ks % kAhead][0] = kload(ks + kAhead, 0);
        kbuf[ks % kAhead][1] = kload(ks + kAhead, 1);
      }
      acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, __builtin_bit_cast(bf16x8_t, q[0][ks]), acc[0][0], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, __builtin_bit_cast(bf16x8_t, q[0][ks]), acc[1][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, __builtin_bit_cast(bf16x8_t, q[1][ks]), acc[0][1], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, __builtin_bit_cast(bf16x8_t, q[1][ks]), acc[1][1], 0, 0, 0);
      extra(kc);  // work placed under this k-step's MFMAs
      // Keep each k-step's reads kAhead steps ahead instead of letting the
      // scheduler hoist all 36 (they would not fit in registers).
      __builtin_amdgcn_sched_barrier(0);
    });
    // acc[kb][hb][i] is key 16kb + 4(lane/16) + i of head 16hb + lane%16.
    // Lane l keeps head block (l/16)%2 (its head l%32) and trades the other
    // block with lane l^16, whose head it is.
    const int g4 = lane >> 4;
    const bool odd = g4 & 1;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float own = odd ? acc[kb][1][i] : acc[kb][0][i];
        const float give = odd ? acc[kb][0][i] : acc[kb][1][i];
        const float got = __shfl_xor(give, 16);
        x[kb][i] = odd ? got : own;
        x[kb][4 + i] = odd ? own : got;
      }
    }
  }

  // Softmax of one tile's scores against the item's reference maximum:
  // p = 2^(s * scale_log2 - m_ref) as the bf16 P^T operand (x[ks][e] is key
  // 16ks + 8 half + e of the lane's head).  The first tile of an attempt
  // fixes the reference (unless a redo has set it); keys past the item's end
  // (last tile only) get probability 0.
  __device__ __forceinline__ void softmax(float (&x)[2][8], int base, bool first, float& m_ref,
                                          float& m_seen, float& l_run, bf16x8_t (&p)[2]) const {
    if (__builtin_expect(base + kTileKeys > kv_end, 0)) {  // the item's last tile only
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = base + 16 * ks + 8 * half + e;
          x[ks][e] = key < kv_end ? x[ks][e] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, x[ks][e]);
    mx *= a.scale_log2;
    m_seen = fmaxf(m_seen, mx);
    if (first) {
      const float mh = fmaxf(mx, __shfl_xor(mx, 32));
      if (m_ref == -INFINITY) m_ref = mh;  // O is still zero
    }
    // No clamp against overflow: a score more than 2^64 above the reference
    // makes the item redo with a new reference, so whatever an overflow
    // leaves in the accumulators is discarded.
    const float neg_ref = -m_ref;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = __builtin_amdgcn_exp2f(__builtin_fmaf(x[ks][e], a.scale_log2, neg_ref));
        l_run += v;
        p[ks][e] = static_cast<__bf16>(v);
      }
  }

  // O^T += V^T . P^T for the tile in stage V with the probabilities of every
  // head slot in P buffer Pb: this wave's 32-column blocks
  // [w kDimBlocks, (w+1) kDimBlocks) times each head group's P^T.
  // Consecutive MFMAs go to different accumulators; V^T operands are read
  // kAhead column blocks early.
  __device__ __forceinline__ void pv(const char* V, f32x16_t (&o)[NW][kDimBlocks]) const {
    const char* Pb = pbuf();
    constexpr int kSteps = 2 * kDimBlocks;  // (key half, column block)
    constexpr int kAhead = NW == 1 ? 4 : 2;
    const char* kv0 = V + pv_off0 + wave * kDimBlocks * 2048;
    const char* kv1 = V + pv_off1 + wave * kDimBlocks * 2048;
    auto vload = [&](int st) {  // column block st % kDimBlocks, key half st / kDimBlocks
      const int off = (st % kDimBlocks) * 2048 + (st / kDimBlocks) * 256;
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(kv0 + off));
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(kv1 + off));
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto pload = [&](int g, int ks) {
      return *reinterpret_cast<const bf16x8_t*>(Pb + g * kPGroupBytes + ks * (kWave * 16) +
                                                lane * 16);
    };
    bf16x8_t pb[NW], pn[NW];
#pragma unroll
    for (int g = 0; g < NW; ++g) pb[g] = pload(g, 0);
    bf16x8_t vbuf[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) vbuf[i] = vload(i);
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      bf16x8_t v = vbuf[st % kAhead];
      in_vgpr(v);  // (at the use: the asm waits for the load)
      if (st + kAhead < kSteps) vbuf[st % kAhead] = vload(st + kAhead);
      const int db = st % kDimBlocks;
      if (st == kDimBlocks / 2) {  // the second key half's P^T, half a pass early
#pragma unroll
        for (int g = 0; g < NW; ++g) pn[g] = pload(g, 1);
      }
      if (st == kDimBlocks) {
#pragma unroll
        for (int g = 0; g < NW; ++g) pb[g] = pn[g];
      }
#pragma unroll
      for (int g = 0; g < NW; ++g) {
        bf16x8_t b = pb[g];
        in_vgpr(b);
        o[g][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, b, o[g][db], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Writes the item's result.  The accumulators are never touched by VALU
  // code here (that makes the compiler shuttle all 256 of them through
  // VGPRs).  Lane l holds, for head group g, head 32g + l%32 and columns
  // 32 (w kDimBlocks + db) + 8 (j/4) + 4 (l/32) + j%4.  The raw sums go
  // through this wave's LDS region head group by head group; then each lane
  // normalises (1/l of the head, from its owner wave through LDS), converts
  // and stores 16 bytes.  The caller has made the LDS stages free.
  __device__ __forceinline__ void finish(f32x16_t (&o)[NW][kDimBlocks], float m_ref,
                                         float l_run) const {
    const int lane = opaque(this->lane);
    const int l32 = lane & 31, half = lane >> 5;
    const int head = wave * 32 + l32;
    const bool head_ok = head < a.num_heads;
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const bool any = l_tot > 0.f;
    const float inv = any ? 1.f / l_tot : 0.f;
    const float lse_v = any ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
    const int H = a.num_heads;
    const int col0 = wave * kDimBlocks * 32;
    // A final item writes the token's output and LSE; a piece of a split
    // token writes the same normalised bf16 rows and LSE to its slot.
    const int64_t row0 = static_cast<int64_t>(slot >= 0 ? slot : token) * H;
    uint16_t* dst_o = (slot >= 0 ? a.part_o : a.out) + row0 * kLoraRank;
    float* dst_lse = slot >= 0 ? a.part_lse + row0 : (a.lse ? a.lse + row0 : nullptr);
    float* X = reinterpret_cast<float*>(smem + kXchgOff);
    if (half == 0) X[head] = inv;
    if (dst_lse && head_ok && half == 0) dst_lse[head] = lse_v;
    lds_barrier();
    float* R = reinterpret_cast<float*>(smem + wave * kFinWaveBytes);
    constexpr int kChunks = kDimBlocks * 4;  // 8-column chunks per head row
#pragma unroll
    for (int g = 0; g < NW; ++g) {
#pragma unroll
      for (int db = 0; db < kDimBlocks; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4_t w = {o[g][db][4 * q4], o[g][db][4 * q4 + 1], o[g][db][4 * q4 + 2],
                             o[g][db][4 * q4 + 3]};
          *reinterpret_cast<f32x4_t*>(R + l32 * kFinRow + db * 32 + q4 * 8 + half * 4) = w;
        }
      // lane: head h = (lane + 64 r) / kChunks of the group, chunk cc.  Reads
      // go out in batches ahead of the conversions and stores.
      constexpr int kIters = 32 * kChunks / kWave;
      constexpr int kBatch = kIters < 8 ? kIters : 8;
#pragma unroll
      for (int r0 = 0; r0 < kIters; r0 += kBatch) {
        f32x4_t v0[kBatch], v1[kBatch];
        float sc[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          const int qi = lane + kWave * (r0 + b);
          const int h = qi / kChunks, cc = qi % kChunks;
          v0[b] = *reinterpret_cast<const f32x4_t*>(R + h * kFinRow + cc * 8);
          v1[b] = *reinterpret_cast<const f32x4_t*>(R + h * kFinRow + cc * 8 + 4);
          sc[b] = X[g * 32 + h];
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          const int qi = lane + kWave * (r0 + b);
          const int h = qi / kChunks, cc = qi % kChunks;
          const int hg = g * 32 + h;
          u32x4_t w;
          w[0] = f32_to_bf16_bits(v0[b][0] * sc[b]) | (static_cast<unsigned>(f32_to_bf16_bits(v0[b][1] * sc[b])) << 16);
          w[1] = f32_to_bf16_bits(v0[b][2] * sc[b]) | (static_cast<unsigned>(f32_to_bf16_bits(v0[b][3] * sc[b])) << 16);
          w[2] = f32_to_bf16_bits(v1[b][0] * sc[b]) | (static_cast<unsigned>(f32_to_bf16_bits(v1[b][1] * sc[b])) << 16);
          w[3] = f32_to_bf16_bits(v1[b][2] * sc[b]) | (static_cast<unsigned>(f32_to_bf16_bits(v1[b][3] * sc[b])) << 16);
          if (hg < H)
            *reinterpret_cast<u32x4_t*>(dst_o + static_cast<int64_t>(hg) * kLoraRank + col0 + cc * 8) = w;
        }
      }
    }
  }
};

template <int NW, bool kTileInPage>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attention_kernel(AttnArgs args) {
  __shared__ __attribute__((aligned(1024))) char smem[Attn<NW, kTileInPage>::kLdsBytes];
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
  if (a.num_heads <= 0 || a.num_heads > kMaxHeads) return hipErrorInvalidValue;
  if (a.num_heads <= 32) return launch_nw<1>(a, num_workers, stream);
  if (a.num_heads <= 64) return launch_nw<2>(a, num_workers, stream);
  return launch_nw<4>(a, num_workers, stream);
}

}  // namespace mla
