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
//     into LDS by global_load_lds (no staging registers): its ckv columns
//     into one of four 32 KiB stages, its kpe columns (read by the scores
//     only) into one of three 4 KiB slots, two tiles ahead of the one being
//     computed, with explicit vmcnt waits and bare s_barriers.  DMA
//     addresses step through the item's page list (staged in LDS) with no
//     division per tile;
//   * one swizzled LDS layout serves both products: 16-byte chunk (key, dc)
//     (dc = 8-column chunk of the latent columns) sits at
//     (dc/2)*1024 + (dc%2)*512 + (key ^ 4*(dc%2) ^ 8*((dc/2)%2))*16 of its
//     stage or slot, which the loader writes as 1 KiB DMA instructions and
//     which keeps both read patterns free of bank conflicts;
//   * S^T = K . Q^T as one chain of 36 v_mfma_f32_32x32x16_bf16 over the
//     576 columns (keys as M, the wave's 32 heads as N).  Its accumulator
//     layout gives lane l 16 scores of head l%32 (keys 8i + 4(l/32) + j),
//     which is the P^T operand of the P . V MFMA once the V^T reads take
//     the keys in the same order: no lane exchange;
//   * O^T += V^T . P^T on v_mfma_f32_32x32x16_bf16 with latent columns as M
//     and heads as N; V^T is read from the same stage with
//     ds_read_b64_tr_b16, whose 16-lane transpose turns four 8-byte row
//     pieces into one column each;
//   * software pipeline (several waves, tiles within pages): iteration t
//     computes S(t), then P . V of tile t-1 with the softmax of S(t) placed
//     between its MFMAs, and publishes P(t) in the other of two LDS
//     buffers; one barrier per tile;
//   * softmax in base 2 against a per-head reference maximum fixed at the
//     item's first tile: p = 2^(x - m_ref) is exact for any reference (output
//     and LSE are normalised with the same value), so the O accumulators are
//     never rescaled inside the key loop.  A later score more than 2^64 above
//     the reference (which would overflow) makes the workgroup redo the item
//     with the largest score seen as the reference;
//   * the query rows are loaded and waited for before the item's first DMA,
//     and page ids come from LDS, so nothing inside the key loop makes the
//     in-order vmcnt drain the DMA queue;
//   * at most 32 heads (one computing wave), two workgroups share a compute
//     unit in 80 KiB of LDS each; with an fp8 cache (and a bf16 one of at
//     most 16 heads) each of them adds a producer wave on an otherwise idle
//     SIMD that loads the rows two tiles ahead into its registers and
//     converts or copies them into the stages while the computing wave runs
//     the products (run_split);
//   * at most 16 heads: the computing wave holds 16 head slots on
//     v_mfma_f32_16x16x32_bf16 (kH16), so no MFMA computes padding, and the
//     probabilities stay in registers between the two products;
//   * items covering a token's whole key range write bf16 output + LSE;
//     pieces of a split token write normalised bf16 partials and their LSE,
//     which a merge kernel combines.
#include <type_traits>
#include <utility>

#include "kernels.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;
typedef short s16x4_t __attribute__((vector_size(8)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(4))) const int32_t const_i32_t;

constexpr int kWave = 64;
constexpr int kQSteps = kLatentDim / 16;          // 36 k-steps of 16 over 576
constexpr int kDmaPerTile = kLatentDim / 16;      // 36 x 1 KiB (two 16-B chunks x 32 keys)
constexpr int kCkvDmas = kLoraRank / 16;          // 32 of the 36 carry ckv columns
constexpr int kCkvBytes = kCkvDmas * 1024;        // a tile's ckv part (32 KiB)
constexpr int kKpeBytes = (kDmaPerTile - kCkvDmas) * 1024;  // its kpe part (4 KiB)
constexpr int kStages = 4;                        // ckv stages
constexpr int kKpeSlots = 3;                      // kpe slots (read by the scores only)
constexpr int kStageBytes = kStages * kCkvBytes;
constexpr int kKpeOff = kStageBytes;
constexpr int kTilesAhead = 2;                    // tiles in flight beyond the current one
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

// v_mfma_f32_32x32x16_bf16 with its accumulator in VGPRs.  The compiler
// gives every MFMA of a function the AGPR form once the function needs
// AGPRs (the output accumulators fill them), so the score chain is issued
// here.  Back-to-back MFMAs into the same accumulator need no wait states;
// mfma_settle provides those before other instructions read the result.
__device__ __forceinline__ void mfma_v_first(f32x16_t& acc, const bf16x8_t& a, const u32x4_t& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x16_t& acc, const bf16x8_t& a, const u32x4_t& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_settle(f32x16_t& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
}

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

// Eight E4M3 codes (two dwords) as eight bf16 values, exactly (every E4M3
// value is a bf16 value).
__device__ __forceinline__ u32x4_t cvt_fp8x8(uint32_t w0, uint32_t w1) {
  u32x4_t o;
  o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
  o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
  o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
  o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  return o;
}

// A per-call copy of a lane value the compiler cannot see through: address
// arithmetic derived from it stays where it is used instead of being hoisted
// out of the item loop, where it would occupy (and spill) registers for the
// whole kernel.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// An fp8 cache (kFp8): a tile's 32 latent rows are 32 x 576 E4M3 codes
// (18 KiB).  Each wave DMAs the raw codes of the latent columns it owns in
// P . V ([512w/NW, 512(w+1)/NW), two 16-column chunks of the 32 keys per
// 1 KiB instruction) and a quarter of the kpe columns (one 16-column chunk
// per 512-byte, half-wave instruction) into its own slice of a two-slot raw
// ring, and converts them itself, exactly (every code is a bf16 value),
// into the bf16 stage layout the score and P . V reads use.  It converts
// tile t+1 right after its own P . V of tile t-1, whose stage (and kpe
// slot) tile t+1 reuses: no other wave reads those columns in P . V, and
// the scores of tile t-1 were done before this iteration's barrier.  So two
// bf16 stages and two raw slots suffice, with the DMAs still two tiles ahead.
// A compact one-wave variant (kCompact, bf16 stages only) in 80 KiB of LDS,
// so that two workgroups share a compute unit (the host plans two workers
// per compute unit for it): two ckv stages and two kpe slots with one tile
// in flight.  With an fp8 cache (and a bf16 one of at most 16 heads) the
// same layout serves the two-wave split kernel (run_split), whose second
// wave fills the stages.
template <int NW, bool kTileInPage, bool kFp8, bool kCompact, bool kH16 = false>
struct Attn {
  static_assert(!kCompact || NW == 1, "the compact variant is one wave");
  static_assert(!kH16 || (NW == 1 && kCompact && !kFp8), "16 head slots: the split kernel");
  static_assert(!(kCompact && kFp8), "an fp8 cache with the compact layout runs run_split");
  // Tiles whose DMAs are in flight beyond the one being computed.
  static constexpr int kAhead = kCompact ? 1 : kTilesAhead;
  static constexpr int kDimBlocks = (kLoraRank / 32) / NW;  // 32-column blocks of O per wave
  // DMA instructions per tile per wave: bf16 36 / NW; fp8 16 / NW ckv + 4 / NW kpe.
  static constexpr int kCkvLoads = kFp8 ? 16 / NW : 0;
  static constexpr int kKpeLoads = kFp8 ? 4 / NW : 0;
  static constexpr int kLoadsPerWave = kFp8 ? kCkvLoads + kKpeLoads : kDmaPerTile / NW;
  static_assert(kDmaPerTile % NW == 0 && (kLoraRank / 32) % NW == 0, "NW must be 1, 2 or 4");
  static_assert(kLoadsPerWave <= 63, "vmcnt holds at most 63");
  static constexpr int kNStages = kFp8 || kCompact ? 2 : kStages;  // bf16 ckv stages
  static constexpr int kNKpe = kFp8 || kCompact ? 2 : kKpeSlots;     // bf16 kpe slots
  static constexpr int kStageB = kNStages * kCkvBytes;
  static constexpr int kKpeO = kStageB;
  // fp8 raw ring: two slots of 18 KiB, wave w's slice at w * kRawWaveBytes
  // (its ckv instructions at 1 KiB steps, then its kpe ones at 512 B steps).
  static constexpr int kRawOff = kKpeO + kNKpe * kKpeBytes;
  static constexpr int kRawSlotBytes = kFp8 ? kLatentDim * kTileKeys : 0;
  static constexpr int kRawWaveBytes = kRawSlotBytes / NW;
  static constexpr int kRawSlots = kFp8 ? 2 : 0;
  static_assert(!kFp8 || kRawWaveBytes == kCkvLoads * 1024 + kKpeLoads * 512, "raw slice");
  static constexpr int kPBufBytes = NW * kPGroupBytes;
  static constexpr int kPOff = kRawOff + kRawSlots * kRawSlotBytes;  // two P buffers
  // Per-wave redo flags (used after the key loop only): in a kpe slot, or
  // for an fp8 cache in the raw ring (the finish staging reaches into the
  // kpe slots there).
  static constexpr int kFlagOff = kFp8 ? kRawOff : kKpeO;
  // Page ids of the current item (tiles that never span pages): an item has
  // at most kMaxItemTiles tiles, so at most that many pages.  Above the
  // query staging, which is in flight with the page-list DMA.
  static constexpr int kQWaveBytes = 32 * kLatentDim * 2;
  static constexpr int kPageOff =
      kPOff + 2 * kPBufBytes > NW * kQWaveBytes ? kPOff + 2 * kPBufBytes : NW * kQWaveBytes;
  static constexpr int kPageLoads = (kMaxItemTiles + NW * kWave - 1) / (NW * kWave);
  // Tiles that may span pages: each wave keeps the page ids of its lanes'
  // keys for kIdSlots tiles (32 ids of 4 bytes per tile), DMA'd kIdAhead
  // tiles ahead of their use.
  static constexpr int kIdSlots = 8;
  static constexpr int kIdAhead = 4;
  static constexpr int kIdWaveBytes = kIdSlots * kTileKeys * 4;
  static constexpr int kLdsBytes = kPageOff + (kTileInPage ? kMaxItemTiles * 4 : NW * kIdWaveBytes);
  static_assert(kLdsBytes <= 160 * 1024, "LDS holds 160 KiB");
  // Output staging in the idle stages: per wave, 32 head rows of its columns.
  static constexpr int kFinRow = kDimBlocks * 32 + 4;  // floats (padding staggers banks)
  static constexpr int kFinWaveBytes = 32 * kFinRow * 4;
  static constexpr int kXchgOff = NW * kFinWaveBytes;  // 1/l of every head slot
  // (a lone wave reads its redo flags before its finish staging covers them)
  static_assert(kXchgOff + 32 * NW * 4 <= (kCompact ? kPOff : (kFp8 ? kRawOff : kStageB)),
                "finish staging fits the stages (and kpe slots)");

  const AttnArgs& a;
  char* smem;
  int lane, l32, half, wave, head;
  bool head_ok;
  int ld_key, ld_off, qk_off_e, qk_off_o, pv_off0, pv_off1;  // per-lane LDS / row offsets
  int k16_off0, k16_off1, v16_off_e, v16_off_o;      // (16 head slots)
  uint32_t lds_base;                               // LDS address of the stages
  float scale_log2;                                // sm_scale * log2(e)
  // current item
  int token, kv_begin, kv_end, slot;
  int page_base;   // index of the row's first page in kv_indices
  int first_page;  // row page index of the item's first key

  __device__ Attn(const AttnArgs& args, char* s) : a(args), smem(s) {
    // (an fp8 cache's scale multiplies every score: out_scale is 1 for bf16)
    scale_log2 = (args.scale_log2_ptr ? *args.scale_log2_ptr : args.scale_log2) * args.out_scale;
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
    // score operand (32x32x16, A = K): lane (key l32, dim half `half`)
    // reads chunk 2ks + half of its key, at ks*1024 + qk_off_e (even ks) or
    // qk_off_o (odd ks): one contiguous 256-byte run per 16 lanes.
    qk_off_e = half * 512 + ((l32 ^ (kSwzA * half)) * 16);
    qk_off_o = half * 512 + ((l32 ^ (kSwzA * half) ^ kSwzB) * 16);
    // P.V operand through the 16-lane transpose read: group G = lane/16 is
    // (key half g2, 16-column group cg).  MFMA k index 8 g2 + 4 r + j of key
    // step kh holds key 16 kh + 8 r + 4 g2 + j (the order in which the score
    // accumulators hold a lane's keys), so source lane s of the group points
    // at key 16 kh + 8 r + 4 g2 + s/4 for read r (0, 1), columns
    // 16 cg + 4 (s%4) .. +3.
    const int G = lane >> 4, sl = lane & 15;
    const int g2 = G >> 1, cg = G & 1;
    const int par = (sl >> 1) & 1;  // chunk parity of the source columns
    const int pv_base = cg * 1024 + par * 512 + (sl & 1) * 8;
    const int swz = kSwzA * par ^ kSwzB * cg;
    pv_off0 = pv_base + (((4 * g2 + (sl >> 2)) ^ swz) * 16);
    pv_off1 = pv_base + (((8 + 4 * g2 + (sl >> 2)) ^ swz) * 16);
    if constexpr (kH16) {
      // 16 head slots on v_mfma_f32_16x16x32_bf16 (lane l: slot l%16, lane
      // group G = l/16).  Score operand of k-step ks (32 columns) and key
      // half kh: key 16 kh + l%16, 8-column chunk dc = 4 ks + G, so the
      // swizzle depends on G only and the k-step adds ks * 2048.
      const int swz16 = kSwzA * (G & 1) ^ kSwzB * (G >> 1);
      const int kb = (G >> 1) * 1024 + (G & 1) * 512;
      k16_off0 = kb + (((sl) ^ swz16) * 16);
      k16_off1 = kb + (((16 + sl) ^ swz16) * 16);
      // P . V operand of 16-column block cb through the 16-lane transposing
      // read: source lane s points at key 16 r + 4 G + s/4, columns
      // 16 cb + 4 (s%4) .. +3 (chunk 2 cb + par, byte 8 (s%2) in it); read
      // r = 1 is 256 bytes on, the block cb * 1024 on, and the chunk
      // swizzle differs between even and odd blocks.
      const int vb = par * 512 + (sl & 1) * 8;
      v16_off_e = vb + ((((4 * G + (sl >> 2)) ^ (kSwzA * par))) * 16);
      v16_off_o = vb + ((((4 * G + (sl >> 2)) ^ (kSwzA * par) ^ kSwzB)) * 16);
    }
  }

  __device__ __forceinline__ char* pbuf(int t) const { return smem + kPOff + (t & 1) * kPBufBytes; }
  __device__ __forceinline__ const char* stage(int t) const {
    return smem + (t % kNStages) * kCkvBytes;
  }
  __device__ __forceinline__ const char* kpe_slot(int t) const {
    return smem + kKpeO + (t % kNKpe) * kKpeBytes;
  }

  // Entry i of the item's page list in LDS (as a VGPR value; the caller
  // makes it uniform where it uses it).  LDS reads keep the compiler's
  // lgkmcnt waits exact, where a scalar load in flight would make every LDS
  // wait a full drain.
  __device__ __forceinline__ int page_at(int i) const {
    return reinterpret_cast<const int*>(smem + kPageOff)[i];
  }

  // Tiles that may span pages: the page id of key k (0 .. 31) of tile t sits
  // in this wave's LDS ring at slot t % kIdSlots.  stage_ids(t) DMAs them
  // there (lanes 0 .. 31, one 4-byte id each; keys past the item's end take
  // its last key's page); the wave reads them kIdAhead tiles later.
  __device__ __forceinline__ uint32_t id_slot_addr(int t) const {
    return lds_base + kPageOff + wave * kIdWaveBytes + (t % kIdSlots) * (kTileKeys * 4);
  }
  // One 4-byte-per-lane DMA: lane i's word lands at LDS dst + 4 i.
  __device__ __forceinline__ static void dma4(const int32_t* src, uint32_t dst) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(src), "s"(__builtin_amdgcn_readfirstlane(dst))
                 : "m0");
  }
  __device__ __forceinline__ void stage_ids(int t) const {
    const int lane = opaque(this->lane);  // (address arithmetic made here, per tile)
    if (lane < kTileKeys) {
      const int P = a.page_size;
      const int key = min(kv_begin + t * kTileKeys + lane, kv_end - 1);
      dma4(a.kv_indices + page_base + (P == 1 ? key : key / P), id_slot_addr(t));
    }
  }
  // The item's page list (tiles that never span pages): entry i of its n
  // pages at LDS kPageOff + 4 i, by DMA (lanes past the end re-read entry
  // n-1).
  __device__ __forceinline__ void stage_pages(int n) const {
    // (opaque: the addresses are made per item, not hoisted out of the item
    // loop into registers the key loop needs)
    const int lane = opaque(this->lane);
#pragma unroll
    for (int k = 0; k < kPageLoads; ++k) {
      const int i0 = (k * NW + wave) * kWave;  // this wave's first entry
      if (i0 < n)
        dma4(a.kv_indices + page_base + first_page + min(i0 + lane, n - 1),
             lds_base + kPageOff + i0 * 4);
    }
  }
  __device__ __forceinline__ int lane_page(int t, int k) const {
    const int* ring = reinterpret_cast<const int*>(smem + kPageOff + wave * kIdWaveBytes +
                                                   (t % kIdSlots) * (kTileKeys * 4));
    return ring[k];
  }

  // Query staging.  Wave w's 32 heads (32 w .. 32 w + 31; heads past H
  // take head 0's row) land at LDS offset w * kQWaveBytes: the q_nope row of
  // head r at r * 1024, its q_pe row at 32 KiB + r * 128.  One DMA moves a
  // whole q_nope row (64 lanes x 16 bytes) or eight whole q_pe rows, so each
  // load reads full cache lines.  Within a row the 16-byte pieces are
  // permuted (slot c holds piece c ^ (r % 16), q_pe: c ^ (r % 8)) so that
  // the operand reads below, one head per lane, fall in distinct banks.
  static_assert(NW * kQWaveBytes <= kPageOff, "the query fits below the page list");
  __device__ __forceinline__ void stage_query(int H) const {
    const char* qn = reinterpret_cast<const char*>(a.q_nope + static_cast<int64_t>(token) * H * kLoraRank);
    const char* qp = reinterpret_cast<const char*>(a.q_pe + static_cast<int64_t>(token) * H * kRopeDim);
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_base + wave * kQWaveBytes);
    // (opaque: computed per item, not kept in 36 registers for the kernel)
    const int lane = opaque(this->lane);
    static_for<32>([&](auto jc) {  // q_nope rows
      constexpr int r = decltype(jc)::value;
      const int h = wave * 32 + r;
      const uint32_t voff = (h < H ? h : 0) * (kLoraRank * 2) + ((lane ^ (r % 16)) * 16);
      dma16s<0, r * 1024>(voff, qn, dst);
    });
    static_for<4>([&](auto jc) {  // 8 q_pe rows each
      constexpr int j = decltype(jc)::value;
      const int r = 8 * j + (lane >> 3);
      const int h = wave * 32 + r;
      const uint32_t voff = (h < H ? h : 0) * (kRopeDim * 2) + (((lane & 7) ^ (r % 8)) * 16);
      dma16s<0, 32768 + j * 1024>(voff, qp, dst);
    });
  }
  // One-wave kernels load the query rows straight into the MFMA operand
  // registers instead: q[ks] of lane (l32, half) is dims 16 ks + 8 half ..
  // +8 of head l32 (q_nope for ks < 32, q_pe after), sixteen bytes per load.
  // (With several waves the scattered loads cost the CU's address path more
  // than LDS staging does.)
  __device__ __forceinline__ void load_query(int H, u32x4_t (&q)[kQSteps]) const {
    const int lane = opaque(this->lane);  // (addresses made per item)
    const int l32 = lane & 31, half = lane >> 5;
    const int h0 = wave * 32 + l32;
    const int64_t h = static_cast<int64_t>(token) * H + (h0 < H ? h0 : 0);
    const u32x4_t* qn = reinterpret_cast<const u32x4_t*>(a.q_nope + h * kLoraRank) + half;
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(a.q_pe + h * kRopeDim) + half;
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks)
      q[ks] = ks < kLoraRank / 16 ? qn[2 * ks] : qp[2 * (ks - kLoraRank / 16)];
  }
  // LDS offset of this lane's query operand for k-step ks.
  __device__ __forceinline__ int query_lds_off(int ks, int lane) const {
    const int l32 = lane & 31, half = lane >> 5;
    if (ks < kLoraRank / 16)
      return wave * kQWaveBytes + l32 * 1024 + (((2 * ks + half) ^ (l32 % 16)) * 16);
    const int kp = ks - kLoraRank / 16;
    return wave * kQWaveBytes + 32768 + l32 * 128 + (((2 * kp + half) ^ (l32 % 8)) * 16);
  }

  // One 16-byte-per-lane DMA from global memory into LDS at
  // m0 + offset + 16 * lane, with m0 = lds_base + kM0 (lds_base uniform, in
  // an SGPR since the tile's set-up): lane row address (64-bit VGPR pair,
  // `off` form) or a uniform base (SGPR pair) plus a 32-bit lane offset,
  // each with a constant byte offset.  Issued through asm so that the
  // compiler, which cannot tell the stages apart, does not make later LDS
  // reads wait for every DMA; the tile pipeline waits on vmcnt itself.  One
  // wait state separates the M0 write from the DMA.  The stage it writes is
  // not read before the next barrier.  Nothing here should wait on a VALU
  // result (the readfirstlane is a copy once lds_base is in an SGPR): such a
  // chain in front of each DMA stalls the in-order wave.
  template <int kOff, int kM0>
  __device__ __forceinline__ static void dma16(const char* src, uint32_t lds_base) {
    asm volatile("s_add_u32 m0, %1, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%3"
                 :
                 : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base)), "i"(kM0), "i"(kOff)
                 : "m0", "scc");
  }
  template <int kOff, int kM0>
  __device__ __forceinline__ static void dma16s(uint32_t voff, const char* sbase, uint32_t lds_base) {
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%4"
                 :
                 : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base)), "i"(kM0),
                   "i"(kOff)
                 : "m0", "scc");
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
    uint32_t voff_o;    //   (several waves: voff_e is this wave's, of its parity)
    uint32_t dst;       // LDS address of DMA I = wave (ckv stage) ...
    uint32_t dst2;      // ... and of I = wave + 32 (kpe slot), less 32 KiB
  };

  // Tile t of the item.  When tiles never span pages, its keys are rows
  // inp .. inp+31 of page pg (the caller steps through the page list, so
  // no division by the page size happens per tile).
  __device__ __forceinline__ TileDma prep_tile(int t, int pg, int inp) const {
    const int base = kv_begin + t * kTileKeys;
    TileDma d;
    if constexpr (kFp8) {
      // Lane l fetches key l%32 (the last key of the item past its end):
      // ckv chunk pair j is at row offset wave * 512/NW + 16 (l/32) + 32 j,
      // kpe chunk k (lanes 0..31) at 512 + 16 (kKpeLoads wave + k).
      d.dst = __builtin_amdgcn_readfirstlane(lds_base + kRawOff + (t % kRawSlots) * kRawSlotBytes +
                                             wave * kRawWaveBytes);
      d.dst2 = d.dst;
      asm volatile("" : "+s"(d.dst));
      // (opaque: per-tile address arithmetic stays here instead of being
      // hoisted out of the item loop into registers the key loop needs)
      const int key = min(opaque(l32), kv_end - 1 - base);
      const int ckv_off = half * 16 + wave * (kLoraRank / NW);
      const int kpe_off = kLoraRank + wave * kKpeLoads * 16;
      if (kTileInPage) {
        d.sbase = reinterpret_cast<const char*>(
            a.kv_cache8 + static_cast<int64_t>(pg * a.page_size + inp) * kLatentDim);
        d.voff_e = static_cast<uint32_t>(key * kLatentDim + ckv_off);
        d.voff_o = static_cast<uint32_t>(key * kLatentDim + kpe_off);
        d.src_e = d.src_o = nullptr;
      } else {
        const int P = a.page_size;
        const int pgk = lane_page(t, key);
        const int r = P == 1 ? pgk : pgk * P + (base + key) % P;
        const char* row = reinterpret_cast<const char*>(a.kv_cache8 + static_cast<int64_t>(r) * kLatentDim);
        d.src_e = row + ckv_off;
        d.src_o = nullptr;  // (kpe addresses are made from src_e when issued)
        d.sbase = nullptr;
        d.voff_e = d.voff_o = 0;
      }
      return d;
    }
    // (uniform: pinned to SGPRs here, or the compiler sinks a readfirstlane
    // in front of every DMA)
    d.dst = __builtin_amdgcn_readfirstlane(lds_base + (t % kNStages) * kCkvBytes + wave * 1024);
    d.dst2 = __builtin_amdgcn_readfirstlane(lds_base + kKpeO + (t % kNKpe) * kKpeBytes +
                                            wave * 1024 - kCkvBytes);
    asm volatile("" : "+s"(d.dst), "+s"(d.dst2));
    if (kTileInPage) {
      const int rem = kv_end - 1 - base;  // keys past the item's end re-read its last key
      const int lane_c = ld_off + wave * 32;
      d.sbase = reinterpret_cast<const char*>(
          a.kv_cache + static_cast<int64_t>(pg * a.page_size + inp) * kLatentDim);
      // With several waves each wave loads one of the two key orders only
      // (selected here, once per tile: a select in front of each DMA puts
      // a VALU result on the DMA's address path).
      const int key_e = NW == 1 || (wave & 1) == 0 ? ld_key : (ld_key ^ kSwzB);
      d.voff_e = static_cast<uint32_t>(min(key_e, rem) * (kLatentDim * 2) + lane_c);
      d.voff_o = NW == 1 ? static_cast<uint32_t>(min(ld_key ^ kSwzB, rem) * (kLatentDim * 2) + lane_c)
                         : d.voff_e;
      d.src_e = d.src_o = nullptr;
    } else {
      const int P = a.page_size;
      const int rem = kv_end - 1 - base;  // keys past the item's end re-read its last key
      auto row_src = [&](int key) {
        const int k = min(key, rem);
        const int pg = lane_page(t, k);
        const int r = P == 1 ? pg : pg * P + (base + k) % P;
        return reinterpret_cast<const char*>(a.kv_cache + static_cast<int64_t>(r) * kLatentDim) +
               ld_off + wave * 32;
      };
      // With several waves each wave loads one of the two key orders only
      // (chosen here: a select between the two in front of every DMA ends
      // up as a load from the stack).
      if (NW == 1) {
        d.src_e = row_src(ld_key);
        d.src_o = row_src(ld_key ^ kSwzB);
      } else {
        d.src_e = d.src_o = row_src((wave & 1) ? (ld_key ^ kSwzB) : ld_key);
      }
      d.sbase = nullptr;
      d.voff_e = d.voff_o = 0;
    }
    return d;
  }

  // DMA instruction I = wave + j NW of this wave for a tile.  With an even
  // number of waves I has the wave's parity; with one wave, j's.
  template <int j>
  __device__ __forceinline__ void issue_one(const TileDma& d) const {
    if constexpr (kFp8) {
      if constexpr (j < kCkvLoads) {  // 1 KiB: two ckv chunks of 32 keys
        constexpr int kOff = 32 * j;
        constexpr int kM0 = 1024 * j - kOff;
        if (kTileInPage)
          dma16s<kOff, kM0>(d.voff_e, d.sbase, d.dst);
        else
          dma16<kOff, kM0>(d.src_e, d.dst);
      } else {  // 512 B, lanes 0..31: one kpe chunk of 32 keys
        constexpr int k = j - kCkvLoads;
        constexpr int kOff = 16 * k;
        constexpr int kM0 = 1024 * kCkvLoads + 512 * k - kOff;
        if (lane < 32) {
          if (kTileInPage) {
            dma16s<kOff, kM0>(d.voff_o, d.sbase, d.dst);
          } else {
            // lanes 0..31 (first half): from this wave's ckv offset to its kpe one
            const int delta = __builtin_amdgcn_readfirstlane(kLoraRank + wave * kKpeLoads * 16 -
                                                             wave * (kLoraRank / NW));
            dma16<kOff, kM0>(d.src_e + delta, d.dst);
          }
        }
      }
      return;
    }
    constexpr int kOff = j * NW * 32;
    // The instruction offset moves the LDS destination as well as the
    // global address, so M0 takes it back off.
    constexpr int kM0 = j * NW * 1024 - kOff;
    const uint32_t dbase = j * NW < kCkvDmas ? d.dst : d.dst2;
    if (kTileInPage)
      dma16s<kOff, kM0>(NW == 1 && (j & 1) ? d.voff_o : d.voff_e, d.sbase, dbase);
    else
      dma16<kOff, kM0>(NW == 1 && (j & 1) ? d.src_o : d.src_e, dbase);
  }

  template <int j0, int j1>
  __device__ __forceinline__ void issue_range(const TileDma& d) const {
    if constexpr (j0 < j1) {
      issue_one<j0>(d);
      issue_range<j0 + 1, j1>(d);
    }
  }

  // fp8 cache: this wave's codes of tile t (its raw slice) converted to
  // bf16 into stage t and kpe slot t, at the places the score and P . V
  // reads expect (16-column chunk c of key k becomes the 8-column chunks
  // 2c and 2c+1).  Exact: every E4M3 value is a bf16 value.
  __device__ __forceinline__ void convert_tile(int t) const {
    const char* raw = smem + kRawOff + (t % kRawSlots) * kRawSlotBytes + wave * kRawWaveBytes +
                      lane * 16;
    char* stg = smem + (t % kNStages) * kCkvBytes;
    char* kp = smem + kKpeO + (t % kNKpe) * kKpeBytes;
    auto cvt = [](uint32_t w0, uint32_t w1) {
      u32x4_t o;
      o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
      o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
      o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
      o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
      return o;
    };
    // (two chunks in flight: the scheduler may not hoist every read, the
    // key loop's registers are nearly all taken)
    constexpr int kAhead = 2;
    u32x4_t r[kAhead];
#pragma unroll
    for (int j = 0; j < kAhead && j < kCkvLoads; ++j)
      r[j] = *reinterpret_cast<const u32x4_t*>(raw + j * 1024);
    static_for<kCkvLoads>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const u32x4_t cur = r[j % kAhead];
      if constexpr (j + kAhead < kCkvLoads)
        r[j % kAhead] = *reinterpret_cast<const u32x4_t*>(raw + (j + kAhead) * 1024);
      const int c = (32 / NW) * wave + 2 * j + half;  // 16-column chunk of the key
      const int sw = kSwzB * (c & 1);
      char* dst = stg + c * 1024;
      *reinterpret_cast<u32x4_t*>(dst + ((l32 ^ sw) * 16)) = cvt(cur[0], cur[1]);
      *reinterpret_cast<u32x4_t*>(dst + 512 + ((l32 ^ kSwzA ^ sw) * 16)) = cvt(cur[2], cur[3]);
      __builtin_amdgcn_sched_barrier(0);
    });
    if (lane < 32) {
#pragma unroll
      for (int k = 0; k < kKpeLoads; ++k) {
        const u32x4_t q = *reinterpret_cast<const u32x4_t*>(raw + kCkvLoads * 1024 + k * 512);
        const int kc = kKpeLoads * wave + k;  // kpe 16-column chunk
        const int sw = kSwzB * (kc & 1);
        char* dst = kp + kc * 1024;
        *reinterpret_cast<u32x4_t*>(dst + ((l32 ^ sw) * 16)) = cvt(q[0], q[1]);
        *reinterpret_cast<u32x4_t*>(dst + 512 + ((l32 ^ kSwzA ^ sw) * 16)) = cvt(q[2], q[3]);
      }
    }
  }

  __device__ __forceinline__ void issue_tile(int t, int pg, int inp) const {
    const TileDma d = prep_tile(t, pg, inp);
    issue_range<0, kLoadsPerWave>(d);
  }

  // Waits for this wave's DMAs except, if `later`, those issued in the
  // previous iteration: the newest tile's and, if `later_id`, one page-id
  // DMA.
  __device__ __forceinline__ static void wait_vm(bool later, bool later_id) {
    if (later && later_id) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadsPerWave + 1));
    else if (later) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadsPerWave));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }

  // The workgroup's start, read with one lane-parallel load: from the host
  // slot (fast_first) the first item with the worker's item range in two of
  // its fields (32 bytes, no shared pool there); otherwise the worker's item
  // range (lanes 8, 9) and the shared pool's (lanes 10, 11) from
  // worker_indptr.
  struct Entry {
    int f_token, f_begin, f_end, f_slot, f_base, f_pages;
    int w_begin, w_end, pool_begin, pool_n;
  };
  __device__ __forceinline__ Entry read_entry(bool fast_first) const {
    int v = 0;
    {
      const int l = opaque(lane);
      const int* src = nullptr;
      if (fast_first) {
        if (l < 8) src = reinterpret_cast<const int*>(a.first_items) + blockIdx.x * 8 + l;
      } else if (l == 8 || l == 9) {
        src = a.worker_indptr + blockIdx.x + (l - 8);
      } else if (l == 10 || l == 11) {
        src = a.worker_indptr + gridDim.x + (l - 10);
      }
      if (src) v = *src;
    }
    Entry e;
    e.f_token = __builtin_amdgcn_readlane(v, 0);
    e.f_begin = __builtin_amdgcn_readlane(v, 2);
    e.f_end = __builtin_amdgcn_readlane(v, 3);
    e.f_slot = __builtin_amdgcn_readlane(v, 4);
    e.f_base = __builtin_amdgcn_readlane(v, 5);
    e.f_pages = __builtin_amdgcn_readlane(v, 7);  // (pad[1]: the page list is staged)
    if (fast_first) {
      e.w_begin = __builtin_amdgcn_readlane(v, 1);  // (row field)
      e.w_end = __builtin_amdgcn_readlane(v, 6);    // (pad[0])
      e.pool_begin = 0;
      e.pool_n = 0;
    } else {
      e.w_begin = __builtin_amdgcn_readlane(v, 8);
      e.w_end = __builtin_amdgcn_readlane(v, 9);
      e.pool_begin = __builtin_amdgcn_readlane(v, 10);
      e.pool_n = __builtin_amdgcn_readlane(v, 11) - e.pool_begin;
    }
    return e;
  }

  __device__ void run() {
    static_assert(!kH16, "16 head slots run in the split kernel");
    // A schedule in the host slot: the first item is read straight from
    // first_items (no dependent worker_indptr read) and, where it was staged,
    // its page list goes out to LDS now, with that read still in flight.
    // The entry reads (first item, worker_indptr pair) go out together as
    // one lane-parallel load: lanes 0..7 the item's fields, lanes 8 and 9
    // this worker's item range, lanes 10 and 11 the shared pool's.
    const bool fast_first = kTileInPage && a.first_items != nullptr;
    if (fast_first && wave == 0 && lane < kFirstPages)
      dma4(a.first_pages + blockIdx.x * kFirstPages + lane, lds_base + kPageOff);
    const Entry e = read_entry(fast_first);
    const int H = a.num_heads;

    // The shared pool (a schedule with many query tokens): once its own
    // items are done, the workgroup takes pool items one at a time.  Wave 0
    // asks for the next one (an atomic on a device counter) before the
    // finish of the item ahead of it, whose output stores cover the atomic's
    // latency; the index reaches the other waves through LDS.  (The vector
    // memory counter completes in order, so an atomic issued any earlier
    // would hold up the key loop's DMA waits.)
    int popped = 0;  // wave 0, lane 0: the pool index for the next pool item
    auto pop = [&] {
      if (wave == 0 && lane == 0)
        popped = __hip_atomic_fetch_add(a.pool_ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    if (e.pool_n > 0 && e.w_begin == e.w_end) pop();

    for (int next = e.w_begin;;) {
      int it;
      if (next < e.w_end) {
        it = next++;
      } else {
        if (e.pool_n <= 0) break;
        // (the page-list area: no wave reads it until after the item's
        // first barrier, and its DMA is issued after that barrier)
        int* xfer = reinterpret_cast<int*>(smem + kPageOff);
        if (wave == 0 && lane == 0) *xfer = popped;
        lds_barrier();
        const int k = __builtin_amdgcn_readfirstlane(*xfer);
        if (k >= e.pool_n) break;
        it = e.pool_begin + k;
      }
      // (the first item of a host-slot schedule was read at entry)
      const bool pre = fast_first && it == e.w_begin;
      if (pre) {
        token = e.f_token;
        kv_begin = e.f_begin;
        kv_end = e.f_end;
        slot = e.f_slot;
        page_base = e.f_base;
      } else {
        const_i32_t* item = (const_i32_t*)(a.items) + it * 8;  // WorkItem fields
        token = item[0];
        kv_begin = item[2];
        kv_end = item[3];
        slot = item[4];
        page_base = item[5];  // kv_indptr[row]
      }
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
        // Every wave is done with the previous item's (or attempt's) LDS.
        // (An item without keys goes straight to its finish, whose 1/l
        // exchange slots the previous item's finish may still be reading.)
        lds_barrier();
        if (ntiles == 0) break;
        // This wave's query rows go through LDS (several waves): whole rows
        // per DMA, where loading them straight into the MFMA operand layout
        // would touch 32 rows per load (see stage_query).  The page ids go
        // out in the same wait, also by DMA: the item's page list (tiles
        // that never span pages) or the first tiles' per-key ids (tiles that
        // may).  A lone wave loads its query after the first tiles' DMAs
        // instead, so that their latencies overlap (its query staging would
        // cover the stages).
        constexpr bool kQueryDirect = NW == 1;
        if (!kQueryDirect) stage_query(H);
        int n_pages = 1;
        if (kTileInPage) {
          const int P = a.page_size;
          first_page = kv_begin / P;
          n_pages = (kv_end - 1) / P - first_page + 1;  // <= kMaxItemTiles
          if (!(pre && e.f_pages)) stage_pages(n_pages);  // (else DMA'd at entry)
        } else {
#pragma unroll
          for (int t = 0; t < kIdAhead; ++t)
            if (t < ntiles) stage_ids(t);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // (the LDS reads stay below)
        // Query as the B operand of the 32x32x16 score MFMAs: lane (l32,
        // half) holds head 32 wave + l32, dims 16 ks + 8 half .. +8.
        u32x4_t q[kQSteps];
        if (!kQueryDirect) {
          const int qlane = opaque(lane);
#pragma unroll
          for (int ks = 0; ks < kQSteps; ++ks)
            q[ks] = *reinterpret_cast<const u32x4_t*>(smem + query_lds_off(ks, qlane));
#pragma unroll
          for (int ks = 0; ks < kQSteps; ++ks) asm volatile("" : : "v"(q[ks]));
        }
        // Every wave has its query in registers (several waves), and the
        // page list is complete.
        lds_barrier();
        // Page-list cursor: entry and first row of the next tile to load.
        int cur_pl = 0, cur_inp = kTileInPage ? kv_begin % a.page_size : 0;
        auto advance = [&] {
          cur_inp += kTileKeys;
          if (cur_inp == a.page_size) {
            cur_inp = 0;
            ++cur_pl;
          }
        };
#pragma unroll
        for (int t = 0; t < kAhead; ++t)
          if (t < ntiles) {
            issue_tile(t, kTileInPage ? __builtin_amdgcn_readfirstlane(page_at(cur_pl)) : 0, cur_inp);
            if (kTileInPage) advance();
          }
        if (kQueryDirect) {
          // Waited for here, with the first tiles issued before it: a wait
          // the compiler placed at the first use inside the key loop would
          // drain the DMAs in flight at every tile.
          load_query(H, q);
#pragma unroll
          for (int ks = 0; ks < kQSteps; ++ks) asm volatile("" : : "v"(q[ks]));
        }
        // The next tile's page id, read a tile ahead.
        int pg_next = kTileInPage ? page_at(min(cur_pl, n_pages - 1)) : 0;
        if constexpr (kFp8) {
          // This wave's codes of tile 0 (tile 1's may still be in flight).
          wait_vm(ntiles > 1, false);
          convert_tile(0);
        }
        // Tile t: S(t), with the DMAs of tile t+2 between its k-steps; the
        // softmax of S(t); P(t) published in LDS; this wave's columns of
        // P(t) . V(t) for every head.  With several waves the tiles are
        // software-pipelined: P . V of tile t-1 runs after S(t), with the
        // softmax of S(t) placed between its MFMAs, and one barrier per tile
        // serves both (tile t has landed, P(t-1) is complete, every wave is
        // done with tile t-2's stage and tile t-1's kpe slot).  A lone wave
        // has no registers for that and keeps the unpipelined order with a
        // second barrier before P . V.
        constexpr bool kPipe = NW > 1;
        for (int t = 0; t < ntiles; ++t) {
          // (iteration t-1 staged the ids of tile t-1+kIdAhead, if any; the
          // prologue stages none after its tiles)
          // (tile t+1's DMAs, and a page-id DMA issued before them, may
          // still be in flight when two tiles are; with one, nothing newer)
          if (!kFp8)
            wait_vm(kAhead > 1 && t + 1 < ntiles,
                    kAhead > 1 && !kTileInPage && t > 0 && t + kIdAhead - 1 < ntiles);
          lds_barrier();
          const bool dma = t + kAhead < ntiles;
          const int base = kv_begin + t * kTileKeys;
          float x[16];
          PvOps pvo;  // operands of this wave's first P . V step (several waves)
          {
            TileDma d{};  // (defined on every path: a phi with undef would put it in VGPRs)
            auto prep = [&] {
              d = prep_tile(t + kAhead, kTileInPage ? __builtin_amdgcn_readfirstlane(pg_next) : 0,
                            cur_inp);
              if (kTileInPage) {
                advance();
                pg_next = page_at(min(cur_pl, n_pages - 1));
              } else if (t + kIdAhead < ntiles) {
                stage_ids(t + kIdAhead);
              }
            };
            // With several waves, the DMA set-up goes under the first
            // k-step's MFMA (a lone wave, with four times the DMAs, has no
            // registers to spare there).  The DMAs go under the other
            // k-steps.
            constexpr bool kPrepUnder = NW > 1;
            // (the DMA test at every k-step is a scalar compare and branch
            // on this wave-uniform value, re-read from an opaque SGPR copy:
            // a condition the compiler keeps live across the k-steps becomes
            // a lane mask, rebuilt by VALU instructions in front of each DMA)
            const int dma_s = __builtin_amdgcn_readfirstlane(dma ? 1 : 0);
            if (!kPrepUnder && dma_s) prep();
            auto extra = [&](auto kc) {
              constexpr int k = decltype(kc)::value;
              // The first P . V operands of tile t-1 (published before this
              // iteration's barrier) go out under the chain's last k-steps,
              // so the P . V chain starts without an LDS round trip.
              if constexpr (kPipe && k == kQSteps - 3) {
                if (t > 0) pv_load(stage(t - 1), pbuf(t - 1), pvo);
              }
              int dsv = __builtin_amdgcn_readfirstlane(dma_s);
              asm volatile("" : "+s"(dsv));
              if (!dsv) return;
              if constexpr (k == 0) {
                if (kPrepUnder) prep();
              } else {
                dma_step<k>(d);
              }
            };
            scores(stage(t), kpe_slot(t), q, x, extra);
          }
          bf16x8_t p[2];
          if (!kPipe || t == 0) {
            const float mx = softmax_max(x, base, m_seen);
            if (t == 0) {
              const float mh = fmaxf(mx, __shfl_xor(mx, 32));
              if (m_ref == -INFINITY) m_ref = mh;  // O is still zero
            }
            softmax_exp<0, 16>(x, -m_ref, l_run, p);
          } else {
            const float neg_ref = -m_ref;
            // The softmax goes under the P . V MFMAs one piece per MFMA
            // (a piece issued after an MFMA runs while that MFMA does; the
            // next MFMA waits for the pipe anyway): the maximum under the
            // first, then about one probability per MFMA.
            pv_run(stage(t - 1), pbuf(t - 1), o, pvo, [&](auto sc) {
              constexpr int st = decltype(sc)::value;
              constexpr int kN = 2 * kDimBlocks * NW - 1;  // P . V MFMAs after the first
              if constexpr (st == 0) {
                softmax_max(x, base, m_seen);
              } else {
                softmax_exp<(st - 1) * 16 / kN, st * 16 / kN>(x, neg_ref, l_run, p);
              }
            });
          }
          store_p(p, pbuf(t));
          if (!kPipe) {
            lds_barrier();
            pv(stage(t), pbuf(t), o, [&](auto) {});
          }
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (kFp8) {
            // Tile t+1 into the stage of tile t-1, whose columns of this wave
            // P . V has just finished with.  Its codes were DMA'd an
            // iteration ago; tile t+2's (and a page-id DMA issued before
            // them) may still be in flight.
            if (t + 1 < ntiles) {
              wait_vm(dma, !kTileInPage && t + kIdAhead < ntiles);
              convert_tile(t + 1);
            }
          }
        }
        if (kPipe) {
          lds_barrier();
          pv(stage(ntiles - 1), pbuf(ntiles - 1), o, [&](auto) {});
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
      if (e.pool_n > 0 && next >= e.w_end) pop();  // the next item comes from the pool
      finish(o, m_ref, l_run);
    }
    // Every read of the schedule (items, page lists) has been consumed by
    // every wave (a workgroup without items waits here for its entry DMA):
    // tell the host this workgroup is done with the slot.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (e.pool_n > 0 && wave == 0 && lane == 0) {
      // This workgroup has drawn past the pool's end; the last one to do so
      // leaves the counters at zero for the next run (every draw of every
      // workgroup has returned by then).
      const int d = __hip_atomic_fetch_add(a.pool_ctr + 1, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      if (d == static_cast<int>(gridDim.x) - 1) {
        __hip_atomic_store(a.pool_ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.pool_ctr + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (a.done_flags && wave == 0 && lane == 0)
      __hip_atomic_store(a.done_flags + blockIdx.x, a.run_seq, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_SYSTEM);
  }

  // fp8 cache with at most 32 heads, or bf16 cache with at most 16: two
  // waves per workgroup.  Wave 0 computes (scores, softmax, P . V and the
  // finish of the compact one-wave kernel over its two bf16 stages); wave 1,
  // on a SIMD the compact kernel leaves idle, produces: it loads each tile's
  // rows into its registers two tiles ahead and writes them into the bf16
  // stage and kpe slot layout the computing wave reads (E4M3 codes
  // converted, exactly; bf16 rows copied).  One barrier per tile: behind it
  // the producer has filled tile t+1 into the stage the computing wave
  // finished with in tile t-1.  Used with the compact bf16 kernel's LDS
  // layout and launched with 128 threads.
  template <bool kCodes>
  __device__ void run_split() {
    static_assert(NW == 1 && kCompact && !kFp8, "the split kernel uses the compact bf16 layout");
    // (one loop per role, so that neither carries the other's registers)
    if (wave == 1)
      split_loop<true, kCodes>();
    else
      split_loop<false, kCodes>();
  }
  // kCodes: the cache holds fp8 codes (converted by the producer); else bf16
  // rows, which the producer copies.
  template <bool producer, bool kCodes>
  __device__ __forceinline__ void split_loop() {
    const bool fast_first = kTileInPage && a.first_items != nullptr;
    if (fast_first && producer && lane < kFirstPages)
      dma4(a.first_pages + blockIdx.x * kFirstPages + lane, lds_base + kPageOff);
    const Entry e = read_entry(fast_first);
    const int H = a.num_heads;

    // (the shared pool as in run(): the computing wave draws, through LDS)
    int popped = 0;
    auto pop = [&] {
      if (wave == 0 && lane == 0)
        popped = __hip_atomic_fetch_add(a.pool_ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    if (e.pool_n > 0 && e.w_begin == e.w_end) pop();

    // Producer: which 16-byte pieces of a tile's rows a lane moves.  bf16
    // rows go as whole 128-byte lines, eight keys per load, with
    // non-temporal loads (each row is read once): load j (key group kg =
    // j / 9, column group g = j % 9) gives lane L chunk 8 g + cx of key
    // 8 kg + (L & 7), where cx spreads each 16-lane group over two chunks
    // whose LDS swizzles differ, so that the copy into LDS has no bank
    // conflict.  (Non-temporal loads of 32-byte pieces, 32 rows per load,
    // would fetch every line once per piece.)  fp8 rows (576 bytes, not
    // line-aligned) go as before: lane (l32, half) takes 16-column chunks
    // 2 j + half of key l32, converted into two 8-column chunks.
    constexpr int kRawLoads = kCodes ? kLatentDim / 32 : kLatentDim / 16;  // 18 or 36 per lane
    // (lane constants made again in each call, through opaque(): hoisted
    // out of the tile loop they would hold registers the tiles need)
    auto lane_key = [&] { return opaque(lane) & 7; };
    auto lane_chunk = [&] {
      const int ln = opaque(lane);
      return 2 * ((ln >> 3) & 1) + ((ln >> 4) & 1) + 4 * (ln >> 5);
    };
    typedef u32x4_t RawTile[kRawLoads];
    auto raw_load = [&](int t, int pg, RawTile& r) {
      const int base = kv_begin + t * kTileKeys;
      const int rem = kv_end - 1 - base;  // keys past the item's end re-read its last key
      const int P = a.page_size;
      if constexpr (kCodes) {
        const int key = min(kv_begin + t * kTileKeys + opaque(l32), kv_end - 1);
        int64_t row;
        if (kTileInPage) {
          row = static_cast<int64_t>(pg) * P + key % P;
        } else {
          const int p = a.kv_indices[page_base + (P == 1 ? key : key / P)];
          row = P == 1 ? p : static_cast<int64_t>(p) * P + key % P;
        }
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.kv_cache8 + row * kLatentDim) + half;
#pragma unroll
        for (int j = 0; j < kRawLoads; ++j) r[j] = src[2 * j];
        return;
      }
      constexpr int kRowBytes = 2 * kLatentDim;
      const int rk = lane_key(), rc = lane_chunk();
      const char* cache = reinterpret_cast<const char*>(a.kv_cache);
      if (kTileInPage) {
        // (the tile stays in page pg: a uniform base and 32-bit lane offsets)
        const char* sb = cache + (static_cast<int64_t>(pg) * P + base % P) * kRowBytes;
        uint32_t off[4];
#pragma unroll
        for (int kg = 0; kg < 4; ++kg)
          off[kg] = static_cast<uint32_t>(min(kg * 8 + rk, rem) * kRowBytes + rc * 16);
#pragma unroll
        for (int j = 0; j < kRawLoads; ++j)
          r[j] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4_t*>(sb + off[j / 9] + (j % 9) * 128));
      } else {
        // (cache rows are below 2^31: the planner rejects larger caches)
        int rows[4];
#pragma unroll
        for (int kg = 0; kg < 4; ++kg) {
          const int key = base + min(kg * 8 + rk, rem);
          const int p = a.kv_indices[page_base + (P == 1 ? key : key / P)];
          rows[kg] = P == 1 ? p : p * P + key % P;
        }
#pragma unroll
        for (int j = 0; j < kRawLoads; ++j)
          r[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
              cache + static_cast<int64_t>(static_cast<uint32_t>(rows[j / 9])) * kRowBytes + rc * 16 +
              (j % 9) * 128));
      }
    };
    auto raw_store = [&](int t, const RawTile& r) {
      char* stg = smem + (t % kNStages) * kCkvBytes;
      char* kp = smem + kKpeO + (t % kNKpe) * kKpeBytes;
      if constexpr (!kCodes) {
        // chunk dc of key kk, where the DMA loader places it
        const int rk = lane_key(), rc = lane_chunk();
#pragma unroll
        for (int j = 0; j < kRawLoads; ++j) {
          const int kk = (j / 9) * 8 + rk, dc = 8 * (j % 9) + rc, blk = dc >> 1, hf = dc & 1;
          char* dst = (blk < kCkvDmas ? stg + blk * 1024 : kp + (blk - kCkvDmas) * 1024) + hf * 512;
          *reinterpret_cast<u32x4_t*>(dst + ((kk ^ (kSwzA * hf) ^ (kSwzB * (blk & 1))) * 16)) = r[j];
        }
        return;
      }
#pragma unroll
      for (int j = 0; j < kRawLoads; ++j) {
        const int c = 2 * j + half;  // 16-column chunk of the lane's key
        const int cc = j < kCkvDmas / 2 ? c : c - kCkvDmas;
        const int sw = kSwzB * (cc & 1);
        char* dst = (j < kCkvDmas / 2 ? stg : kp) + cc * 1024;
        *reinterpret_cast<u32x4_t*>(dst + ((l32 ^ sw) * 16)) = cvt_fp8x8(r[j][0], r[j][1]);
        *reinterpret_cast<u32x4_t*>(dst + 512 + ((l32 ^ kSwzA ^ sw) * 16)) = cvt_fp8x8(r[j][2], r[j][3]);
      }
    };

    for (int next = e.w_begin;;) {
      int it;
      if (next < e.w_end) {
        it = next++;
      } else {
        if (e.pool_n <= 0) break;
        int* xfer = reinterpret_cast<int*>(smem + kPageOff);
        if (wave == 0 && lane == 0) *xfer = popped;
        lds_barrier();
        const int k = __builtin_amdgcn_readfirstlane(*xfer);
        if (k >= e.pool_n) break;
        it = e.pool_begin + k;
      }
      const bool pre = fast_first && it == e.w_begin;
      if (pre) {
        token = e.f_token;
        kv_begin = e.f_begin;
        kv_end = e.f_end;
        slot = e.f_slot;
        page_base = e.f_base;
      } else {
        const_i32_t* item = (const_i32_t*)(a.items) + it * 8;
        token = item[0];
        kv_begin = item[2];
        kv_end = item[3];
        slot = item[4];
        page_base = item[5];
      }
      const int ntiles = (kv_end - kv_begin + kTileKeys - 1) / kTileKeys;

      f32x16_t o[NW][kDimBlocks];
      f32x4_t o16[32];  // (16 head slots)
      float m_ref = -INFINITY, m_seen = -INFINITY, l_run = 0.f;
      for (;;) {
        if constexpr (!producer && kH16) {
#pragma unroll
          for (int cb = 0; cb < 32; ++cb) o16[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        } else if constexpr (!producer) {
#pragma unroll
          for (int db = 0; db < kDimBlocks; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) o[0][db][j] = 0.f;
        }
        l_run = 0.f;
        m_seen = -INFINITY;
        lds_barrier();  // (both waves are done with the previous item's LDS)
        if (ntiles == 0) break;
        if constexpr (producer) {
          RawTile ra, rb;
          int n_pages = 1;
          if (kTileInPage) {
            const int P = a.page_size;
            first_page = kv_begin / P;
            n_pages = (kv_end - 1) / P - first_page + 1;
            if (!(pre && e.f_pages)) {
              const int ln = opaque(lane);
#pragma unroll
              for (int k = 0; k < kPageLoads; ++k) {
                const int i0 = k * kWave;
                if (i0 < n_pages)
                  dma4(a.kv_indices + page_base + first_page + min(i0 + ln, n_pages - 1),
                       lds_base + kPageOff + i0 * 4);
              }
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          }
          auto tile_page = [&](int t) {
            return kTileInPage ? __builtin_amdgcn_readfirstlane(
                                     page_at((kv_begin + t * kTileKeys) / a.page_size - first_page))
                               : 0;
          };
          // Two register tiles alternate (even tiles in ra, odd in rb), so
          // that no copy waits for loads in flight; one barrier per tile.
          raw_load(0, tile_page(0), ra);
          if (ntiles > 1) raw_load(1, tile_page(1), rb);
          raw_store(0, ra);
          lds_barrier();  // tile 0 is in stage 0
          for (int t = 0; t < ntiles; t += 2) {
            if (t + 2 < ntiles) raw_load(t + 2, tile_page(t + 2), ra);
            if (t + 1 < ntiles) raw_store(t + 1, rb);
            lds_barrier();  // (the computing wave has finished tile t)
            if (t + 1 >= ntiles) break;
            if (t + 3 < ntiles) raw_load(t + 3, tile_page(t + 3), rb);
            if (t + 2 < ntiles) raw_store(t + 2, ra);
            lds_barrier();  // (... and tile t+1)
          }
        } else if constexpr (kH16) {
          u32x4_t q16[kQ16];
          load_query16(H, q16);
#pragma unroll
          for (int ks = 0; ks < kQ16; ++ks) asm volatile("" : : "v"(q16[ks]));
          lds_barrier();  // tile 0 is in stage 0
          for (int t = 0; t < ntiles; ++t) {
            const int base = kv_begin + t * kTileKeys;
            f32x4_t acc16[2];
            scores16(stage(t), kpe_slot(t), q16, acc16, [&](auto) {});
            float x8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) x8[j] = acc16[j >> 2][j & 3];
            const float mx = softmax16_max(x8, base, m_seen);
            if (t == 0) {
              const float mh = slot_max16(mx);
              if (m_ref == -INFINITY) m_ref = mh;  // O is still zero
            }
            bf16x8_t p16;
            softmax16_exp(x8, -m_ref, l_run, p16);
            pv16(stage(t), p16, o16);
            lds_barrier();  // (tile t's stage is free; tile t+1 is in the other)
          }
        } else {
          u32x4_t q[kQSteps];
          load_query(H, q);
#pragma unroll
          for (int ks = 0; ks < kQSteps; ++ks) asm volatile("" : : "v"(q[ks]));
          lds_barrier();  // tile 0 is in stage 0
          for (int t = 0; t < ntiles; ++t) {
            const int base = kv_begin + t * kTileKeys;
            float x[16];
            scores(stage(t), kpe_slot(t), q, x, [&](auto) {});
            bf16x8_t p[2];
            const float mx = softmax_max(x, base, m_seen);
            if (t == 0) {
              const float mh = fmaxf(mx, __shfl_xor(mx, 32));
              if (m_ref == -INFINITY) m_ref = mh;  // O is still zero
            }
            softmax_exp<0, 16>(x, -m_ref, l_run, p);
            store_p(p, pbuf(t));
            pv(stage(t), pbuf(t), o, [&](auto) {});
            lds_barrier();  // (tile t's stage is free; tile t+1 is in the other)
          }
        }
        // Redo the item if a head overflowed its reference (decided by the
        // computing wave, read by both).
        int* flags = reinterpret_cast<int*>(smem + kFlagOff);
        if constexpr (!producer) {
          const bool redo = __any(m_seen > m_ref + kMaxExponent);
          if (lane == 0) flags[0] = redo ? 1 : 0;
        }
        lds_barrier();
        const int any_redo = __builtin_amdgcn_readfirstlane(flags[0]);
        if (!any_redo) break;
        m_ref = kH16 ? slot_max16(m_seen) : fmaxf(m_seen, __shfl_xor(m_seen, 32));
        lds_barrier();  // (the flag is read before the next attempt's barrier reuses the slot)
      }
      if (e.pool_n > 0 && next >= e.w_end) pop();
      if constexpr (producer) {
        if constexpr (!kH16) lds_barrier();  // (the one barrier of the finish; finish16 has none)
      } else if constexpr (kH16)
        finish16(o16, m_ref, l_run);
      else
        finish(o, m_ref, l_run);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (e.pool_n > 0 && wave == 0 && lane == 0) {
      const int d = __hip_atomic_fetch_add(a.pool_ctr + 1, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      if (d == static_cast<int>(gridDim.x) - 1) {
        __hip_atomic_store(a.pool_ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.pool_ctr + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (a.done_flags && wave == 0 && lane == 0)
      __hip_atomic_store(a.done_flags + blockIdx.x, a.run_seq, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_SYSTEM);
  }

  __device__ __forceinline__ void store_p(const bf16x8_t (&p)[2], char* pb) const {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      *reinterpret_cast<bf16x8_t*>(pb + wave * kPGroupBytes + ks * (kWave * 16) + lane * 16) = p[ks];
  }

  // The DMAs issued under k-step ks = 1 .. 35 of a score pass (k-step 0
  // prepares them), spread evenly.
  template <int ks>
  __device__ __forceinline__ void dma_step(const TileDma& d) const {
    static_assert(ks >= 1 && ks < kQSteps, "DMAs go under k-steps 1 .. 35");
    constexpr int kN = kQSteps - 1;
    issue_range<(ks - 1) * kLoadsPerWave / kN, ks * kLoadsPerWave / kN>(d);
  }

  // S^T of the tile in stage K / kpe slot Kpe (keys x this wave's 32
  // heads) as one chain of
  // 36 v_mfma_f32_32x32x16_bf16 over the 576 latent columns, K operands read
  // kAhead k-steps early; a later tile's DMAs go out between the k-steps.
  // On return x[4 i + j] is the score of key 8 i + 4 (lane/32) + j for head
  // lane%32: the accumulator layout, which the P . V step consumes as is.
  template <typename Extra>
  __device__ __forceinline__ void scores(const char* K, const char* Kpe, const u32x4_t (&q)[kQSteps],
                                         float (&x)[16], Extra&& extra) const {
    constexpr int kAhead = 3;
    const char* ke = K + qk_off_e;
    const char* ko = K + qk_off_o;
    const char* pe = Kpe + qk_off_e - kCkvBytes;
    const char* po = Kpe + qk_off_o - kCkvBytes;
    auto kload = [&](int ks) {  // k-steps 32 .. 35 (the kpe columns) from the kpe slot
      const char* b = ks < kCkvDmas ? (ks & 1 ? ko : ke) : (ks & 1 ? po : pe);
      return *reinterpret_cast<const bf16x8_t*>(b + ks * 1024);
    };
    f32x16_t acc;
    bf16x8_t kbuf[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) kbuf[i] = kload(i);
    static_for<kQSteps>([&](auto kc) {
      constexpr int ks = decltype(kc)::value;
      const bf16x8_t k0 = kbuf[ks % kAhead];  // (the asm operand is a VGPR)
      if constexpr (ks + kAhead < kQSteps) kbuf[ks % kAhead] = kload(ks + kAhead);
      if constexpr (ks == 0)
        mfma_v_first(acc, k0, q[ks]);
      else
        mfma_v(acc, k0, q[ks]);
      extra(kc);  // work placed under this k-step's MFMA
      // Keep each k-step's read kAhead steps ahead instead of letting the
      // scheduler hoist all 36 (they would not fit in registers).
      __builtin_amdgcn_sched_barrier(0);
    });
    mfma_settle(acc);
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = acc[j];
  }

  // Softmax of one tile's scores against the item's reference maximum,
  // p = 2^(s * scale_log2 - m_ref), in pieces that the pipeline spreads
  // between MFMAs.  x[4 i + j] is key 8 i + 4 half + j of the lane's head.
  //
  // softmax_max: keys past the item's end (last tile only) get score -inf;
  // returns the lane's largest scaled score and folds it into m_seen.
  __device__ __forceinline__ float softmax_max(float (&x)[16], int base, float& m_seen) const {
    if (__builtin_expect(base + kTileKeys > kv_end, 0)) {  // the item's last tile only
      // (made here from the lane id: kept for the kernel, it was spilled)
      const int h4 = 4 * (opaque(lane) >> 5);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = base + 8 * (j >> 2) + h4 + (j & 3);
        x[j] = key < kv_end ? x[j] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, x[j]);
    mx *= scale_log2;
    m_seen = fmaxf(m_seen, mx);
    return mx;
  }

  // softmax_exp: probabilities of x[j0 .. j1) as bf16 P^T operands
  // (p[kh][e] = x[8 kh + e]) and their sum.  No clamp against overflow: a
  // score more than 2^64 above the reference makes the item redo with a new
  // reference, so whatever an overflow leaves in the accumulators is
  // discarded.
  template <int j0, int j1>
  __device__ __forceinline__ void softmax_exp(const float (&x)[16], float neg_ref, float& l_run,
                                              bf16x8_t (&p)[2]) const {
#pragma unroll
    for (int j = j0; j < j1; ++j) {
      const float v = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], scale_log2, neg_ref));
      l_run += v;
      p[j >> 3][j & 7] = static_cast<__bf16>(v);
    }
  }

  // O^T += V^T . P^T for the tile in stage V with the probabilities of every
  // head slot in P buffer Pb: this wave's 32-column blocks
  // [w kDimBlocks, (w+1) kDimBlocks) times each head group's P^T.
  // Consecutive MFMAs go to different accumulators; V^T operands are read
  // kPvAhead column blocks early.  pv_load issues the first operand reads
  // (every head group's P^T for the first key half, the first V^T blocks),
  // which the caller may place earlier; pv_run is the MFMA chain, with
  // extra(i) placed under its i-th MFMA.
  static constexpr int kPvAhead = 2;
  struct PvOps {
    bf16x8_t pb[NW];
    bf16x8_t vbuf[kPvAhead];
  };
  __device__ __forceinline__ bf16x8_t pv_vload(const char* V, int st) const {
    // column block st % kDimBlocks, key half st / kDimBlocks
    const char* kv0 = V + pv_off0 + wave * kDimBlocks * 2048;
    const char* kv1 = V + pv_off1 + wave * kDimBlocks * 2048;
    const int off = (st % kDimBlocks) * 2048 + (st / kDimBlocks) * 256;
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(kv0 + off));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(kv1 + off));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
  __device__ __forceinline__ bf16x8_t pv_pload(const char* Pb, int g, int ks) const {
    return *reinterpret_cast<const bf16x8_t*>(Pb + g * kPGroupBytes + ks * (kWave * 16) + lane * 16);
  }
  __device__ __forceinline__ void pv_load(const char* V, const char* Pb, PvOps& ops) const {
#pragma unroll
    for (int g = 0; g < NW; ++g) ops.pb[g] = pv_pload(Pb, g, 0);
#pragma unroll
    for (int i = 0; i < kPvAhead; ++i) ops.vbuf[i] = pv_vload(V, i);
  }
  template <typename Extra>
  __device__ __forceinline__ void pv(const char* V, const char* Pb, f32x16_t (&o)[NW][kDimBlocks],
                                     Extra&& extra) const {
    PvOps ops;
    pv_load(V, Pb, ops);
    pv_run(V, Pb, o, ops, extra);
  }
  template <typename Extra>
  __device__ __forceinline__ void pv_run(const char* V, const char* Pb, f32x16_t (&o)[NW][kDimBlocks],
                                         PvOps& ops, Extra&& extra) const {
    constexpr int kSteps = 2 * kDimBlocks;  // (key half, column block)
    constexpr int kAhead = kPvAhead;
    bf16x8_t (&pb)[NW] = ops.pb;
    bf16x8_t (&vbuf)[kAhead] = ops.vbuf;
    auto vload = [&](int st) { return pv_vload(V, st); };
    auto pload = [&](int g, int ks) { return pv_pload(Pb, g, ks); };
    static_for<kSteps>([&](auto sc) {
      constexpr int st = decltype(sc)::value;
      bf16x8_t v = vbuf[st % kAhead];
      in_vgpr(v);  // (at the use: the asm waits for the load)
      if constexpr (st + kAhead < kSteps) vbuf[st % kAhead] = vload(st + kAhead);
      const int db = st % kDimBlocks;
      static_for<NW>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        bf16x8_t b = pb[g];
        in_vgpr(b);
        o[g][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, b, o[g][db], 0, 0, 0);
        // After its last use for the first key half, the group's operand
        // register takes the second half's (a pass of MFMAs ahead of use).
        if (st == kDimBlocks - 1) pb[g] = pload(g, 1);
        extra(std::integral_constant<int, st * NW + g>{});  // work under this MFMA
        __builtin_amdgcn_sched_barrier(0);
      });
    });
  }

  // Writes the item's result.  The accumulators are never touched by VALU
  // code here (that makes the compiler shuttle all 256 of them through
  // VGPRs).  Lane l holds, for head group g, head 32g + l%32 and columns
  // 32 (w kDimBlocks + db) + 8 (j/4) + 4 (l/32) + j%4.  The raw sums go
  // through this wave's LDS region head group by head group (stored straight
  // from the AGPRs); then each lane normalises 8 columns of one head (1/l of
  // the head, from its owner wave through LDS), converts them and stores 16
  // bytes.  The caller has made the LDS stages free.
  __device__ __forceinline__ void finish(f32x16_t (&o)[NW][kDimBlocks], float m_ref,
                                         float l_run) const {
    const int lane = opaque(this->lane);
    const int l32 = lane & 31, half = lane >> 5;
    const int head = wave * 32 + l32;
    const bool head_ok = head < a.num_heads;
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const bool any = l_tot > 0.f;
    const float inv = any ? a.out_scale / l_tot : 0.f;
    const float lse_v = any ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
    const int H = a.num_heads;
    // A final item writes the token's output and LSE; a piece of a split
    // token writes the same normalised bf16 rows and LSE to its slot.
    const int64_t row0 = static_cast<int64_t>(slot >= 0 ? slot : token) * H;
    uint16_t* dst_o = (slot >= 0 ? a.part_o : a.out) + row0 * kLoraRank + wave * kDimBlocks * 32;
    float* dst_lse = slot >= 0 ? a.part_lse + row0 : (a.lse ? a.lse + row0 : nullptr);
    float* X = reinterpret_cast<float*>(smem + kXchgOff);
    if (half == 0) X[head] = inv;
    if (dst_lse && head_ok && half == 0) dst_lse[head] = lse_v;
    lds_barrier();
    float* R = reinterpret_cast<float*>(smem + wave * kFinWaveBytes);
    // Read-back task of lane: head hb + kHStep r of the group, 8-column chunk cc.
    constexpr int kChunks = kDimBlocks * 4;  // 8-column chunks per head row (16, 32 or 64)
    constexpr int kHStep = kWave / kChunks;  // heads per read-back round
    constexpr int kRounds = 32 / kHStep;
    const int hb = lane / kChunks, cc = lane % kChunks;
    const float* rsrc = R + hb * kFinRow + cc * 8;
    const float* xsrc = X + hb;
    char* obase = reinterpret_cast<char*>(dst_o);
    const uint32_t ooff = static_cast<uint32_t>((hb * kLoraRank + cc * 8) * 2);
    // Padding head slots (H not a multiple of 32) are not stored.
    auto write_out = [&](auto masked_c) {
      constexpr bool kMasked = decltype(masked_c)::value;
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
        // Reads go out in batches ahead of the conversions and stores.
        constexpr int kBatch = kRounds < 8 ? kRounds : 8;
#pragma unroll
        for (int r0 = 0; r0 < kRounds; r0 += kBatch) {
          f32x4_t v0[kBatch], v1[kBatch];
          float sc[kBatch];
#pragma unroll
          for (int b = 0; b < kBatch; ++b) {
            const float* src = rsrc + kHStep * (r0 + b) * kFinRow;
            v0[b] = *reinterpret_cast<const f32x4_t*>(src);
            v1[b] = *reinterpret_cast<const f32x4_t*>(src + 4);
            sc[b] = xsrc[g * 32 + kHStep * (r0 + b)];
          }
#pragma unroll
          for (int b = 0; b < kBatch; ++b) {
            const int hrel = g * 32 + kHStep * (r0 + b);  // head of the task, less hb
            u32x4_t w;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const f32x2_t lo = {v0[b][2 * e] * sc[b], v0[b][2 * e + 1] * sc[b]};
              const f32x2_t hi = {v1[b][2 * e] * sc[b], v1[b][2 * e + 1] * sc[b]};
              w[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2_t));
              w[2 + e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2_t));
            }
            if (!kMasked || hb + hrel < H)
              *reinterpret_cast<u32x4_t*>(obase + (ooff + hrel * kLoraRank * 2)) = w;
          }
        }
      }
    };
    if (H >= NW * 32)
      write_out(std::false_type{});
    else
      write_out(std::true_type{});
  }

  // ---- At most 16 heads: one wave on v_mfma_f32_16x16x32_bf16 ----
  // With 32 head slots on the 32x32x16 MFMA, half of every MFMA of a 16-head
  // batch computed padding.  Here lane l holds head slot l%16 with lane
  // group G = l/16, every product is a 16x16x32 MFMA of the same rate per
  // flop, and the probabilities never leave the registers: the score
  // accumulators of the two key halves (kh) give lane l the keys
  // 16 kh + 4 G + j, which are the P^T operand of P . V once its k index
  // 8 G + 4 r + j stands for key 16 r + 4 G + j, and the transposing V^T
  // reads take their keys in that order.
  static constexpr int kQ16 = kLatentDim / 32;  // k-steps of 32 over 576

  // Query as the B operand: q[ks] of lane l is dims 32 ks + 8 G .. +8 of head
  // slot l%16 (q_nope for ks < 16, q_pe after); head slots beyond H load
  // head 0 and are never stored.
  __device__ __forceinline__ void load_query16(int H, u32x4_t (&q)[kQ16]) const {
    const int lane = opaque(this->lane);
    const int hs = lane & 15, G = lane >> 4;
    const int64_t h = static_cast<int64_t>(token) * H + (hs < H ? hs : 0);
    const u32x4_t* qn = reinterpret_cast<const u32x4_t*>(a.q_nope + h * kLoraRank) + G;
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(a.q_pe + h * kRopeDim) + G;
#pragma unroll
    for (int ks = 0; ks < kQ16; ++ks)
      q[ks] = ks < kLoraRank / 32 ? qn[4 * ks] : qp[4 * (ks - kLoraRank / 32)];
  }

  // S^T of the tile in stage K / kpe slot Kpe: MFMA i is k-step i/2, key half
  // i%2 (two accumulators, 36 MFMAs like the 32-slot chain, so the DMA
  // schedule placed by extra(i) is the same); K operands read 3 MFMAs ahead.
  // acc[kh][j] is the score of key 16 kh + 4 G + j for head slot l%16.
  template <typename Extra>
  __device__ __forceinline__ void scores16(const char* K, const char* Kpe,
                                           const u32x4_t (&q)[kQ16], f32x4_t (&acc)[2],
                                           Extra&& extra) const {
    constexpr int kAheadK = 3;
    const char* k0 = K + k16_off0;
    const char* k1 = K + k16_off1;
    const char* p0 = Kpe + k16_off0;
    const char* p1 = Kpe + k16_off1;
    auto kload = [&](int i) {
      const int ks = i >> 1, kh = i & 1;
      const char* b = ks < kLoraRank / 32 ? (kh ? k1 : k0) : (kh ? p1 : p0);
      return *reinterpret_cast<const bf16x8_t*>(
          b + (ks < kLoraRank / 32 ? ks : ks - kLoraRank / 32) * 2048);
    };
    bf16x8_t kbuf[kAheadK];
#pragma unroll
    for (int i = 0; i < kAheadK; ++i) kbuf[i] = kload(i);
    acc[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    static_for<2 * kQ16>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      bf16x8_t kv = kbuf[i % kAheadK];
      in_vgpr(kv);
      if constexpr (i + kAheadK < 2 * kQ16) kbuf[i % kAheadK] = kload(i + kAheadK);
      acc[i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          kv, __builtin_bit_cast(bf16x8_t, q[i >> 1]), acc[i & 1], 0, 0, 0);
      extra(ic);
      __builtin_amdgcn_sched_barrier(0);
    });
  }

  // Softmax of the lane's 8 scores (x[4 kh + j]: key 16 kh + 4 G + j), as
  // softmax_max / softmax_exp; the probabilities come out as the P^T operand.
  __device__ __forceinline__ float softmax16_max(float (&x)[8], int base, float& m_seen) const {
    if (__builtin_expect(base + kTileKeys > kv_end, 0)) {  // the item's last tile only
      const int g4 = 4 * (opaque(lane) >> 4);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = base + 16 * (j >> 2) + g4 + (j & 3);
        x[j] = key < kv_end ? x[j] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) mx = fmaxf(mx, x[j]);
    mx *= scale_log2;
    m_seen = fmaxf(m_seen, mx);
    return mx;
  }
  __device__ __forceinline__ void softmax16_exp(const float (&x)[8], float neg_ref, float& l_run,
                                                bf16x8_t& p) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], scale_log2, neg_ref));
      l_run += v;
      p[j] = static_cast<__bf16>(v);
    }
  }
  // The largest of a value over the four lanes of a head slot.
  __device__ __forceinline__ static float slot_max16(float v) {
    v = fmaxf(v, __shfl_xor(v, 16));
    return fmaxf(v, __shfl_xor(v, 32));
  }

  // O^T += V^T . P^T for the tile in stage V: 32 column blocks of 16, one
  // MFMA each (K = the tile's 32 keys), V^T read two blocks ahead.  o[cb][j]
  // of lane l is column 16 cb + 4 G + j of head slot l%16.
  __device__ __forceinline__ void pv16(const char* V, const bf16x8_t& p, f32x4_t (&o)[32]) const {
    constexpr int kAheadV = 2;
    const char* ve = V + v16_off_e;
    const char* vo = V + v16_off_o;
    auto vload = [&](int cb) {
      const char* b = (cb & 1 ? vo : ve) + cb * 1024;
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(b));
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(b + 256));
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8_t vbuf[kAheadV];
#pragma unroll
    for (int i = 0; i < kAheadV; ++i) vbuf[i] = vload(i);
    static_for<32>([&](auto cc) {
      constexpr int cb = decltype(cc)::value;
      bf16x8_t v = vbuf[cb % kAheadV];
      in_vgpr(v);
      if constexpr (cb + kAheadV < 32) vbuf[cb % kAheadV] = vload(cb + kAheadV);
      bf16x8_t b = p;
      in_vgpr(b);
      o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, b, o[cb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
  }

  // Writes the item's result (as finish): each lane stores its 4 columns of
  // every block, scaled by 1/l of its head slot, as 8 bytes of bf16.
  __device__ __forceinline__ void finish16(f32x4_t (&o)[32], float m_ref, float l_run) const {
    const int lane = opaque(this->lane);
    const int hs = lane & 15, G = lane >> 4;
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    const bool any = l_tot > 0.f;
    const float inv = any ? a.out_scale / l_tot : 0.f;
    const float lse_v = any ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
    const int H = a.num_heads;
    const int64_t row0 = static_cast<int64_t>(slot >= 0 ? slot : token) * H;
    float* dst_lse = slot >= 0 ? a.part_lse + row0 : (a.lse ? a.lse + row0 : nullptr);
    if (dst_lse && hs < H && G == 0) dst_lse[hs] = lse_v;
    if (hs >= H) return;
    uint16_t* dst = (slot >= 0 ? a.part_o : a.out) + (row0 + hs) * kLoraRank + 4 * G;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      const f32x2_t lo = {o[cb][0] * inv, o[cb][1] * inv};
      const f32x2_t hi = {o[cb][2] * inv, o[cb][3] * inv};
      const u32x2_t w = {__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2_t)),
                         __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2_t))};
      *reinterpret_cast<u32x2_t*>(dst + cb * 16) = w;
    }
  }
};

template <int NW, bool kTileInPage, bool kFp8, bool kCompact, bool kH16 = false>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attention_kernel(AttnArgs args) {
  __shared__ __attribute__((aligned(1024)))
  char smem[Attn<NW, kTileInPage, kFp8, kCompact, kH16>::kLdsBytes];
  Attn<NW, kTileInPage, kFp8, kCompact, kH16> k(args, smem);
  k.run();
}

// fp8 cache with at most 32 heads (kCodes) or bf16 cache with at most 16,
// two workgroups per compute unit: a computing and a producing wave per
// workgroup (Attn::run_split).
template <bool kTileInPage, bool kH16, bool kCodes>
__global__ __launch_bounds__(2 * kWave) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attention_split_kernel(AttnArgs args) {
  __shared__ __attribute__((aligned(1024)))
  char smem[Attn<1, kTileInPage, false, true, kH16>::kLdsBytes];
  Attn<1, kTileInPage, false, true, kH16> k(args, smem);
  k.template run_split<kCodes>();
}

template <int NW, bool kFp8, bool kCompact = false, bool kH16 = false>
hipError_t launch_nw(const AttnArgs& a, int num_workers, hipStream_t stream) {
  if (a.page_size % kTileKeys == 0)
    hipLaunchKernelGGL((attention_kernel<NW, true, kFp8, kCompact, kH16>), dim3(num_workers),
                       dim3(NW * kWave), 0, stream, a);
  else
    hipLaunchKernelGGL((attention_kernel<NW, false, kFp8, kCompact, kH16>), dim3(num_workers),
                       dim3(NW * kWave), 0, stream, a);
  return hipGetLastError();
}

template <bool kH16, bool kCodes>
hipError_t launch_split(const AttnArgs& a, int num_workers, hipStream_t stream) {
  if (a.page_size % kTileKeys == 0)
    hipLaunchKernelGGL((attention_split_kernel<true, kH16, kCodes>), dim3(num_workers),
                       dim3(2 * kWave), 0, stream, a);
  else
    hipLaunchKernelGGL((attention_split_kernel<false, kH16, kCodes>), dim3(num_workers),
                       dim3(2 * kWave), 0, stream, a);
  return hipGetLastError();
}

template <bool kFp8>
hipError_t launch_dtype(const AttnArgs& a, int num_workers, hipStream_t stream) {
  if (a.num_heads <= 32) {
    // (at most 16 heads: the 16-slot layout of the same kernels)
    if constexpr (kFp8) {
      // (any worker count; the planner gives it two per compute unit)
      if (a.num_heads <= 16) return launch_split<true, true>(a, num_workers, stream);
      return launch_split<false, true>(a, num_workers, stream);
    } else {
      // (at most 16 heads: a producer wave stages the bf16 rows through its
      // registers two tiles ahead, as for fp8 codes)
      if (a.compact && a.num_heads <= 16) return launch_split<true, false>(a, num_workers, stream);
      if (a.compact) return launch_nw<1, false, true>(a, num_workers, stream);
      return launch_nw<1, false>(a, num_workers, stream);
    }
  }
  if (a.num_heads <= 64) return launch_nw<2, kFp8>(a, num_workers, stream);
  return launch_nw<4, kFp8>(a, num_workers, stream);
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int num_workers, hipStream_t stream) {
  if (num_workers <= 0) return hipSuccess;
  if (a.num_heads <= 0 || a.num_heads > kMaxHeads) return hipErrorInvalidValue;
  return a.kv_cache8 ? launch_dtype<true>(a, num_workers, stream)
                     : launch_dtype<false>(a, num_workers, stream);
}

}  // namespace mla
