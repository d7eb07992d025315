// Per-head projections around latent attention, for gfx950 (page
// "mstar.engine.resources.attn.flashinfer_mla", module description: the
// query entering the kernel is absorbed, q_nope @ W_UK, and the latent output
// is brought back to the value heads by W_UV):
//   out[t, h, :] = x[t, h, :] @ w[h]      x [T, H, K], w [H, K, N], out [T, H, N]
// bf16 in, fp32 accumulation, bf16 out (round to nearest even).  Absorption
// is K = 128, N = 512; the up-projection K = 512, N = 128.
//
// A workgroup takes one head and N / kNSplit output columns, and loops over
// blocks of kTok tokens.
// Its slice of w[h] is staged in LDS transposed (row n holds the K weights
// of output column n), so that both MFMA operands are 16-byte reads with K
// contiguous: out^T[n, t] = sum_k w^T[n, k] x^T[k, t] on
// v_mfma_f32_32x32x16_bf16 with columns as M and tokens as N.  Wave w takes
// tokens 32 w .. 32 w + 31 of the block and every column of the slice; the
// token rows are loaded straight from global memory into the B operand.
// At these shapes the products are bound by HBM traffic (the [T, H, 512]
// side dominates), so the design aims at streaming, not at MFMA peak.
#include <algorithm>

#include "kernels.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

constexpr int kProjWaves = 4;
constexpr int kTok = 32 * kProjWaves;  // tokens per block (32 per wave)
constexpr int kChunk = 128;            // columns per coalesced row piece (256 bytes)
constexpr int kPieceRow = kChunk + 8;  // bf16 per LDS row of a piece (padding staggers banks)

// kNSplit workgroups share a (head, token block): each stages N / kNSplit
// columns of the head's weights (absorption: 4, 70 KB of LDS, two workgroups
// per compute unit; up-projection: 2, 101 KB, one, so that each input row
// is read by two workgroups only).  The [T, H, 512] side of each product goes
// through per-wave LDS pieces of 32 tokens x 128 columns, so that global
// memory sees 256-byte row pieces (4 tokens per wave instruction): the
// absorption's output, the up-projection's input.
template <int K, int N>
struct ProjShape {
  static constexpr bool kStageOut = N > K;  // absorption: stage the output
  static constexpr int kNSplit = kStageOut ? 4 : 2;
  static constexpr int kCols = N / kNSplit;  // output columns per workgroup
  static constexpr int kRow = K + 8;         // bf16 per LDS row of transposed weights
  static constexpr int kWBytes = kCols * kRow * 2;
  static constexpr int kPieceBytes = 32 * kPieceRow * 2;  // one wave's piece
  static constexpr int kLdsBytes = kWBytes + kProjWaves * kPieceBytes;
  static constexpr int kKSteps = K / 16;
  static constexpr int kNBlocks = kCols / 32;
  static_assert(K % kChunk == 0 && kCols % 32 == 0, "shape");
  static_assert(!kStageOut || kCols == kChunk, "an output piece is one row chunk");
  static_assert(kLdsBytes <= 160 * 1024, "LDS holds 160 KiB");
};

__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14));  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// The grid is one-dimensional: workgroups go round-robin over the 8 XCDs of
// the device, each with its own L2, and the kNSplit workgroups that read the
// same input rows (one (token-block, head) pair, different output columns)
// are numbered 8 apart, so they run on one XCD at about the same time and
// all but the first find the rows in its L2.
template <int K, int N>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void head_matmul_kernel(
    const uint16_t* x, const uint16_t* w, uint16_t* out, int64_t T, int H, int n_bx) {
  using S = ProjShape<K, N>;
  __shared__ __attribute__((aligned(16))) uint32_t lds[S::kLdsBytes / 4];
  constexpr int kXcds = 8;
  const int id = blockIdx.x;
  const int r = id % (kXcds * S::kNSplit);
  const int pair = (id / (kXcds * S::kNSplit)) * kXcds + r % kXcds;
  if (pair >= n_bx * H) return;  // (the grid is rounded up to whole groups)
  const int bx = pair % n_bx;
  const int h = pair / n_bx;
  const int n_base = (r / kXcds) * S::kCols;
  // Stage w[h][:, n_base .. n_base + kCols) transposed: task (k pair kp,
  // 8-column group g) reads rows 2 kp and 2 kp + 1 (16 bytes each) and writes
  // eight dwords {w[2kp][n], w[2kp+1][n]} to LDS row n at column 2 kp.
  // Consecutive lanes take consecutive k pairs, so the dword writes of a
  // wave fall in distinct banks.
  {
    const uint16_t* wh = w + static_cast<int64_t>(h) * K * N + n_base;
    constexpr int kTasks = (K / 2) * (S::kCols / 8);
    for (int task = threadIdx.x; task < kTasks; task += blockDim.x) {
      const int kp = task % (K / 2), g = task / (K / 2);
      const u32x4_t r0 = *reinterpret_cast<const u32x4_t*>(wh + (2 * kp) * N + 8 * g);
      const u32x4_t r1 = *reinterpret_cast<const u32x4_t*>(wh + (2 * kp + 1) * N + 8 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = (r0[j] & 0xFFFFu) | (r1[j] << 16);
        const uint32_t hi = (r0[j] >> 16) | (r1[j] & 0xFFFF0000u);
        lds[((8 * g + 2 * j) * S::kRow + 2 * kp) / 2] = lo;
        lds[((8 * g + 2 * j + 1) * S::kRow + 2 * kp) / 2] = hi;
      }
    }
  }
  __syncthreads();
  // The staged weights serve every token block this workgroup takes:
  // blocks bx, bx + n_bx, ...
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, half = lane >> 5;
  const char* lrow = reinterpret_cast<const char*>(lds) + (l32 * S::kRow + 8 * half) * 2;
  char* piece = reinterpret_cast<char*>(lds) + S::kWBytes + wave * S::kPieceBytes;
  // Row-piece task of a lane: token 4 j + lane / 16 of the wave's 32 (j = 0..7),
  // columns 8 (lane % 16) .. + 7 of the piece.
  const int pr = lane >> 4, pc = 8 * (lane & 15);
  // Up-projection input pieces: piece c (columns 128 c .. + 127) of this
  // wave's 32 tokens of a block, 8 loads of 16 bytes per lane.  All K / 128
  // pieces of the next block are in flight while this block's are used:
  // piece c of block b+1 is loaded as soon as piece c of block b has gone to
  // LDS.
  constexpr int kPieces = S::kStageOut ? 1 : K / kChunk;
  u32x4_t buf[kPieces][8];
  auto load_piece = [&](int64_t tw, int c, u32x4_t (&v)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int64_t t = tw + 4 * j + pr;
      t = t < T ? t : T - 1;
      v[j] = *reinterpret_cast<const u32x4_t*>(x + (t * H + h) * K + c * kChunk + pc);
    }
  };
  if constexpr (!S::kStageOut) {
    const int64_t tw0 = static_cast<int64_t>(bx) * kTok + 32 * wave;
    if (tw0 < T)
#pragma unroll
      for (int c = 0; c < kPieces; ++c) load_piece(tw0, c, buf[c]);
  }
  for (int64_t t0 = static_cast<int64_t>(bx) * kTok; t0 < T; t0 += static_cast<int64_t>(n_bx) * kTok) {
    const int64_t tw = t0 + 32 * wave;
    if (tw >= T) break;
    const int64_t tw_next = tw + static_cast<int64_t>(n_bx) * kTok;
    f32x16_t acc[S::kNBlocks];
#pragma unroll
    for (int nb = 0; nb < S::kNBlocks; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nb][r] = 0.f;
    auto mfma_step = [&](int ks, const u32x4_t& xv) {
      const bf16x8_t b = __builtin_bit_cast(bf16x8_t, xv);
#pragma unroll
      for (int nb = 0; nb < S::kNBlocks; ++nb) {
        const bf16x8_t a =
            *reinterpret_cast<const bf16x8_t*>(lrow + (nb * 32 * S::kRow + 16 * ks) * 2);
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[nb], 0, 0, 0);
      }
    };
    if constexpr (S::kStageOut) {
      // B operand straight from global memory: token tw + l32 (clamped into
      // the batch; not stored), its columns 16 ks + 8 half .. + 7.
      const int64_t tl = tw + l32 < T ? tw + l32 : T - 1;
      const uint16_t* xr = x + (tl * H + h) * K + 8 * half;
      u32x4_t xb[S::kKSteps];
#pragma unroll
      for (int ks = 0; ks < S::kKSteps; ++ks) xb[ks] = *reinterpret_cast<const u32x4_t*>(xr + 16 * ks);
#pragma unroll
      for (int ks = 0; ks < S::kKSteps; ++ks) mfma_step(ks, xb[ks]);
    } else {
      // The input rows arrive in 128-column pieces, 256 bytes per token per
      // load, through LDS (buf holds this block's pieces, loaded during the
      // previous block).
#pragma unroll
      for (int c = 0; c < kPieces; ++c) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<u32x4_t*>(piece + ((4 * j + pr) * kPieceRow + pc) * 2) = buf[c][j];
        if (tw_next < T) load_piece(tw_next, c, buf[c]);
        wave_lds_sync();
#pragma unroll
        for (int kk = 0; kk < kChunk / 16; ++kk) {
          const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(
              piece + (l32 * kPieceRow + 16 * kk + 8 * half) * 2);
          mfma_step(c * (kChunk / 16) + kk, xv);
        }
        wave_lds_sync();  // (the piece is rewritten next)
      }
    }
    // acc[nb][4 i + j] is out^T[n, t] for column n = 32 nb + 8 i + 4 half + j
    // of the slice and token tw + l32.
    auto pack4 = [&](int nb, int i) {
      const f32x2_t p0 = {acc[nb][4 * i], acc[nb][4 * i + 1]};
      const f32x2_t p1 = {acc[nb][4 * i + 2], acc[nb][4 * i + 3]};
      return u32x2_t{__builtin_bit_cast(uint32_t, __builtin_convertvector(p0, bf16x2_t)),
                     __builtin_bit_cast(uint32_t, __builtin_convertvector(p1, bf16x2_t))};
    };
    if constexpr (S::kStageOut) {
      // The 32 x 128 output piece goes through LDS and leaves as 256-byte
      // row pieces.
#pragma unroll
      for (int nb = 0; nb < S::kNBlocks; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<u32x2_t*>(piece + (l32 * kPieceRow + 32 * nb + 8 * i + 4 * half) * 2) =
              pack4(nb, i);
      wave_lds_sync();
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t t = tw + 4 * j + pr;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(piece + ((4 * j + pr) * kPieceRow + pc) * 2);
        // (whole 16-byte pieces of rows written once: non-temporal)
        if (t < T)
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(out + (t * H + h) * N + n_base + pc));
      }
      wave_lds_sync();  // (the piece is rewritten next)
    } else if (tw + l32 < T) {
      uint16_t* orow = out + ((tw + l32) * H + h) * N + n_base + 4 * half;
#pragma unroll
      for (int nb = 0; nb < S::kNBlocks; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x2_t*>(orow + 32 * nb + 8 * i) = pack4(nb, i);
    }
  }
}

template <int K, int N>
hipError_t launch(const uint16_t* x, const uint16_t* w, uint16_t* out, int64_t T, int H,
                  hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  if (H > 65535) return hipErrorInvalidValue;
  // One round of workgroups (256 compute units; two resident workgroups per
  // unit for the absorption, one for the up-projection), each looping over
  // token blocks with its staged weights: a second round stages the weights
  // again and leaves a tail (up-projection at T = 4096: 156 against 170 us
  // with four workgroups per unit).
  const int64_t need = (T + kTok - 1) / kTok;
  constexpr int kNSplit = ProjShape<K, N>::kNSplit;
  constexpr int64_t kSlots = ProjShape<K, N>::kStageOut ? 512 : 256;
  const int64_t per_head = std::max<int64_t>(1, kSlots / (static_cast<int64_t>(H) * kNSplit));
  const int64_t blocks = std::min(need, per_head);
  const int64_t groups = (blocks * H + 7) / 8;  // of 8 (token-block, head) pairs
  const int64_t grid = groups * 8 * kNSplit;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((head_matmul_kernel<K, N>), dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                     stream, x, w, out, T, H, static_cast<int>(blocks));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_absorb_query(const uint16_t* q, const uint16_t* w_uk, uint16_t* q_abs, int64_t T,
                               int H, hipStream_t stream) {
  return launch<kNopeDim, kLoraRank>(q, w_uk, q_abs, T, H, stream);
}

hipError_t launch_up_project(const uint16_t* o, const uint16_t* w_uv, uint16_t* v, int64_t T,
                             int H, hipStream_t stream) {
  return launch<kLoraRank, kValueDim>(o, w_uv, v, T, H, stream);
}

}  // namespace mla
