// Small-M (decode) block-scaled W4A4 contraction: paper "Why Gated DeltaNet
// Survives 4-Bit Quantization", section 2 "NVFP4" (both operands NVFP4, FP32
// accumulate).  W arrives as packed codes and scale bytes and is expanded
// exactly to fp16 in registers; X arrives already expanded to fp16 by the
// quantize kernel.  The epilogue applies RN(gs_x * gs_w).
//
// With kA16 the same kernels compute W4A16 (model card "Gemma-4-31B-IT-
// NVFP4-FP8attn-text", section "Limitations"): bf16 operands, X the caller's
// bf16 activations as given, W expanded exactly to bf16, and gs_w alone in
// the epilogue.
#include "encode.h"
#include "launch.h"
#include "mfma_util.h"

#include <type_traits>

namespace nvfp4 {

// ====================================================================== GEMV
// M <= 16 (decode).  MFMA 16x16x32 with W as the 16-row A operand and the
// (zero-padded) activations as the 16-column B operand.  A workgroup owns
// NT*16 rows of W; its 4 waves split K round-robin in 128-k chunks and their
// partial sums are added in a fixed order through LDS, so the result does
// not depend on scheduling.
template <int NT, bool kA16, bool kYBf16>
__global__ __launch_bounds__(256) void gemv_kernel(const uint4* __restrict__ x16, uint32_t kp_chunks, int M,
                                                    const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws,
                                                    int N, int K, const float* __restrict__ gsx_p,
                                                    const float* __restrict__ gsw_p, uint8_t* __restrict__ y,
                                                    size_t ld_y_bytes) {
  using O = Op<kA16>;
  __shared__ floatx4 part[4][NT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * (NT * 16);
  const size_t kh = (size_t)K / 2, ks = (size_t)K / 16;

  const uint8_t* wrow[NT];
  const uint8_t* srow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int n = n0 + t * 16 + l16;
    n = n < N ? n : N - 1;
    wrow[t] = wc + (size_t)n * kh;
    srow[t] = ws + (size_t)n * ks;
  }
  const bool mvalid = l16 < M;
  const uint4* xrow = x16 + (size_t)(mvalid ? l16 : 0) * kp_chunks;

  floatx4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int kb = wave * 128; kb < K; kb += 512) {
    const int kk = kb + 32 * g;
    const bool kvalid = kk < K;
    uint4 wv[NT];
    uint32_t sv[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      wv[t] = kvalid ? *reinterpret_cast<const uint4*>(wrow[t] + kk / 2) : make_uint4(0, 0, 0, 0);
      sv[t] = kvalid ? *reinterpret_cast<const uint16_t*>(srow[t] + kk / 16) : 0u;
    }
    uint4 xv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) xv[j] = (mvalid && kvalid) ? xrow[kk / 8 + j] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t s0 = O::scale_bits(sv[t]), s1 = O::scale_bits(sv[t] >> 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t e[4];
        O::expand(dword_of(wv[t], j), j < 2 ? s0 : s1, e);
        acc[t] = O::mfma16(O::vec(make_uint4(e[0], e[1], e[2], e[3])), O::vec(xv[j]), acc[t]);
      }
    }
  }

#pragma unroll
  for (int t = 0; t < NT; ++t) part[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave != 0) return;
  const float scale = kA16 ? *gsw_p : (*gsx_p) * (*gsw_p);
  if (!mvalid) return;
  uint8_t* yrow = y + (size_t)l16 * ld_y_bytes;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    floatx4 s = part[0][t][lane];
    floatx4 s1 = part[1][t][lane], s2 = part[2][t][lane], s3 = part[3][t][lane];
    s = s + s1;
    s = s + s2;
    s = s + s3;
    const int n = n0 + t * 16 + 4 * g;
    store4<kYBf16>(yrow, n, N, s[0] * scale, s[1] * scale, s[2] * scale, s[3] * scale);
  }
}

// ---------------------------------------------------------------- M <= 4
// Decode: the GEMV reads 100 MB of weights once, so it is bound by how many
// bytes are in flight and by how cheaply each instruction moves them.  A
// workgroup is one wave; it owns a 16-row tile of W over the whole of K.
//
// Everything reaches LDS by direct global->LDS transfers that the compiler
// does not see, so every wait is an explicit, exact s_waitcnt:
//   * first the tile's scale bytes (16 rows x K/16, contiguous in memory),
//     in 1 KB pieces;
//   * then a ring of D chunks of 256 k: the codes (16 rows x 128 B, two
//     transfers that each fill 8 whole 128-byte lines) and the activations
//     (M rows x 512 B of fp16, 32 lanes per row).
// Code piece p of row r lands in 16-byte slot p ^ (r & 7) of its 128-byte
// LDS row, and activation piece 8a + b in slot 8a + (b ^ a) of its row, so
// the lanes of one read pass hit distinct bank groups.
//
// Inside a chunk, lane (r = lane % 16, g = lane / 16) takes k 64g .. 64g+63
// of row r: 32 code bytes, read as two 16-byte pieces, whose dword t feeds
// MFMA step t (16x16x32, k = 64g + 8t .. +7 on both operands); the lane's
// four scale bytes for those k are one dword of the staged scales.  Lanes of
// activation rows m >= M keep zero operands.  Partial sums stay in the wave,
// so the result does not depend on scheduling.
constexpr uint32_t kGvChunkCodes = 2048;  // 16 rows x 128 B

template <int D, int XI, bool kA16, bool kYBf16>
__global__ __launch_bounds__(64) void gemv_stream_kernel(const uint8_t* __restrict__ x16, uint32_t ld_x16_bytes,
                                                          int M, const uint8_t* __restrict__ wc,
                                                          const uint8_t* __restrict__ ws, int N, int K,
                                                          const float* __restrict__ gsx_p,
                                                          const float* __restrict__ gsw_p,
                                                          uint8_t* __restrict__ y, size_t ld_y_bytes) {
  using O = Op<kA16>;
  extern __shared__ uint4 smem[];
  constexpr uint32_t kSlot = kGvChunkCodes + XI * 1024u;
  uint8_t* lds = reinterpret_cast<uint8_t*>(smem);
  uint8_t* sc_lds = lds + D * kSlot;                    // staged scales [16][K/16]

  const int lane = threadIdx.x, l16 = lane & 15, g = lane >> 4;
  const int tile = blockIdx.x;
  const uint32_t kh = (uint32_t)K / 2, ks = (uint32_t)K / 16;
  const int nck = K >> 8;  // a multiple of D

  // ---- transfers
  const uint32_t ring0 = lds_addr(lds), sc0 = lds_addr(sc_lds);
  // codes: transfer h, lane i -> row 8h + i/8, slot i%8 holding piece (i%8) ^ (row & 7)
  int crow[2];
  uint32_t coff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 8 * h + (lane >> 3);
    int n = tile * 16 + r;
    n = n < N ? n : N - 1;
    crow[h] = r;
    coff[h] = (uint32_t)n * kh + 16u * (uint32_t)((lane & 7) ^ (r & 7));
  }
  // activations: transfer v, lane i -> row 2v + i/32 (clamped to M-1), LDS
  // slot p = i % 32 of that row holding piece 8 (p / 8) + ((p % 8) ^ (p / 8))
  uint32_t xoff[XI];
#pragma unroll
  for (int v = 0; v < XI; ++v) {
    int m = 2 * v + (lane >> 5);
    m = m < M ? m : M - 1;
    const uint32_t p = (uint32_t)(lane & 31), piece = (p & ~7u) | ((p & 7u) ^ (p >> 3));
    xoff[v] = (uint32_t)m * ld_x16_bytes + 16u * piece;
  }
  int next = 0;  // next chunk to transfer
  auto issue = [&](int d) {
    const int c = next < nck ? next : nck - 1;
    const uint32_t slot = ring0 + (uint32_t)d * kSlot;
    lds_dma16(wc, coff[0] + (uint32_t)c * 128u, slot);
    lds_dma16(wc, coff[1] + (uint32_t)c * 128u, slot + 1024u);
#pragma unroll
    for (int v = 0; v < XI; ++v) lds_dma16(x16, xoff[v] + (uint32_t)c * 512u, slot + kGvChunkCodes + 1024u * v);
    ++next;
  };

  // Scales first: 16 rows x ks bytes are contiguous; pieces past the end
  // re-read the last piece (their LDS bytes are never read).
  {
    int n0 = tile * 16;
    const uint32_t rows_here = (uint32_t)((N - n0) < 16 ? (N - n0) : 16);
    const uint32_t bytes = rows_here * ks;  // a multiple of 4 (K % 64 == 0)
    const uint32_t base = (uint32_t)n0 * ks;
    const uint32_t npieces = (16u * ks + 1023u) / 1024u;
    for (uint32_t q = 0; q < npieces; ++q) {
      uint32_t off = q * 1024u + 16u * (uint32_t)lane;
      off = off + 16u <= bytes ? off : (bytes >= 16u ? bytes - 16u : 0u);
      lds_dma16(ws, base + off, sc0 + q * 1024u);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d);

  const bool mvalid = l16 < M;
  const float scale = kA16 ? *gsw_p : (*gsx_p) * (*gsw_p);
  // this lane's reads
  const uint32_t sw = (uint32_t)(l16 & 7);
  const uint32_t cpos0 = (uint32_t)l16 * 128u + 16u * ((2u * g) ^ sw);
  const uint32_t cpos1 = (uint32_t)l16 * 128u + 16u * ((2u * g + 1u) ^ sw);
  const uint8_t* sc_row = sc_lds + (uint32_t)l16 * ks + 4u * g;

  const uint32_t xg = (uint32_t)g;
  uint4 xv[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) xv[t] = make_uint4(0, 0, 0, 0);
  // two accumulators: alternate MFMAs do not wait for each other's result
  floatx4 acc[2] = {floatx4{0.0f, 0.0f, 0.0f, 0.0f}, floatx4{0.0f, 0.0f, 0.0f, 0.0f}};
  for (int c0 = 0; c0 < nck; c0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      wait_vmcnt<(D - 1) * (2 + XI)>();
      const uint8_t* slot = lds + d * kSlot;
      const uint4 w0 = *reinterpret_cast<const uint4*>(slot + cpos0);
      const uint4 w1 = *reinterpret_cast<const uint4*>(slot + cpos1);
      const uint32_t sd = *reinterpret_cast<const uint32_t*>(sc_row + (uint32_t)(c0 + d) * 16u);
      // Only the lanes of real activation rows read them; the others keep
      // the zeros their operand registers started with.
      if (mvalid) {
        const uint8_t* xb = slot + kGvChunkCodes + 512u * l16 + 128u * g;
#pragma unroll
        for (int t = 0; t < 8; ++t) xv[t] = *reinterpret_cast<const uint4*>(xb + 16u * ((uint32_t)t ^ xg));
      }
      // the slot's reads are complete: refill it before computing, so the
      // transfer is not held back by this chunk's arithmetic
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(d);
      const uint32_t s0 = O::scale_bits(sd), s1 = O::scale_bits(sd >> 8), s2 = O::scale_bits(sd >> 16),
                     s3 = O::scale_bits(sd >> 24);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t sp = t < 2 ? s0 : (t < 4 ? s1 : (t < 6 ? s2 : s3));
        uint32_t e[4];
        O::expand(dword_of(t < 4 ? w0 : w1, t & 3), sp, e);
        acc[t & 1] = O::mfma16(O::vec(make_uint4(e[0], e[1], e[2], e[3])), O::vec(xv[t]), acc[t & 1]);
      }
    }
  }
  wait_vmcnt<0>();
  const floatx4 a = acc[0] + acc[1];
  if (mvalid)
    store4<kYBf16>(y + (size_t)l16 * ld_y_bytes, tile * 16 + 4 * g, N, a[0] * scale, a[1] * scale, a[2] * scale,
                   a[3] * scale);
}

// --------------------------------------------------- M <= 4, FP4 contraction
// Up to four activation rows against W with both operands NVFP4: the
// contraction runs on the FP4 MFMA (16x16x128, E2M1 operands with unit
// scales) over the raw codes, so no weight element is converted: each output
// column of an MFMA collects one (activation row, 16-element block) pair, and
// its exact sum is multiplied by the block's two E4M3 scales afterwards (the
// product of two NVFP4 blocks, paper "Why Gated DeltaNet Survives 4-Bit
// Quantization", section 2 "NVFP4").  Only the fp32 accumulation over blocks
// rounds, as in every other contraction kernel, in another order.
//
// The rows come either as bf16, quantized by the kernel itself (the whole
// decode step in one launch; the tensor scale from their absmax, or given),
// or already quantized: the packed codes [M][K/2] and scale bytes [M][K/16]
// nvfp4_gemm_prepare leaves in its workspace, with gs_x.  A separate quantize
// launch costs the step more than its work; here every workgroup quantizes
// the rows (at most 4 x 5120 elements) into its own LDS while its weight
// transfers are in flight.
//
// A workgroup is kW waves, one 16-row weight tile each, sharing the
// quantized rows in LDS (codes, 8 B a block, then the scale bytes, both in
// row order).  The M * K/16 blocks, counted row after row, are dealt to the
// waves in sets of 64 (set j to wave j % kW; lane l takes block
// 64 j + l).  Order of work in a wave:
//   1. prepared rows: direct transfers into LDS of 1 KB pieces q with
//      q % kW = wave of the codes and scale bytes, then of its tile's
//      scale bytes (16 rows x K/16, contiguous) and the first D chunks of
//      codes (16 rows x 128 B per chunk, two transfers filling 8 lines
//      each); transfers complete in the order issued, so the wave waits for
//      its pieces alone.
//      One bf16 row: the same, with the bytes of its own sets in place of
//      the pieces (staged at their row offsets).
//      Two to four bf16 rows (twice to four times the LDS): its sets are
//      loaded into registers, and the weight transfers are issued once the
//      loads have landed (the compiler's wait for a register load would
//      also wait for every transfer issued before it is used);
//   2. bf16 rows: the absmax of its blocks (exact: integer max of the
//      magnitudes), combined over the wave and, through LDS and a barrier,
//      over the workgroup; the tensor scale RN(amax / 2688) (or the given
//      one); the encode of its blocks into codes and scale bytes in LDS
//      (one staged row: written over its bf16 bytes, after a barrier, as
//      they overlap other waves' blocks);
//   3. one barrier, then the streaming loop below;
//   4. bf16 rows: workgroup 0 writes the quantized rows to the workspace as
//      nvfp4_gemm_prepare would (the fp16 values E2M1 * E4M3, the codes and
//      scale bytes, the tensor scale).  Stored last: a store can be
//      acknowledged before older loads return, so stores issued while loads
//      are in flight would let a compiler-counted wait for those loads pass
//      early.
typedef int i32x8 __attribute__((ext_vector_type(8)));  // operands of the scaled MFMAs
constexpr int kFuDepth = 4;
constexpr int kFuMaxWaves = 16;
// Waves per workgroup: the quantizing forms repeat the encode of all rows in
// every workgroup, so more rows take wider (and fewer) workgroups.
constexpr int fp4_waves(int M) { return M == 1 ? 3 : 9; }
enum FuMode { kFuDynamic = 0, kFuGiven = 1, kFuPrepared = 2 };

// Set i of wave w among NS sets of 64 blocks (NS or more: none).  Fewer than
// four waves take every W-th set.  With four or more, the sets go to the
// four SIMDs in turn (wave w runs on SIMD w % 4) and then to the waves of
// each SIMD in turn, so the SIMDs get equal shares of the encode.
constexpr int fp4_set(int W, int w, int i) {
  return W < 4 ? w + W * i : (w & 3) + 4 * ((w >> 2) + (W - (w & 3) + 3) / 4 * i);
}
constexpr int fp4_sets_per_wave(int W, int NS) {
  int most = 0;
  for (int w = 0; w < W; ++w) {
    int n = 0;
    while (fp4_set(W, w, n) < NS) ++n;
    most = most > n ? most : n;
  }
  return most;
}

template <int NCK, int kM, int kW, int kMode, bool kYBf16>
__global__ __launch_bounds__(64 * kW) void gemv_fp4_kernel(const uint8_t* __restrict__ x, size_t ldx,
                                                                 const float* __restrict__ gs_in,
                                                                 const uint8_t* __restrict__ wc,
                                                                 const uint8_t* __restrict__ ws, int N, int tiles,
                                                                 const float* __restrict__ gsw_p,
                                                                 uint8_t* __restrict__ y, size_t ldy,
                                                                 uint4* __restrict__ x16_out,
                                                                 float* __restrict__ gsx_out,
                                                                 uint8_t* __restrict__ q_out) {
  constexpr int K = NCK * 256, NB = K / 16, D = kFuDepth;
  static_assert(NB % 64 == 0, "whole sets of 64 blocks");
  static_assert(kM >= 1 && kM <= 4, "one to four rows");
  static_assert(kW >= 1 && kW <= kFuMaxWaves, "waves");
  constexpr int SPR = NB / 64;                          // sets per row
  constexpr int NS = kM * SPR;                          // sets over all rows
  constexpr int SPW = fp4_sets_per_wave(kW, NS);        // sets of the busiest wave
  constexpr bool kStage = kMode != kFuPrepared && kM == 1;  // the bf16 row staged in LDS
  constexpr uint32_t kh = K / 2, ks = K / 16;
  constexpr uint32_t kScBytes = (16u * ks + 1023u) / 1024u * 1024u;
  constexpr uint32_t kQBytes = (uint32_t)kM * (kh + ks);        // codes, then scale bytes
  constexpr uint32_t kQPieces = (kQBytes + 1023u) / 1024u;      // in 1 KB pieces
  constexpr uint32_t kRowBytes = kStage ? 2u * K : kQPieces * 1024u;
  constexpr int kScT = (int)(kScBytes / 1024u);                 // scale transfers per wave
  // rows [kRowBytes: bf16 (one staged row), then codes | scale bytes] |
  // ring [wave][D][2048 B] | scales [wave][kScBytes] | wave maxima [kW]
  extern __shared__ uint4 smem[];
  const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // uniform: scalar bases
  const int tile_raw = blockIdx.x * kW + wave;
  const int tile = tile_raw < tiles ? tile_raw : tiles - 1;  // a surplus wave redoes the last tile, unstored
  uint8_t* xrow = reinterpret_cast<uint8_t*>(smem);
  uint8_t* ring = xrow + kRowBytes + (size_t)wave * D * kGvChunkCodes;
  uint8_t* sc_lds = xrow + kRowBytes + (size_t)kW * D * kGvChunkCodes + (size_t)wave * kScBytes;
  uint32_t* wmax = reinterpret_cast<uint32_t*>(xrow + kRowBytes + (size_t)kW * (D * kGvChunkCodes + kScBytes));
  uint2* xcodes = reinterpret_cast<uint2*>(xrow);  // [kM][NB]
  uint8_t* xsb = xrow + kM * kh;                    // [kM][NB]
  const uint32_t x0 = lds_addr(xrow);

  const int n0 = tile * 16;
  const uint8_t* wtile = wc + (size_t)n0 * kh;
  uint32_t coff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 8 * h + (lane >> 3);
    const int n = n0 + r < N ? n0 + r : N - 1;
    coff[h] = (uint32_t)(n - n0) * kh + 16u * (uint32_t)((lane & 7) ^ (r & 7));
  }
  const uint32_t ring0 = lds_addr(ring);
  auto issue = [&](int c, int d) {  // chunk c (clamped) into ring slot d
    c = c < NCK ? c : NCK - 1;
    const uint32_t slot = ring0 + (uint32_t)d * kGvChunkCodes;
    lds_dma16(wtile, coff[0] + (uint32_t)c * 128u, slot);
    lds_dma16(wtile, coff[1] + (uint32_t)c * 128u, slot + 1024u);
  };
  // the tile's scale bytes (pieces past the end re-read the last piece;
  // their LDS bytes are never read), then the first D chunks of codes
  auto issue_weights = [&]() {
    const uint32_t rows_here = (uint32_t)((N - n0) < 16 ? (N - n0) : 16);
    const uint32_t bytes = rows_here * ks;  // a multiple of 16 (K % 256 == 0)
    const uint32_t sc0 = lds_addr(sc_lds);
#pragma unroll
    for (uint32_t q = 0; q < kScBytes / 1024u; ++q) {
      uint32_t off = q * 1024u + 16u * (uint32_t)lane;
      off = off + 16u <= bytes ? off : bytes - 16u;
      lds_dma16(ws + (size_t)n0 * ks, off, sc0 + q * 1024u);
    }
#pragma unroll
    for (int d = 0; d < D; ++d) issue(d, d);
  };

  // 1. the activation bytes, then the weight transfers
  uint32_t xw[kMode == kFuPrepared ? 1 : SPW][BlockWords<true>::n];
  if constexpr (kMode == kFuPrepared) {
#pragma unroll
    for (uint32_t q = 0; q < kQPieces; ++q) {
      if (q % kW != (uint32_t)wave) continue;
      uint32_t off = 1024u * q + 16u * (uint32_t)lane;
      off = off + 16u <= kQBytes ? off : kQBytes - 16u;  // bytes past the rows are never read
      lds_dma16(x, off, x0 + 1024u * q);
    }
    issue_weights();
    wait_vmcnt<kScT + 2 * D>();  // this wave's pieces have landed
  } else if constexpr (kStage) {
    // set j = bytes 2048 j .. 2048 j + 2047 of the bf16 row, two 1 KB transfers
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if (j % kW != wave) continue;
      lds_dma16(x, 2048u * j + 16u * (uint32_t)lane, x0 + 2048u * j);
      lds_dma16(x, 2048u * j + 1024u + 16u * (uint32_t)lane, x0 + 2048u * j + 1024u);
    }
    issue_weights();
    wait_vmcnt<kScT + 2 * D>();  // this wave's row bytes have landed
    const uint4* xs = reinterpret_cast<const uint4*>(xrow);
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int j = fp4_set(kW, wave, i);
      if (j >= NS) continue;
      const uint4 a = xs[2 * (lane + 64 * j)], b = xs[2 * (lane + 64 * j) + 1];
      xw[i][0] = a.x; xw[i][1] = a.y; xw[i][2] = a.z; xw[i][3] = a.w;
      xw[i][4] = b.x; xw[i][5] = b.y; xw[i][6] = b.z; xw[i][7] = b.w;
    }
  } else {
    // a surplus set (the last wave may own one fewer) reloads the last set:
    // its absmax repeats a max, and it is not encoded
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int j = fp4_set(kW, wave, i) < NS ? fp4_set(kW, wave, i) : NS - 1;
      const uint4* p = reinterpret_cast<const uint4*>(x + (size_t)(j / SPR) * ldx) + 2 * (64 * (j % SPR) + lane);
      const uint4 a = p[0], b = p[1];
      xw[i][0] = a.x; xw[i][1] = a.y; xw[i][2] = a.z; xw[i][3] = a.w;
      xw[i][4] = b.x; xw[i][5] = b.y; xw[i][6] = b.z; xw[i][7] = b.w;
    }
    // every loaded word is in its register before the first transfer is
    // issued (ordered volatile asm statements that read them)
#pragma unroll
    for (int i = 0; i < SPW; ++i)
#pragma unroll
      for (int k = 0; k < BlockWords<true>::n; ++k) asm volatile("" ::"v"(xw[i][k]));
    issue_weights();
  }

  // 2. the quantized rows
  float gs;
  if constexpr (kMode == kFuPrepared) {
    gs = *gs_in;
  } else {
    if constexpr (kMode == kFuGiven) {
      gs = *gs_in;
    } else {
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < SPW; ++i) {
        if (kStage && fp4_set(kW, wave, i) >= NS) continue;
        const uint32_t a = words_absmax_bits<true>(xw[i]);
        m = m > a ? m : a;
      }
      m = wave_max_u32(m);
      if (lane == 0) wmax[wave] = m;
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
      for (int w = 0; w < kW; ++w) m = m > wmax[w] ? m : wmax[w];
      gs = tensor_scale(__uint_as_float(m));
    }
    // A staged row's codes and scale bytes overwrite bf16 bytes of other
    // blocks, so every wave has read its blocks first (the barrier above, or
    // this one with a given scale).
    if constexpr (kStage && kMode == kFuGiven) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // Half-blocks whose code brackets straddle a decision point (nearly
    // every set has one in some lane on decode rows with outlier channels)
    // are settled after the fast pass: each lane keeps up to two of them
    // (their bf16 words, es and position; picked with compile-time set
    // indices, so the sets stay in registers), settled in two passes over
    // the wave, so the divisions run once or twice per wave rather than once
    // per set.  A lane's third one is settled at once.
    const FastScale fsc = fast_scale(gs);
    uint32_t dw[2][4] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    float des[2] = {0.0f, 0.0f};
    uint32_t dpos[2] = {0u, 0u};  // 2 * block + half
    uint32_t nd = 0;
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int j = fp4_set(kW, wave, i);
      if (j >= NS) continue;
      const int b = lane + 64 * j;
      float xv[16];
      words_to_floats<true>(xw[i], xv);
      uint32_t sb, lo, hi, straddle;
      float es;
      if (!encode_block_fast_parts(xv, words_absmax_bits<true>(xw[i]), fsc, sb, lo, hi, es, straddle)) {
        sb = encode_block_exact(xv, gs, lo, hi);
        straddle = 0;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (straddle & (1u << h)) {
          if (nd < 2) {
#pragma unroll
            for (int d = 0; d < 2; ++d)
              if (nd == (uint32_t)d) {
#pragma unroll
                for (int q = 0; q < 4; ++q) dw[d][q] = xw[i][4 * h + q];
                des[d] = es;
                dpos[d] = 2u * (uint32_t)b + (uint32_t)h;
              }
          } else {
            const uint32_t c = exact_codes8(xv, 8 * h, es);
            if (h) hi = c; else lo = c;
          }
          ++nd;
        }
      }
      xcodes[b] = make_uint2(lo, hi);
      xsb[b] = (uint8_t)sb;
    }
    uint32_t* xcw = reinterpret_cast<uint32_t*>(xcodes);
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      if (__ballot(nd > (uint32_t)d) && nd > (uint32_t)d) {
        float x8[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          x8[2 * q] = __uint_as_float(dw[d][q] << 16);
          x8[2 * q + 1] = __uint_as_float(dw[d][q] & 0xFFFF0000u);
          x8[8 + 2 * q] = 0.0f;
          x8[9 + 2 * q] = 0.0f;
        }
        xcw[dpos[d]] = exact_codes8(x8, 0, des[d]);
      }
    }
  }
  // 3. the quantized rows complete and visible to every wave (the transfers
  //    in flight are not waited for: a bare barrier, no fence)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // The streaming loop.  Per chunk (256 k), MFMA H of each pair takes k
  // 128H .. 128H+127 of the chunk, lane group g k 32g .. 32g+31 of that
  // (weight piece 4H + g of the row), and output column c holds one
  // (activation row, block) pair:
  //   M = 1: block c of the chunk; both MFMAs accumulate into one tile, MFMA
  //          H filling columns 8H .. 8H+7;
  //   M = 2: row c / 8, block 8H + c % 8 (one MFMA per half);
  //   M = 3, 4: row c / 4, block 8H + 4Q + c % 4 (MFMAs Q = 0, 1 per half;
  //          a fourth row of zeros for M = 3).
  // The activation operand of lane (c, g) holds the codes of its column's
  // block in half (block % 2) of its 32 k when g = (block % 8) / 2, zeros
  // elsewhere (per-lane masks).  The products and their 16-term sums are
  // multiples of 1/4 below 600, exact in fp32, and so is each sum times the
  // two block scales (at most 12 + 4 + 4 significant bits): lane (c, g) adds
  // them to its partial sums of weight rows 4g .. 4g+3 in fp32 in a fixed
  // order, and the lanes of one activation row are added at the end in a
  // fixed tree.
  constexpr int kRM = kM == 1 ? 1 : (kM == 2 ? 2 : 4);  // activation rows per MFMA, padded
  constexpr int kBPM = kRM == 4 ? 4 : 8;                // blocks per activation row and MFMA
  constexpr int kQ = kRM == 4 ? 2 : 1;                  // MFMAs per 128-k half
  const uint32_t sw = (uint32_t)(l16 & 7);
  const uint32_t apos0 = (uint32_t)l16 * 128u + 16u * ((uint32_t)g ^ sw);
  const uint32_t apos1 = (uint32_t)l16 * 128u + 16u * ((4u + (uint32_t)g) ^ sw);
  const int mrow = kRM == 1 ? 0 : l16 / kBPM;           // this column's activation row
  const int bl = l16 % kBPM;                            // its block within the MFMA's set
  const int mc = mrow < kM ? mrow : kM - 1;             // clamped for addressing
  const int ql = kQ == 2 ? (g >> 1) : 0;                // the only MFMA of a half this lane feeds
  const bool act = mrow < kM && (kQ == 2 ? ((bl >> 1) == (g & 1)) : (g == (bl >> 1)));
  uint32_t mk[kRM == 1 ? 2 : kQ][2];
  if constexpr (kRM == 1) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 2; ++e) mk[h][e] = (act && (l16 >> 3) == h && (l16 & 1) == e) ? ~0u : 0u;
  } else {
#pragma unroll
    for (int q = 0; q < kQ; ++q)
#pragma unroll
      for (int e = 0; e < 2; ++e) mk[q][e] = (act && q == ql && (bl & 1) == e) ? ~0u : 0u;
  }
  const uint32_t xbase = (uint32_t)mc * NB + (uint32_t)(kRM == 1 ? l16 : kBPM * ql + bl);  // + 16c (+ 8H)
  const uint32_t sxbase = (uint32_t)mc * NB + (uint32_t)(kRM == 1 ? l16 : bl);           // + 16c (+ 8H + kBPM Q)
  const uint32_t srow = (uint32_t)(4 * g) * ks + (uint32_t)(kRM == 1 ? l16 : bl);       // + j ks + 16c (+ ...)
  float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < NCK; ++c) {
    const int d = c % D;
    wait_vmcnt<(D - 1) * 2>();
    const uint8_t* slot = ring + d * kGvChunkCodes;
    const uint4 a0 = *reinterpret_cast<const uint4*>(slot + apos0);
    const uint4 a1 = *reinterpret_cast<const uint4*>(slot + apos1);
    const i32x8 A[2] = {{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, 0, 0, 0, 0},
                        {(int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w, 0, 0, 0, 0}};
    if constexpr (kRM == 1) {
      const uint2 xv = xcodes[16 * c + xbase];
      const uint32_t xsc_b = xsb[16 * c + sxbase];
      uint32_t swb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) swb[j] = sc_lds[srow + (uint32_t)j * ks + 16u * (uint32_t)c];
      // the slot's reads are complete: refill it before computing, so the
      // transfer is not held back by this chunk's arithmetic
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(c + D, d);
      floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const i32x8 B = {(int)(xv.x & mk[h][0]), (int)(xv.y & mk[h][0]), (int)(xv.x & mk[h][1]),
                         (int)(xv.y & mk[h][1]), 0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[h], B, acc, 4, 4, 0, 127, 0, 127);
      }
      const float sx = __builtin_amdgcn_cvt_f32_fp8((int)xsc_b, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        part[j] = __builtin_fmaf(acc[j] * sx, __builtin_amdgcn_cvt_f32_fp8((int)(swb[j] & 0x7Fu), 0), part[j]);
    } else {
      uint2 xv[2];
      float sxf[2][kQ], swf[2][kQ][4];  // the E4M3 values of each MFMA's two block scales
#pragma unroll
      for (int h = 0; h < 2; ++h) xv[h] = xcodes[16 * c + 8 * h + xbase];
      if constexpr (kRM == 4) {
        // the chunk's 16 scale bytes of activation row mc and of weight rows
        // 4g .. 4g+3, one read each: the block of MFMA (H, Q) in this lane's
        // column is byte bl of dword 2H + Q
        const uint4 xr = *reinterpret_cast<const uint4*>(xsb + sxbase - bl + 16u * (uint32_t)c);
        uint4 wr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          wr[j] = *reinterpret_cast<const uint4*>(sc_lds + srow - bl + (uint32_t)j * ks + 16u * (uint32_t)c);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        // byte bl of dwords 2H and 2H + 1 side by side (one byte permute
        // with a per-lane selector), both decoded by one conversion
        const uint32_t sel = (uint32_t)bl | ((4u + (uint32_t)bl) << 8) | 0x0C0C0000u;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const auto x2 = __builtin_amdgcn_cvt_pk_f32_fp8(
              (int)__builtin_amdgcn_perm(dword_of(xr, 2 * h + 1), dword_of(xr, 2 * h), sel), false);
          sxf[h][0] = x2[0];
          sxf[h][1] = x2[1];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const auto w2 = __builtin_amdgcn_cvt_pk_f32_fp8(
                (int)(__builtin_amdgcn_perm(dword_of(wr[j], 2 * h + 1), dword_of(wr[j], 2 * h), sel) & 0x7F7Fu),
                false);
            swf[h][0][j] = w2[0];
            swf[h][1][j] = w2[1];
          }
        }
      } else {
        uint32_t xsc_b[2][kQ], swb[2][kQ][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int q = 0; q < kQ; ++q) {
            const uint32_t o = 16u * (uint32_t)c + 8u * (uint32_t)h + (uint32_t)(kBPM * q);
            xsc_b[h][q] = xsb[sxbase + o];
#pragma unroll
            for (int j = 0; j < 4; ++j) swb[h][q][j] = sc_lds[srow + (uint32_t)j * ks + o];
          }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int q = 0; q < kQ; ++q) {
            sxf[h][q] = __builtin_amdgcn_cvt_f32_fp8((int)xsc_b[h][q], 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) swf[h][q][j] = __builtin_amdgcn_cvt_f32_fp8((int)(swb[h][q][j] & 0x7Fu), 0);
          }
      }
      issue(c + D, d);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
          const i32x8 B = {(int)(xv[h].x & mk[q][0]), (int)(xv[h].y & mk[q][0]), (int)(xv[h].x & mk[q][1]),
                           (int)(xv[h].y & mk[q][1]), 0, 0, 0, 0};
          const floatx4 acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              A[h], B, floatx4{0.0f, 0.0f, 0.0f, 0.0f}, 4, 4, 0, 127, 0, 127);
#pragma unroll
          for (int j = 0; j < 4; ++j) part[j] = __builtin_fmaf(acc[j] * sxf[h][q], swf[h][q][j], part[j]);
        }
    }
  }
  wait_vmcnt<0>();
  // weight rows 4g .. 4g+3: the lanes of one activation row (M = 1: all 16
  // of the row group), added in a fixed tree
#pragma unroll
  for (int o = (kRM == 1 ? 16 : kBPM) / 2; o > 0; o >>= 1)
#pragma unroll
    for (int j = 0; j < 4; ++j) part[j] += __shfl_xor(part[j], o, 64);
  if (bl == 0 && (kRM == 1 ? l16 == 0 : mrow < kM) && tile_raw < tiles) {
    const float scale = gs * (*gsw_p);
    store4<kYBf16>(y + (size_t)mrow * ldy, n0 + 4 * g, N, part[0] * scale, part[1] * scale, part[2] * scale,
                   part[3] * scale);
  }
  // 4. the quantized rows for the workspace: fp16 values E2M1 * E4M3, codes
  //    and scale bytes, tensor scale
  if constexpr (kMode != kFuPrepared) {
    if (blockIdx.x == 0) {
      for (int i = (int)threadIdx.x; i < kM * K / 8; i += 64 * kW) {
        const uint2 cw = xcodes[i >> 1];
        uint32_t e[4];
        expand8((i & 1) ? cw.y : cw.x, scale_f16x2(xsb[i >> 1]), e);
        x16_out[i] = make_uint4(e[0], e[1], e[2], e[3]);
      }
      for (int i = (int)threadIdx.x; i < (int)kQBytes / 16; i += 64 * kW)
        reinterpret_cast<uint4*>(q_out)[i] = reinterpret_cast<const uint4*>(xrow)[i];
      if (threadIdx.x == 0) *gsx_out = gs;
    }
  }
}

static size_t fp4_lds(int64_t M, int64_t K, bool prepared, int W) {
  const size_t kh = (size_t)K / 2, ks = (size_t)K / 16;
  const size_t row = (!prepared && M == 1) ? (size_t)K * 2u : ((size_t)M * (kh + ks) + 1023u) / 1024u * 1024u;
  return row + (size_t)W * kFuDepth * kGvChunkCodes +
         (size_t)W * ((16u * ks + 1023u) / 1024u * 1024u) +  // 16 rows of K/16 scale bytes
         4u * kFuMaxWaves;                                           // the waves' maxima
}

template <int kMode>
static void fp4_go(int64_t M, int64_t K, const void* x, size_t ldx, const float* gs_in, const uint8_t* wc,
                   const uint8_t* ws, int64_t N, const float* gsw, void* y, bool y_bf16, size_t ldy,
                   void* x16_out, float* gsx_out, uint8_t* q_out, hipStream_t s) {
  const int tiles = (int)((N + 15) / 16);
  auto go = [&](auto nc, auto m, auto yb) {
    constexpr int W = fp4_waves(decltype(m)::value);
    const int grid = (tiles + W - 1) / W;
    const size_t lds = fp4_lds(M, K, kMode == kFuPrepared, W);
    gemv_fp4_kernel<decltype(nc)::value, decltype(m)::value, W, kMode, decltype(yb)::value>
        <<<grid, 64 * W, lds, s>>>((const uint8_t*)x, ldx, gs_in, wc, ws, (int)N, tiles, gsw, (uint8_t*)y, ldy,
                                   (uint4*)x16_out, gsx_out, q_out);
  };
  auto by_y = [&](auto nc, auto m) {
    if (y_bf16) go(nc, m, std::true_type());
    else go(nc, m, std::false_type());
  };
  auto by_m = [&](auto nc) {
    switch (M) {
      case 1: by_y(nc, std::integral_constant<int, 1>()); break;
      case 2: by_y(nc, std::integral_constant<int, 2>()); break;
      case 3: by_y(nc, std::integral_constant<int, 3>()); break;
      default: by_y(nc, std::integral_constant<int, 4>()); break;
    }
  };
  if (K == 5120) by_m(std::integral_constant<int, 20>());
  else by_m(std::integral_constant<int, 16>());
}

// One-launch decode step for up to four bf16 rows when the shape has an
// instantiation; false otherwise (nothing launched: the caller quantizes and
// runs the GEMV in two launches).
bool launch_gemv_fp4(const void* x, bool x_bf16, int64_t M, int64_t K, size_t ldx_bytes, const float* gs_in,
                     const uint8_t* wc, const uint8_t* ws, int64_t N, const float* gsw, void* y, bool y_bf16,
                     size_t ldy_bytes, void* x16_out, float* gsx_out, uint8_t* q_out, hipStream_t s) {
  if (!x_bf16 || !gemv_fp4_has_form(M, K)) return false;
  if (gs_in)
    fp4_go<kFuGiven>(M, K, x, ldx_bytes, gs_in, wc, ws, N, gsw, y, y_bf16, ldy_bytes, x16_out, gsx_out, q_out, s);
  else
    fp4_go<kFuDynamic>(M, K, x, ldx_bytes, gs_in, wc, ws, N, gsw, y, y_bf16, ldy_bytes, x16_out, gsx_out, q_out,
                       s);
  return true;
}

// The GEMV for up to four prepared rows (codes [M][K/2] at q, scale bytes
// [M][K/16] after them, tensor scale *gsx) when the shape has an
// instantiation; false otherwise.
bool launch_gemv_fp4_prepared(const uint8_t* q, int64_t M, int64_t K, const float* gsx, const uint8_t* wc,
                              const uint8_t* ws, int64_t N, const float* gsw, void* y, bool y_bf16,
                              size_t ldy_bytes, hipStream_t s) {
  if (!gemv_fp4_has_form(M, K)) return false;
  fp4_go<kFuPrepared>(M, K, q, 0, gsx, wc, ws, N, gsw, y, y_bf16, ldy_bytes, nullptr, nullptr, nullptr, s);
  return true;
}

// ------------------------------------------------------------ 4 < M <= 16
// With more activation rows the activation operand outweighs the weights
// (16 rows of fp16 against 16 rows of 4-bit codes), so the activations are
// shared: a workgroup of 8 waves owns 128 rows of W (16 per wave) and all
// waves read one copy of each activation chunk from LDS.  K advances 256 per
// step through a ring of three stages, one barrier per step, transfers of
// step kt+2 in flight while step kt is computed.  Every wave issues the same
// four transfers per step: its 16 rows of codes (two transfers of 8 rows x
// 128 B), its 16 rows of scale bytes (16 lanes x 16 B) and two activation
// rows (rows past M repeat row M-1; their lanes never read them).  The
// per-lane computation is the one of the kernel above.
constexpr int kGwWaves = 8;
struct GwStage {
  uint4 codes[128 * 8];  // 16 KB: [row][8 slots]
  uint4 scales[128];     //  2 KB: [row] 16 scale bytes
  uint4 x[16 * 32];      //  8 KB: [m][32 slots]
};

template <bool kA16, bool kYBf16>
__global__ __launch_bounds__(512) void gemv_shared_kernel(const uint8_t* __restrict__ x16, uint32_t ld_x16_bytes,
                                                          int M, const uint8_t* __restrict__ wc,
                                                          const uint8_t* __restrict__ ws, int N, int K,
                                                          const float* __restrict__ gsx_p,
                                                          const float* __restrict__ gsw_p,
                                                          uint8_t* __restrict__ y, size_t ld_y_bytes) {
  using O = Op<kA16>;
  __shared__ GwStage st0, st1, st2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
  const int tile = blockIdx.x * kGwWaves + wave;  // 16-row tile of this wave
  const uint32_t kh = (uint32_t)K / 2, ks = (uint32_t)K / 16;
  const int nk = K >> 8;

  // transfer offsets (fixed; + 128 B codes, 16 B scales, 512 B activations per step)
  uint32_t coff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 8 * h + (lane >> 3);
    int n = tile * 16 + r;
    n = n < N ? n : N - 1;
    coff[h] = (uint32_t)n * kh + 16u * (uint32_t)((lane & 7) ^ (r & 7));
  }
  uint32_t soff;
  {
    int n = tile * 16 + l16;
    n = n < N ? n : N - 1;
    soff = (uint32_t)n * ks;
  }
  uint32_t xoff;
  {
    int m = 2 * wave + (lane >> 5);
    m = m < M ? m : M - 1;
    const uint32_t p = (uint32_t)(lane & 31), piece = (p & ~7u) | ((p & 7u) ^ (p >> 3));
    xoff = (uint32_t)m * ld_x16_bytes + 16u * piece;
  }
  const uint32_t lc[3] = {lds_addr(&st0.codes[wave * 128]), lds_addr(&st1.codes[wave * 128]),
                          lds_addr(&st2.codes[wave * 128])};
  const uint32_t lsc[3] = {lds_addr(&st0.scales[wave * 16]), lds_addr(&st1.scales[wave * 16]),
                           lds_addr(&st2.scales[wave * 16])};
  const uint32_t lxx[3] = {lds_addr(&st0.x[wave * 64]), lds_addr(&st1.x[wave * 64]),
                           lds_addr(&st2.x[wave * 64])};
  auto issue = [&](int kt, int b) {
    kt = kt < nk ? kt : nk - 1;  // past the end: repeat the last step into a stage no longer read
    lds_dma16(wc, coff[0] + (uint32_t)kt * 128u, lc[b]);
    lds_dma16(wc, coff[1] + (uint32_t)kt * 128u, lc[b] + 1024u);
    if (lane < 16) lds_dma16(ws, soff + (uint32_t)kt * 16u, lsc[b]);
    lds_dma16(x16, xoff + (uint32_t)kt * 512u, lxx[b]);
  };

  const bool mvalid = l16 < M;
  const uint32_t sw = (uint32_t)(l16 & 7), xg = (uint32_t)g;
  const int crow = wave * 16 + l16;
  const uint32_t cpos0 = (uint32_t)crow * 8u + ((2u * g) ^ sw), cpos1 = (uint32_t)crow * 8u + ((2u * g + 1u) ^ sw);
  uint4 xv[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) xv[t] = make_uint4(0, 0, 0, 0);
  floatx4 acc = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](const GwStage& S) {
    const uint4 w0 = S.codes[cpos0], w1 = S.codes[cpos1];
    const uint32_t sd = reinterpret_cast<const uint32_t*>(&S.scales[crow])[g];
    if (mvalid) {
      const uint4* xr = &S.x[l16 * 32 + 8 * g];
#pragma unroll
      for (int t = 0; t < 8; ++t) xv[t] = xr[(uint32_t)t ^ xg];
    }
    const uint32_t s0 = O::scale_bits(sd), s1 = O::scale_bits(sd >> 8), s2 = O::scale_bits(sd >> 16),
                   s3 = O::scale_bits(sd >> 24);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t sp = t < 2 ? s0 : (t < 4 ? s1 : (t < 6 ? s2 : s3));
      uint32_t e[4];
      O::expand(dword_of(t < 4 ? w0 : w1, t & 3), sp, e);
      acc = O::mfma16(O::vec(make_uint4(e[0], e[1], e[2], e[3])), O::vec(xv[t]), acc);
    }
  };
  // Step kt: wait for this wave's transfers of step kt (those of kt+1 may
  // still fly), barrier (everyone's have landed, and everyone is done with
  // the stage of step kt-1), issue step kt+2 into that stage, compute.
  auto step = [&](int kt, const GwStage& S, int nb) {
    asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    issue(kt + 2, nb);
    compute(S);
  };

  issue(0, 0);
  issue(1, 1);
  for (int kt = 0; kt < nk; kt += 3) {
    step(kt, st0, 2);
    if (kt + 1 < nk) step(kt + 1, st1, 0);
    if (kt + 2 < nk) step(kt + 2, st2, 1);
  }
  wait_vmcnt<0>();
  const float scale = kA16 ? *gsw_p : (*gsx_p) * (*gsw_p);
  if (mvalid)
    store4<kYBf16>(y + (size_t)l16 * ld_y_bytes, tile * 16 + 4 * g, N, acc[0] * scale, acc[1] * scale,
                   acc[2] * scale, acc[3] * scale);
}

// Cross-lane exchanges of gfx950, per 32-bit word of a 16-byte value:
// swap_lanes32(u, v) swaps the upper 32 lanes of u with the lower 32 lanes
// of v; swap_rows16(u, v) swaps the odd 16-lane rows of u with the even rows
// of v.
__device__ __forceinline__ void swap_lanes32(uint4& u, uint4& v) {
  auto x = __builtin_amdgcn_permlane32_swap(u.x, v.x, false, false);
  auto y = __builtin_amdgcn_permlane32_swap(u.y, v.y, false, false);
  auto z = __builtin_amdgcn_permlane32_swap(u.z, v.z, false, false);
  auto w = __builtin_amdgcn_permlane32_swap(u.w, v.w, false, false);
  u = make_uint4(x[0], y[0], z[0], w[0]);
  v = make_uint4(x[1], y[1], z[1], w[1]);
}
__device__ __forceinline__ void swap_rows16(uint4& u, uint4& v) {
  auto x = __builtin_amdgcn_permlane16_swap(u.x, v.x, false, false);
  auto y = __builtin_amdgcn_permlane16_swap(u.y, v.y, false, false);
  auto z = __builtin_amdgcn_permlane16_swap(u.z, v.z, false, false);
  auto w = __builtin_amdgcn_permlane16_swap(u.w, v.w, false, false);
  u = make_uint4(x[0], y[0], z[0], w[0]);
  v = make_uint4(x[1], y[1], z[1], w[1]);
}

// ---------------------------------------------------------- K split (M <= 16)
// A workgroup of K/512 waves covers all of K for a run of 16-row tiles: wave
// w owns k [512w, 512w + 512) and keeps the activations of that slice in
// registers for the whole kernel (16 rows x 512 k of fp16: 64 registers a
// lane), so the activations are read once per workgroup.  The weights of
// the wave's slice stream through a ring of three LDS slots by direct
// global->LDS transfers with explicit waits (as in the streaming kernel):
// per tile, the codes (16 rows x 256 B, four transfers of 4 rows x 256 B,
// code piece p of row r in slot p ^ (r & 7) of its row) and the scales (16
// rows x 32 B, one 32-lane gather).  Lane (r, g) takes k 128g .. 128g+127 of
// the slice: 64 code bytes and 8 scale bytes; MFMA step s (16x16x32) uses
// dword s of the codes, and the activation operand holds the same k.  Per
// tile the slices' partial sums meet in LDS; wave (tile index mod waves)
// adds them in wave order and keeps the result in registers until the end,
// so nothing but the transfers touches memory inside the loop and the result
// does not depend on scheduling.
constexpr int kKsMaxWaves = 10;     // K <= 5120
constexpr int kKsMaxResults = 4;    // tiles a wave reduces (bounded by the grid)
constexpr uint32_t kKsSlot = 4096 + 512;  // codes + scales of one wave and tile

template <bool kA16, bool kYBf16>
__global__ __launch_bounds__(640) void gemv_ksplit_kernel(const uint8_t* __restrict__ x16, uint32_t ld_x16_bytes,
                                                          int M, const uint8_t* __restrict__ wc,
                                                          const uint8_t* __restrict__ ws, int N, int K,
                                                          int tiles, const float* __restrict__ gsx_p,
                                                          const float* __restrict__ gsw_p,
                                                          uint8_t* __restrict__ y, size_t ld_y_bytes) {
  using O = Op<kA16>;
  __shared__ __attribute__((aligned(16))) uint8_t ring[3][kKsMaxWaves][kKsSlot];
  __shared__ floatx4 part[2][kKsMaxWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
  const int waves = blockDim.x >> 6;
  const uint32_t ks0 = (uint32_t)wave * 512u;                 // slice start
  const uint32_t kh = (uint32_t)K / 2, ks = (uint32_t)K / 16;
  const bool mvalid = l16 < M;

  // activations of the slice, loaded unconditionally (rows m >= M read row 0
  // and are zeroed), all before the first transfer.  Lane (r, g) needs the
  // 16-byte pieces 16g .. 16g+15 of row r's slice (xv[s] = piece 16g + s).
  // Loaded that way, each load instruction would touch 64 lines; instead
  // load q reads piece 4q + g, so the four lanes of a row read 64 contiguous
  // bytes, and the pieces are then moved to their lanes in registers.
  // Writing q = 4a + b, lane g holds piece (a, b, g) (= 16a + 4b + g) in
  // register q; exchanging the lane index g with the register field a (a
  // 4 x 4 transpose over the rows of 16 lanes: bit 1 by swapping the upper
  // 32 lanes of one register with the lower 32 of another, bit 0 by swapping
  // odd 16-lane rows with even ones) leaves piece (g, b, c) in register
  // 4c + b of lane g, which is xv[4b + c].
  uint4 xv[16];
  {
    const uint8_t* xr = x16 + (size_t)(mvalid ? l16 : 0) * ld_x16_bytes + ks0 * 2u + 16u * (uint32_t)g;
    uint4 L[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) L[q] = *reinterpret_cast<const uint4*>(xr + 64u * q);
#pragma unroll
    for (int q = 0; q < 16; ++q) L[q] = mvalid ? L[q] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int a0 = 0; a0 < 2; ++a0)
#pragma unroll
      for (int b = 0; b < 4; ++b) swap_lanes32(L[4 * a0 + b], L[4 * (2 + a0) + b]);
#pragma unroll
    for (int a1 = 0; a1 < 2; ++a1)
#pragma unroll
      for (int b = 0; b < 4; ++b) swap_rows16(L[8 * a1 + b], L[8 * a1 + 4 + b]);
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int c = 0; c < 4; ++c) xv[4 * b + c] = L[4 * c + b];
  }

  // transfer offsets within a tile (+ 16 rows of W per tile)
  uint32_t coff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t r = 4u * q + (uint32_t)(lane >> 4), p = (uint32_t)(lane & 15);
    coff[q] = r * kh + (ks0 >> 1) + 16u * (p ^ (r & 7u));
  }
  const uint32_t soff = (uint32_t)(lane >> 1) * ks + (ks0 >> 4) + 16u * (uint32_t)(lane & 1);
  const uint32_t lr0 = lds_addr(&ring[0][wave][0]);
  constexpr uint32_t kSlotStride = kKsMaxWaves * kKsSlot;  // between ring slots
  const int first = blockIdx.x, step = gridDim.x;
  auto issue = [&](int t, int b) {
    t = t < tiles ? t : tiles - 1;  // past the end: repeat the last tile into a slot not read again
    const uint32_t rows = (uint32_t)t * 16u;
    const uint32_t dst = lr0 + (uint32_t)b * kSlotStride;
    const int last = N - 1;
    // rows past N repeat row N-1 (their sums are never stored)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t r = 4u * q + (uint32_t)(lane >> 4);
      const uint32_t n = rows + r < (uint32_t)N ? rows + r : (uint32_t)last;
      lds_dma16(wc, coff[q] + (n - r) * kh, dst + 1024u * q);
    }
    if (lane < 32) {
      const uint32_t r = (uint32_t)(lane >> 1);
      const uint32_t n = rows + r < (uint32_t)N ? rows + r : (uint32_t)last;
      lds_dma16(ws, soff + (n - r) * ks, dst + 4096u);
    }
  };

  const float scale = kA16 ? *gsw_p : (*gsx_p) * (*gsw_p);
  const uint32_t sw = (uint32_t)(l16 & 7);
  floatx4 res[kKsMaxResults];
  int res_tile[kKsMaxResults];
#pragma unroll
  for (int r = 0; r < kKsMaxResults; ++r) res_tile[r] = -1;
  int nres = 0;

  auto compute = [&](int t, int b, int pb, int local) {
    const uint8_t* slot = &ring[b][wave][0];
    uint4 w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = *reinterpret_cast<const uint4*>(slot + l16 * 256 + 16 * (((uint32_t)(4 * g + q)) ^ sw));
    const uint2 sc = *reinterpret_cast<const uint2*>(slot + 4096 + l16 * 32 + 8 * g);
    floatx4 acc = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const uint32_t sb = (s < 8 ? sc.x : sc.y) >> (8 * ((s >> 1) & 3));
      uint32_t e[4];
      O::expand(dword_of(w[s >> 2], s & 3), O::scale_bits(sb), e);
      acc = O::mfma16(O::vec(make_uint4(e[0], e[1], e[2], e[3])), O::vec(xv[s]), acc);
    }
    part[pb][wave][lane] = acc;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (wave == local % waves) {
      floatx4 sum = part[pb][0][lane];
      for (int v = 1; v < waves; ++v) sum = sum + part[pb][v][lane];
#pragma unroll
      for (int r = 0; r < kKsMaxResults; ++r)
        if (r == nres) {
          res[r] = sum;
          res_tile[r] = t;
        }
      ++nres;
    }
  };

  // ring: slot b of tile i is i % 3; tile i+2 goes out once every wave is
  // past tile i-1 (the barrier in tile i's step)
  issue(first, 0);
  issue(first + step, 1);
  int local = 0;
  for (int t = first; t < tiles; t += 3 * step) {
    wait_vmcnt<5>();
    issue(t + 2 * step, 2);
    compute(t, 0, local & 1, local);
    ++local;
    if (t + step >= tiles) break;
    wait_vmcnt<5>();
    issue(t + 3 * step, 0);
    compute(t + step, 1, local & 1, local);
    ++local;
    if (t + 2 * step >= tiles) break;
    wait_vmcnt<5>();
    issue(t + 4 * step, 1);
    compute(t + 2 * step, 2, local & 1, local);
    ++local;
  }
  wait_vmcnt<0>();
  if (mvalid) {
#pragma unroll
    for (int r = 0; r < kKsMaxResults; ++r)
      if (res_tile[r] >= 0)
        store4<kYBf16>(y + (size_t)l16 * ld_y_bytes, res_tile[r] * 16 + 4 * g, N, res[r][0] * scale,
                       res[r][1] * scale, res[r][2] * scale, res[r][3] * scale);
  }
}

// ------------------------------------------------------------ FP8 weights
// W8A16 / W8A8 GEMV (M <= 16; model card "Gemma-4-31B-IT-NVFP4-FP8attn-
// text", section "What was quantized, exactly": float8_e4m3 weights with one
// per-tensor scale, served against bf16 activations).  W is [N, K] E4M3
// bytes.  A workgroup of ceil(K / 512) waves covers all of K for a run of
// 16-row tiles (as the K-split kernel above; K <= 5120): wave w owns k [512w, 512w+512)
// and keeps the activations of that slice in registers.  Lane (r, g) takes
// 128 k of row r, interleaved with the other three lanes of the row so that
// each load instruction reads 64 contiguous bytes of W per row (16-byte
// pieces: piece 4q + g of the slice is the lane's load q); the activations
// follow the same k order, which is any order as long as both operands share
// it.  The weights of a tile (128 bytes a lane) go
// straight to registers, the next tile's while the current one is computed
// (two register sets, used alternately).  Past K the activations are zero.  The
// partial tiles of the waves are added in LDS in wave order (one barrier a
// tile, double-buffered), so the result does not depend on scheduling.
//   kA8 = false: bf16 activations; W bytes become bf16 pairs (exact) for
//     16 MFMA 16x16x32 bf16 steps of 8 k.
//   kA8 = true: FP8 activations; 4 MFMA 16x16x128 FP8 steps of 32 k, both
//     operands unconverted (unit block scales).
constexpr int kF8MaxWaves = 10;    // K <= 5120 (wider K takes the tile kernel)

template <bool kA8, bool kYBf16>
__global__ __launch_bounds__(640) void gemv_fp8w_kernel(const uint8_t* __restrict__ x, uint32_t ld_x_bytes, int M,
                                                         const uint8_t* __restrict__ wq, int N, int K, int tiles,
                                                         const float* __restrict__ sx_p,
                                                         const float* __restrict__ sw_p, uint8_t* __restrict__ y,
                                                         size_t ld_y_bytes) {
  __shared__ floatx4 part[2][kF8MaxWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
  const int waves = blockDim.x >> 6;
  const bool mvalid = l16 < M;
  // k of the lane's W load q (16 weights): piece 4q + g of the wave's slice.
  // kA8: MFMA step s takes loads 2s and 2s+1 (32 k), so those are pieces
  // 8s + 2g and 8s + 2g + 1, i.e. 32-k pieces 4s + g.
  auto wk = [&](int q) {
    return wave * 512 + (kA8 ? 32 * (4 * (q >> 1) + g) + 16 * (q & 1) : 16 * (4 * q + g));
  };

  // activations of the slice in the same k order (zeros past K and for
  // m >= M): kA8: 16 FP8 values per load, as W; bf16: MFMA step s (8 k) is
  // half s & 1 of W load s >> 1
  constexpr int kXq = kA8 ? 8 : 16;  // uint4 per lane
  uint4 xv[kXq];
  {
    const uint8_t* xr = x + (size_t)(mvalid ? l16 : 0) * ld_x_bytes;
#pragma unroll
    for (int q = 0; q < kXq; ++q) {
      const int kq = kA8 ? wk(q) : wk(q >> 1) + 8 * (q & 1);
      xv[q] = (mvalid && kq < K) ? *reinterpret_cast<const uint4*>(xr + (size_t)kq * (kA8 ? 1u : 2u))
                                 : make_uint4(0, 0, 0, 0);
    }
  }

  auto load_w = [&](int t, uint4 (&w)[8]) {
    t = t < tiles ? t : tiles - 1;  // past the end: a valid tile whose sums are never used
    int n = t * 16 + l16;
    n = n < N ? n : N - 1;
    // k past K re-reads the row's last 16 bytes: finite weights that meet
    // zero activations, so every load is unconditional
    const uint8_t* wr = wq + (size_t)n * (size_t)K;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int kq = wk(q) < K ? wk(q) : K - 16;
      w[q] = *reinterpret_cast<const uint4*>(wr + kq);
    }
  };
  auto mma = [&](const uint4 (&w)[8]) {
    floatx4 acc = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (kA8) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 wa[2] = {w[2 * s], w[2 * s + 1]};
        const uint4 xa[2] = {xv[2 * s], xv[2 * s + 1]};
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(__builtin_bit_cast(i32x8, wa),
                                                                __builtin_bit_cast(i32x8, xa), acc, 0, 0, 0, 127, 0,
                                                                127);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const uint32_t d0 = dword_of(w[s >> 1], 2 * (s & 1)), d1 = dword_of(w[s >> 1], 2 * (s & 1) + 1);
        const uint4 e = make_uint4(
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true)));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, e),
                                                      __builtin_bit_cast(bf16x8, xv[s]), acc, 0, 0, 0);
      }
    }
    return acc;
  };

  const float scale = kA8 ? (*sx_p) * (*sw_p) : *sw_p;
  int local = 0;
  // the wave whose turn it is adds the partial tiles in wave order and
  // stores the tile's outputs
  auto finish = [&](int t, const floatx4& acc) {
    const int pb = local & 1;
    part[pb][wave][lane] = acc;
    __syncthreads();
    if (wave == local % waves && mvalid) {
      floatx4 sum = part[pb][0][lane];
      for (int v = 1; v < waves; ++v) sum = sum + part[pb][v][lane];
      store4<kYBf16>(y + (size_t)l16 * ld_y_bytes, t * 16 + 4 * g, N, sum[0] * scale, sum[1] * scale,
                     sum[2] * scale, sum[3] * scale);
    }
    ++local;
  };

  const int first = blockIdx.x, step = gridDim.x;
  uint4 wa[8], wb[8];
  load_w(first, wa);
  for (int t = first; t < tiles; t += 2 * step) {
    load_w(t + step, wb);
    finish(t, mma(wa));
    if (t + step >= tiles) break;
    load_w(t + 2 * step, wa);
    finish(t + step, mma(wb));
  }
}

// FP8 weights, M <= 4: one wave per 16-row tile over all of K, as the NVFP4
// streaming kernel.  Chunks of 256 k reach LDS through a ring of D slots by
// direct transfers with explicit waits: the weights (16 rows x 256 B, four
// transfers of 4 rows; piece p of row r in slot p ^ r of its row) and the
// activations (bf16: M rows x 512 B, two transfers of 2 rows, piece 8a + b in
// slot 8a + (b ^ a); FP8: M rows x 256 B, one transfer of 4 rows).  Lane
// (r, g) takes k 64g .. 64g+63 of weight row r: eight bf16 MFMA steps of 8 k
// (W8A16) or two FP8 steps of 32 k (W8A8), the activation operand read with
// the same k.  Partial sums stay in the wave.
constexpr uint32_t kF8Chunk = 4096;

template <int D, bool kA8, bool kYBf16>
__global__ __launch_bounds__(64) void gemv_fp8w_stream_kernel(const uint8_t* __restrict__ x, uint32_t ld_x_bytes,
                                                               int M, const uint8_t* __restrict__ wq, int N, int K,
                                                               const float* __restrict__ sx_p,
                                                               const float* __restrict__ sw_p,
                                                               uint8_t* __restrict__ y, size_t ld_y_bytes) {
  extern __shared__ uint4 smem[];
  constexpr int kXI = kA8 ? 1 : 2;                       // activation transfers per chunk
  constexpr uint32_t kSlot = kF8Chunk + 1024u * kXI;
  uint8_t* lds = reinterpret_cast<uint8_t*>(smem);
  const int lane = threadIdx.x, l16 = lane & 15, g = lane >> 4;
  const int tile = blockIdx.x;
  const int nck = K >> 8;  // a multiple of D
  const uint32_t ring0 = lds_addr(lds);

  uint32_t woff[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int r = 4 * h + (lane >> 4);
    int n = tile * 16 + r;
    n = n < N ? n : N - 1;
    woff[h] = (uint32_t)n * (uint32_t)K + 16u * (uint32_t)((lane & 15) ^ r);
  }
  uint32_t xoff[kXI];
#pragma unroll
  for (int v = 0; v < kXI; ++v) {
    if constexpr (kA8) {
      int m = lane >> 4;
      m = m < M ? m : M - 1;
      xoff[v] = (uint32_t)m * ld_x_bytes + 16u * (uint32_t)(lane & 15);
    } else {
      int m = 2 * v + (lane >> 5);
      m = m < M ? m : M - 1;
      const uint32_t p = (uint32_t)(lane & 31), piece = (p & ~7u) | ((p & 7u) ^ (p >> 3));
      xoff[v] = (uint32_t)m * ld_x_bytes + 16u * piece;
    }
  }
  int next = 0;
  auto issue = [&](int d) {
    const int c = next < nck ? next : nck - 1;  // past the end: repeat the last chunk into a slot not read again
    const uint32_t slot = ring0 + (uint32_t)d * kSlot;
#pragma unroll
    for (int h = 0; h < 4; ++h) lds_dma16(wq, woff[h] + (uint32_t)c * 256u, slot + 1024u * h);
#pragma unroll
    for (int v = 0; v < kXI; ++v)
      lds_dma16(x, xoff[v] + (uint32_t)c * (kA8 ? 256u : 512u), slot + kF8Chunk + 1024u * v);
    ++next;
  };
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d);

  const bool mvalid = l16 < M;
  const float scale = kA8 ? (*sx_p) * (*sw_p) : *sw_p;
  floatx4 acc = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int c0 = 0; c0 < nck; c0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      wait_vmcnt<(D - 1) * (4 + kXI)>();
      const uint8_t* slot = lds + d * kSlot;
      uint4 w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = *reinterpret_cast<const uint4*>(slot + l16 * 256 + 16 * ((4 * g + j) ^ l16));
      if constexpr (kA8) {
        uint4 xa[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0),
                       make_uint4(0, 0, 0, 0)};
        if (mvalid) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            xa[j] = *reinterpret_cast<const uint4*>(slot + kF8Chunk + l16 * 256 + 16 * (4 * g + j));
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint4 wa[2] = {w[2 * t], w[2 * t + 1]};
          const uint4 xb[2] = {xa[2 * t], xa[2 * t + 1]};
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(__builtin_bit_cast(i32x8, wa),
                                                                  __builtin_bit_cast(i32x8, xb), acc, 0, 0, 0, 127, 0,
                                                                  127);
        }
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          uint4 xv = make_uint4(0, 0, 0, 0);
          if (mvalid)
            xv = *reinterpret_cast<const uint4*>(slot + kF8Chunk + l16 * 512 + 128 * g + 16 * (t ^ g));
          const uint32_t d0 = dword_of(w[t >> 1], 2 * (t & 1)), d1 = dword_of(w[t >> 1], 2 * (t & 1) + 1);
          const uint4 e = make_uint4(
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true)));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, e), __builtin_bit_cast(bf16x8, xv),
                                                        acc, 0, 0, 0);
        }
      }
      issue(d);
    }
  }
  wait_vmcnt<0>();
  if (mvalid)
    store4<kYBf16>(y + (size_t)l16 * ld_y_bytes, tile * 16 + 4 * g, N, acc[0] * scale, acc[1] * scale,
                   acc[2] * scale, acc[3] * scale);
}

template <bool kA8>
static bool gemv_fp8w_stream_go(const void* x, uint32_t ldx, int64_t M, int64_t K, const uint8_t* wq, int64_t N,
                                const float* sx, const float* sw, void* y, bool y_bf16, size_t ldb, int cus,
                                hipStream_t s) {
  // the deepest ring (4 or 2 slots, dividing the chunk count) whose
  // workgroups all fit on the machine at once
  const int tiles = (int)((N + 15) / 16);
  const int nck = (int)(K / 256);
  const size_t slot = kF8Chunk + 1024u * (kA8 ? 1 : 2);
  int depth = 0;
  for (int d : {4, 2}) {
    if (nck % d) continue;
    const int64_t per_cu = (int64_t)(160 * 1024) / (int64_t)(d * slot);
    if (per_cu * cus < tiles && d > 2) continue;
    depth = d;
    break;
  }
  if (!depth) return false;
  const size_t lds = (size_t)depth * slot;
  auto go = [&](auto dc) {
    constexpr int D = decltype(dc)::value;
    if (y_bf16)
      gemv_fp8w_stream_kernel<D, kA8, true><<<tiles, 64, lds, s>>>((const uint8_t*)x, ldx, (int)M, wq, (int)N, (int)K,
                                                                  sx, sw, (uint8_t*)y, ldb);
    else
      gemv_fp8w_stream_kernel<D, kA8, false><<<tiles, 64, lds, s>>>((const uint8_t*)x, ldx, (int)M, wq, (int)N,
                                                                   (int)K, sx, sw, (uint8_t*)y, ldb);
  };
  if (depth == 4) go(std::integral_constant<int, 4>());
  else go(std::integral_constant<int, 2>());
  return true;
}

void launch_gemv_fp8w(bool a8, const void* x, size_t ld_x_bytes, int64_t M, int64_t K, const uint8_t* wq, int64_t N,
                      const float* sx, const float* sw, void* y, bool y_bf16, int64_t ld_y, hipStream_t s) {
  int cus = 0, lds_cu = 0;
  if (!device_caps(cus, lds_cu)) cus = 256;
  if (M <= 4 && K >= 256 && K % 256 == 0) {
    const size_t ldb4 = (size_t)ld_y * (y_bf16 ? 2u : 4u);
    const bool done = a8 ? gemv_fp8w_stream_go<true>(x, (uint32_t)ld_x_bytes, M, K, wq, N, sx, sw, y, y_bf16, ldb4,
                                                     cus, s)
                         : gemv_fp8w_stream_go<false>(x, (uint32_t)ld_x_bytes, M, K, wq, N, sx, sw, y, y_bf16, ldb4,
                                                      cus, s);
    if (done) return;
  }
  const int tiles = (int)((N + 15) / 16);
  const int waves = (int)((K + 511) / 512);
  const int grid = tiles < cus ? tiles : cus;
  const size_t ldb = (size_t)ld_y * (y_bf16 ? 2u : 4u);
  const uint32_t ldx = (uint32_t)ld_x_bytes;
  if (a8) {
    if (y_bf16)
      gemv_fp8w_kernel<true, true><<<grid, waves * 64, 0, s>>>((const uint8_t*)x, ldx, (int)M, wq, (int)N, (int)K,
                                                              tiles, sx, sw, (uint8_t*)y, ldb);
    else
      gemv_fp8w_kernel<true, false><<<grid, waves * 64, 0, s>>>((const uint8_t*)x, ldx, (int)M, wq, (int)N, (int)K,
                                                               tiles, sx, sw, (uint8_t*)y, ldb);
  } else {
    if (y_bf16)
      gemv_fp8w_kernel<false, true><<<grid, waves * 64, 0, s>>>((const uint8_t*)x, ldx, (int)M, wq, (int)N, (int)K,
                                                               tiles, sx, sw, (uint8_t*)y, ldb);
    else
      gemv_fp8w_kernel<false, false><<<grid, waves * 64, 0, s>>>((const uint8_t*)x, ldx, (int)M, wq, (int)N,
                                                                (int)K, tiles, sx, sw, (uint8_t*)y, ldb);
  }
}

// LDS of one streaming workgroup, and the depth that keeps every tile in one
// round of the machine; 0 when the streaming kernel does not apply.
struct GvPlan {
  int depth, xi;
  size_t lds;
};

static GvPlan plan_gemv_stream(int64_t M, int64_t N, int64_t K) {
  GvPlan p{0, 0, 0};
  if (M < 1 || M > 4 || K < 256 || K % 256 != 0 || (uint64_t)N * (uint64_t)K / 2 >= (1ull << 32)) return p;
  int cus = 0, lds_cu = 0;
  if (!device_caps(cus, lds_cu)) return p;
  const int xi = M <= 2 ? 1 : 2;
  const int64_t tiles = (N + 15) / 16;
  const size_t sc = (size_t)((16 * (K / 16) + 1023) / 1024) * 1024;
  const int nck = (int)(K / 256);
  for (int d : {4, 2, 1}) {
    if (nck % d) continue;
    const size_t lds = (size_t)d * (kGvChunkCodes + 1024u * xi) + sc;
    if (lds > 65536) continue;
    const int64_t per_cu = lds_cu / (int64_t)lds;
    if (d > 1 && per_cu * cus < tiles) continue;
    p.depth = d;
    p.xi = xi;
    p.lds = lds;
    return p;
  }
  return p;
}

template <int NT, bool kA16>
static void gemv_nt(const void* x, size_t ld_x_bytes, int64_t M, const uint8_t* wc, const uint8_t* ws, int64_t N,
                    int64_t K, const float* gsx, const float* gsw, void* y, bool y_bf16, int64_t ld_y,
                    hipStream_t s) {
  const int grid = (int)((N + NT * 16 - 1) / (NT * 16));
  const size_t ldb = (size_t)ld_y * (y_bf16 ? 2u : 4u);
  const uint32_t kpc = (uint32_t)(ld_x_bytes / 16);
  if (y_bf16)
    gemv_kernel<NT, kA16, true><<<grid, 256, 0, s>>>((const uint4*)x, kpc, (int)M, wc, ws, (int)N, (int)K, gsx,
                                                     gsw, (uint8_t*)y, ldb);
  else
    gemv_kernel<NT, kA16, false><<<grid, 256, 0, s>>>((const uint4*)x, kpc, (int)M, wc, ws, (int)N, (int)K, gsx,
                                                      gsw, (uint8_t*)y, ldb);
}

template <bool kA16>
static void gemv_go(const void* x16, size_t ld_x_bytes, int64_t M, const uint8_t* wc, const uint8_t* ws, int64_t N,
                    int64_t K, const float* gsx, const float* gsw, void* y, bool y_bf16, int64_t ld_y,
                    hipStream_t s) {
  const uint32_t ldx = (uint32_t)ld_x_bytes;
  if (M > 4 && M <= 16 && K >= 512 && K <= 512 * kKsMaxWaves && K % 512 == 0 &&
      (uint64_t)N * (uint64_t)K / 2 < (1ull << 32)) {
    int cus = 0, lds_cu = 0;
    if (device_caps(cus, lds_cu)) {
      const int tiles = (int)((N + 15) / 16);
      const int waves = (int)(K / 512);
      // one workgroup per compute unit, but enough of them that no wave
      // reduces more than kKsMaxResults tiles
      int grid = tiles < cus ? tiles : cus;
      const int need = (tiles + waves * kKsMaxResults - 1) / (waves * kKsMaxResults);
      grid = grid > need ? grid : need;
      const int threads = waves * 64;
      const size_t ldb = (size_t)ld_y * (y_bf16 ? 2u : 4u);
      if (y_bf16)
        gemv_ksplit_kernel<kA16, true><<<grid, threads, 0, s>>>((const uint8_t*)x16, ldx, (int)M, wc, ws, (int)N,
                                                               (int)K, tiles, gsx, gsw, (uint8_t*)y, ldb);
      else
        gemv_ksplit_kernel<kA16, false><<<grid, threads, 0, s>>>((const uint8_t*)x16, ldx, (int)M, wc, ws, (int)N,
                                                                (int)K, tiles, gsx, gsw, (uint8_t*)y, ldb);
      return;
    }
  }
  const GvPlan gp = plan_gemv_stream(M, N, K);
  if (gp.depth) {
    const int tiles = (int)((N + 15) / 16);
    const size_t ldb = (size_t)ld_y * (y_bf16 ? 2u : 4u);
    auto go = [&](auto dc, auto xc) {
      constexpr int D = decltype(dc)::value, XI = decltype(xc)::value;
      if (y_bf16)
        gemv_stream_kernel<D, XI, kA16, true><<<tiles, 64, gp.lds, s>>>((const uint8_t*)x16, ldx, (int)M, wc, ws,
                                                                        (int)N, (int)K, gsx, gsw, (uint8_t*)y, ldb);
      else
        gemv_stream_kernel<D, XI, kA16, false><<<tiles, 64, gp.lds, s>>>((const uint8_t*)x16, ldx, (int)M, wc, ws,
                                                                         (int)N, (int)K, gsx, gsw, (uint8_t*)y,
                                                                         ldb);
    };
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I4 = std::integral_constant<int, 4>;
    if (gp.xi == 1) {
      if (gp.depth == 4) go(I4(), I1()); else if (gp.depth == 2) go(I2(), I1()); else go(I1(), I1());
    } else {
      if (gp.depth == 4) go(I4(), I2()); else if (gp.depth == 2) go(I2(), I2()); else go(I1(), I2());
    }
    return;
  }
  if (M > 4 && M <= 16 && K >= 256 && K % 256 == 0 && (uint64_t)N * (uint64_t)K / 2 < (1ull << 32)) {
    const int grid = (int)((N + 16 * kGwWaves - 1) / (16 * kGwWaves));
    const size_t ldb = (size_t)ld_y * (y_bf16 ? 2u : 4u);
    if (y_bf16)
      gemv_shared_kernel<kA16, true><<<grid, kGwWaves * 64, 0, s>>>((const uint8_t*)x16, ldx, (int)M, wc, ws,
                                                                     (int)N, (int)K, gsx, gsw, (uint8_t*)y, ldb);
    else
      gemv_shared_kernel<kA16, false><<<grid, kGwWaves * 64, 0, s>>>((const uint8_t*)x16, ldx, (int)M, wc, ws,
                                                                      (int)N, (int)K, gsx, gsw, (uint8_t*)y, ldb);
    return;
  }
  // One 16-row tile per workgroup keeps the grid fine-grained when the
  // activations are few; more rows per workgroup amortise the activation
  // reads when M is larger.
  if (M <= 4)
    gemv_nt<1, kA16>(x16, ld_x_bytes, M, wc, ws, N, K, gsx, gsw, y, y_bf16, ld_y, s);
  else
    gemv_nt<4, kA16>(x16, ld_x_bytes, M, wc, ws, N, K, gsx, gsw, y, y_bf16, ld_y, s);
}

void launch_gemv(bool a16, const void* x, size_t ld_x_bytes, int64_t M, int64_t K, const uint8_t* wc,
                 const uint8_t* ws, int64_t N, const float* gsx, const float* gsw, void* y, bool y_bf16,
                 int64_t ld_y, hipStream_t s) {
  if (a16)
    gemv_go<true>(x, ld_x_bytes, M, wc, ws, N, K, gsx, gsw, y, y_bf16, ld_y, s);
  else
    gemv_go<false>(x, ld_x_bytes, M, wc, ws, N, K, gsx, gsw, y, y_bf16, ld_y, s);
}

}  // namespace nvfp4
