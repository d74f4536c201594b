// Block-scaled W4A4 contraction (paper "Why Gated DeltaNet Survives 4-Bit
// Quantization", section 2 "NVFP4": both operands NVFP4, FP32 accumulate).
//
// Both kernels compute C[n, m] = sum_k W[n, k] X[m, k] on the MFMA units in
// fp16: every NVFP4 element E2M1(code) * E4M3(scale) is exact in fp16, so the
// products are exact and only the FP32 accumulation rounds.  X arrives
// already expanded to fp16 (the quantize kernel writes it); W is read as
// packed codes and scale bytes and expanded in registers right before the
// MFMA.  The epilogue applies RN(gs_x * gs_w) and stores Y[m, n].
//
// The same kernels serve W4A16 (model card "Gemma-4-31B-IT-NVFP4-FP8attn-
// text", section "Limitations": NVFP4 weights against 16-bit activations):
// with kA16 the operands are bf16, X is the caller's bf16 tensor read as
// given, W expands exactly to bf16, and the epilogue applies gs_w alone.
//
// Inside one MFMA the order of K is free as long as both operands agree.
// Each lane loads 16 bytes of W codes (32 consecutive k) and feeds dword j
// of them to sub-step j; the X operand is read with the same k permutation.
#include "encode.h"
#include "launch.h"
#include "mfma_util.h"

namespace nvfp4 {

// ====================================================================== GEMM
// Workgroup tile 256 (W rows) x 256 (X rows), 8 waves in a 4 x 2 grid (two
// per SIMD, so one can issue while the other waits), each wave 64 x 128 =
// 2 x 4 MFMA 32x32x16 tiles (128 fp32 accumulators per lane, held in the
// accumulation registers).  K advances 64 per step.
//
// Every operand byte reaches LDS by direct global->LDS transfers
// (global_load_lds), six per wave per step, so every step issues the same
// number and the wait before each barrier is exact:
//   X: the 256 x 64 fp16 tile of the step (32 KB), four transfers per wave;
//   W codes: 64 B of every W row, i.e. two steps at once (16 KB per group),
//     one transfer per wave per step, each covering 16 rows x 64 B;
//   W scale bytes: 16 B of every W row, i.e. four steps at once (4 KB per
//     group), one 32-lane transfer per wave per step covering 8 rows x 16 B.
// A transfer costs roughly in proportion to the 128-byte lines it touches,
// so wide groups for the strided W rows matter: a per-step 32 B code slice
// and 4 B scale slice of each row would touch twice and four times as many
// lines.  Each operand has a ring of three buffers: step i computes from
// X buffer i%3, code group (i/2)%3 and scale group (i/4)%3, while the
// transfers for X step i+2, half (i%2) of code group i/2+2 and quarter (i%4)
// of scale group i/4+2 are in flight; steps are counted from the first step
// of the workgroup's K range.  The main loop is unrolled by three, so the X
// buffer is a constant and the W buffers are picked per step.
//
// LDS layouts (16-byte slots unless noted):
//   X chunk (row, c) in slot c ^ (row & 7) ^ ((row >> 3) & 1) of its row;
//   W code piece p (16 B = 32 k; pieces 0, 1 = first step of the group) of
//     row r in slot p ^ swz(r), swz(r) = ((r>>2 ^ r>>3) & 1) << 1 | ((r>>1 ^ r>>2) & 1);
//   W scale dword d (the four block scales of one step) of row r in dword
//     slot d ^ ((r >> 3) & 3) of the row's 16 bytes.
// Any 8 or 16 consecutive rows then hit distinct 16-byte bank groups for the
// 128-bit operand reads, and 32 consecutive rows distinct banks for the
// scale dwords.

// Tile coordinates of a workgroup.  Workgroups go to the eight compute dies
// (XCDs, each with its own L2) round-robin by index, so workgroup b runs on
// die b % 8.  Whole tiles are renumbered so that the tiles one die holds at
// a time are consecutive in an order that walks groups of four tile rows
// column by column: the 32 concurrent tiles of a die then share 4 activation
// tiles and 8 weight tiles.  The renumbering is a bijection on the whole
// tiles (row-major indices below full_tiles), so the split tail keeps its
// tiles.  Measured under sustained load: about 0.7% faster.
__device__ __forceinline__ void tile_coords(int tile, int full_tiles, int tiles_n, int& tm, int& tn) {
  constexpr int kDies = 8, kGroupRows = 4;
  int p = tile;
  const int f8 = full_tiles - full_tiles % kDies;
  if (tile < f8) p = (tile % kDies) * (f8 / kDies) + tile / kDies;
  const int rows = full_tiles / tiles_n;  // complete tile rows among the whole tiles
  if (p < rows * tiles_n) {
    const int span = kGroupRows * tiles_n;
    const int first = (p / span) * kGroupRows;
    const int gm = rows - first < kGroupRows ? rows - first : kGroupRows;
    const int local = p - (p / span) * span;
    tm = first + local % gm;
    tn = local / gm;
  } else {
    tm = p / tiles_n;
    tn = p % tiles_n;
  }
}

struct GemmSmem {
  uint4 x[3][kGemmBM * 8];      // 3 x 32 KB
  uint4 wc[3][kGemmBN * 4];     // 3 x 16 KB
  uint32_t ws[3][kGemmBN * 2];  // 3 x 2 KB
};

constexpr int kGemmWaves = 8;
constexpr int kDmaPerStep = 6;  // per wave: 4 (X) + 1 (W codes) + 1 (W scales)

__device__ __forceinline__ uint32_t wc_swz(uint32_t r) {
  return ((((r >> 2) ^ (r >> 3)) & 1u) << 1) | (((r >> 1) ^ (r >> 2)) & 1u);
}

template <bool kA16, bool kYBf16>
__global__ __launch_bounds__(512, 1) void gemm_kernel(const uint4* __restrict__ x16, uint32_t kp_chunks,
                                                       const uint8_t* __restrict__ wc,
                                                       const uint8_t* __restrict__ ws, int N, int K, int M,
                                                       const float* __restrict__ gsx_p,
                                                       const float* __restrict__ gsw_p, uint8_t* __restrict__ y,
                                                       size_t ld_y_bytes, int tiles_n, int nk, int full_tiles,
                                                       int split, float* __restrict__ partials) {
  using O = Op<kA16>;
  using V = typename O::vec8;
  __shared__ GemmSmem sm;
  __shared__ uint32_t scale_lut[128];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS and global bases stay scalar
  const int wave_n = wave >> 1, wave_m = wave & 1;  // W rows 64 wave_n.., X rows 128 wave_m..
  // Whole tiles first; the workgroups past full_tiles each take one K part
  // (steps [kb, ke)) of a remaining tile.
  int tile = blockIdx.x, part = -1, kb = 0, ke = nk;
  if (tile >= full_tiles) {
    const int i = tile - full_tiles;
    tile = full_tiles + i / split;
    part = i % split;
    kb = part * nk / split;
    ke = (part + 1) * nk / split;
  }
  int tm, tn;
  tile_coords(tile, full_tiles, tiles_n, tm, tn);
  const int n0 = tn * kGemmBN, m0 = tm * kGemmBM;
  const int l32 = lane & 31, h = lane >> 5;
  const uint32_t kh = (uint32_t)K / 2, ks = (uint32_t)K / 16;
  const int n = ke - kb;  // steps of this workgroup

  // ---- transfer sources: a wave-uniform base per step or group plus per-lane
  // byte offsets fixed for the whole loop.
  const uint8_t* xbase = reinterpret_cast<const uint8_t*>(x16 + (size_t)m0 * kp_chunks) + (size_t)kb * 128;
  const uint8_t* wcbase = wc + (size_t)n0 * kh;
  const uint8_t* wsbase = ws + (size_t)n0 * ks;
  uint32_t xoff[4];  // X: instruction j fills slots (wave*4+j)*64 + lane (row (wave*4+j)*8 + lane/8)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int row = (wave * 4 + j) * 8 + (lane >> 3);
    row = m0 + row < M ? row : M - 1 - m0;   // rows past M repeat the last one (not stored)
    xoff[j] = ((uint32_t)row * kp_chunks + ((lane & 7) ^ ((lane >> 3) & 7) ^ (j & 1))) * 16u;
  }
  // W codes: the transfer of half hh fills rows 128 hh + 16 wave + lane/4,
  // slot lane%4 of the row, with piece (lane%4) ^ swz(row).  Pieces past the
  // end of a row (a group reaching past K) re-read the row's last 16 bytes.
  // W scales: the transfer of half hh fills (lanes 0..31) rows
  // 128 hh + 16 wave + lane/2, dword slot lane%2 of the row holding the
  // group's step (lane%2) ^ ((row >> 4) & 1) = (lane%2) ^ (wave & 1), so that
  // rows 16 apart, read by one pass of the LDS, use different banks.  Rows
  // past N repeat the last one (never stored).  These offsets are
  // recomputed per transfer (a few integer operations) rather than held in
  // registers.
  // LDS byte address of a place in sm: one address-space conversion for the
  // whole kernel, then integer offsets (a conversion per use would also test
  // the pointer for null every time)
  const uint32_t sm0 = lds_addr(&sm);
  auto soff = [&](const void* p) {
    return sm0 + (uint32_t)(reinterpret_cast<const char*>(p) - reinterpret_cast<const char*>(&sm));
  };
  const int nrows = N - n0;
  const int last = n - 1;
  const int glast = last >> 1;

  // Transfers into buffer b of each ring.  Sources past the range repeat
  // the last step or group (into buffers that are no longer read).
  auto issue_x = [&](int i, int b) {
    const uint8_t* xb = xbase + (size_t)(i < last ? i : last) * 128;
    const uint32_t lx = soff(&sm.x[b][wave * 256]);
#pragma unroll
    for (int j = 0; j < 4; ++j) lds_dma16(xb, xoff[j], lx + j * 1024);
  };
  auto issue_wc = [&](int g, int hh, int b) {
    const uint32_t goff = (uint32_t)(kb + 2 * (g < glast ? g : glast)) * 32u;
    const int row = 128 * hh + 16 * wave + (lane >> 2);
    const uint32_t piece = (((uint32_t)lane & 3u) ^ wc_swz((uint32_t)row)) * 16u;
    const uint32_t off = (uint32_t)(row < nrows ? row : nrows - 1) * kh + min(goff + piece, kh - 16u);
    lds_dma16(wcbase, off, soff(&sm.wc[b][(128 * hh + 16 * wave) * 4]));
  };
  auto issue_ws = [&](int g, int hh, int b) {
    const uint32_t goff = (uint32_t)(kb + 2 * (g < glast ? g : glast)) * 4u;
    const int row = 128 * hh + 16 * wave + (l32 >> 1);
    const uint32_t dw = (((uint32_t)lane & 1u) ^ ((uint32_t)wave & 1u)) * 4u;
    const uint32_t off = (uint32_t)(row < nrows ? row : nrows - 1) * ks + min(goff + dw, ks - 4u);
    // the LDS address is wave-uniform: taken out of the divergent branch
    const uint32_t lds = __builtin_amdgcn_readfirstlane(soff(&sm.ws[b][(128 * hh + 16 * wave) * 2]));
    if (lane < 32) lds_dma4(wsbase, off, lds);
  };

  floatx16 acc[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][u][r] = 0.0f;

  // What a scale byte becomes for the W expansion (the sign bit ignored).
  // fp16 operands: the magnitude bits shifted into an fp16 pair, a few
  // instructions, computed in place.  bf16 operands: the fp32 E4M3 value,
  // longer to compute, so a table in LDS (entry b for byte b) is read
  // instead.
  if (kA16 && tid < 128) scale_lut[tid] = O::scale_bits((uint32_t)tid);

  // Operand fragments of sub-step j from X buffer b.
  auto read_x = [&](int b, int j, V (&bx)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = wave_m * 128 + u * 32 + l32;
      bx[u] = O::vec(sm.x[b][row * 8 + ((4 * h + j) ^ (row & 7) ^ ((row >> 3) & 1))]);
    }
  };
  // W codes of one step (one 16-byte piece per row and lane) and the two
  // block scales of this lane: step s of code group buffer bc (s%2 = its
  // position in the group) and scale group buffer bs (s%4).
  auto read_w = [&](int bc, int sp2, uint4 (&wv)[2], uint32_t (&sw)[2]) {
    const uint4* cb = sm.wc[bc];
    const uint32_t* sb = sm.ws[bc];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t row = wave_n * 64 + t * 32 + l32;
      wv[t] = cb[row * 4 + ((uint32_t)(2 * sp2 + h) ^ wc_swz(row))];
      sw[t] = sb[row * 2 + ((uint32_t)sp2 ^ ((row >> 4) & 1u))] >> (16 * h);
    }
  };
  auto split_w = [&](const uint32_t (&sw)[2], uint32_t (&sp)[2][2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if constexpr (kA16) {
        sp[t][0] = scale_lut[sw[t] & 0x7Fu];
        sp[t][1] = scale_lut[(sw[t] >> 8) & 0x7Fu];
      } else {
        sp[t][0] = O::scale_bits(sw[t] & 0x7Fu);
        sp[t][1] = O::scale_bits((sw[t] >> 8) & 0x7Fu);
      }
    }
  };
  auto expand_w = [&](const uint4 (&wv)[2], const uint32_t (&sp)[2][2], int j, V (&aw)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint32_t e[4];
      O::expand(dword_of(wv[t], j), sp[t][j >> 1], e);
      aw[t] = O::vec(make_uint4(e[0], e[1], e[2], e[3]));
    }
  };
  auto mfma8 = [&](const V (&aw)[2], const V (&bx)[4]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[t][u] = O::mfma32(aw[t], bx[u], acc[t][u]);
  };

  // Register-resident operands carried across sub-steps and steps: the W
  // codes and scale splits of the current step and the operands of its next
  // sub-step.
  uint4 wv[2];
  uint32_t sp[2][2];
  V bx[4], aw[2];

  // One main-loop step, i = I (mod 6), so that every ring index is known
  // when compiling: X buffer i % 3, code and scale group buffer (i / 2) % 3,
  // position i % 2 in the group.  Sub-steps 0..2 run from X buffer i % 3,
  // each overlapping the LDS reads and expansion of the following sub-step.
  // Then the wave waits for its transfers issued one step earlier and meets
  // the barrier with the operands of sub-step 3 in registers; its 16 MFMAs
  // run after the barrier and cover the LDS reads, scale lookups and first
  // expansion of step i+1.  Step i+1's operands are prepared even after the
  // last step (the buffers then hold repeated, finite data), which keeps
  // this branch-free.
  auto step = [&](auto ic, int i) {
    constexpr int I = decltype(ic)::value, X = I % 3, I1 = I + 1;
    issue_x(i + 2, (X + 2) % 3);
    issue_wc((i >> 1) + 2, I & 1, ((I >> 1) + 2) % 3);
    issue_ws((i >> 1) + 2, I & 1, ((I >> 1) + 2) % 3);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      V bxn[4], awn[2];
      read_x(X, j + 1, bxn);
      mfma8(aw, bx);
      expand_w(wv, sp, j + 1, awn);
#pragma unroll
      for (int q = 0; q < 4; ++q) bx[q] = bxn[q];
#pragma unroll
      for (int q = 0; q < 2; ++q) aw[q] = awn[q];
    }
    // All LDS reads of this step have completed and this wave's transfers of
    // the previous step have landed (only this step's 6 may be in flight);
    // after the barrier every wave's have.  The barrier is a bare s_barrier:
    // a workgroup fence would also wait for the transfers still in flight.
    asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    V bx3[4], aw3[2];
#pragma unroll
    for (int q = 0; q < 4; ++q) bx3[q] = bx[q];
#pragma unroll
    for (int q = 0; q < 2; ++q) aw3[q] = aw[q];
    uint32_t sw[2];
    read_w((I1 >> 1) % 3, I1 & 1, wv, sw);
    read_x(I1 % 3, 0, bx);
    mfma8(aw3, bx3);
    split_w(sw, sp);
    expand_w(wv, sp, 0, aw);
  };
  static_assert(kDmaPerStep == 6, "the wait count above must match the transfers per step");

  if (n > 0) {
    // Steps 0 and 1 of X, code and scale groups 0 and 1 (steps 0..3): eight
    // transfers for step 0, then eight more.
    issue_x(0, 0);
    issue_wc(0, 0, 0);
    issue_wc(0, 1, 0);
    issue_ws(0, 0, 0);
    issue_ws(0, 1, 0);
    issue_x(1, 1);
    issue_wc(1, 0, 1);
    issue_wc(1, 1, 1);
    issue_ws(1, 0, 1);
    issue_ws(1, 1, 1);
    // (bf16 operands) the scale table above is written with ordinary LDS stores
    asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    {
      uint32_t sw[2];
      read_w(0, 0, wv, sw);
      read_x(0, 0, bx);
      split_w(sw, sp);
      expand_w(wv, sp, 0, aw);
    }
    for (int i = 0; i < n; i += 6) {
      step(std::integral_constant<int, 0>{}, i);
      if (i + 1 >= n) break;
      step(std::integral_constant<int, 1>{}, i + 1);
      if (i + 2 >= n) break;
      step(std::integral_constant<int, 2>{}, i + 2);
      if (i + 3 >= n) break;
      step(std::integral_constant<int, 3>{}, i + 3);
      if (i + 4 >= n) break;
      step(std::integral_constant<int, 4>{}, i + 4);
      if (i + 5 >= n) break;
      step(std::integral_constant<int, 5>{}, i + 5);
    }
    // drain the repeated transfers before the workgroup can exit
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  if (part >= 0) {
    // raw fp32 partial sums, tile-local [256 x 256] row-major (m, n)
    float* pp = partials + ((size_t)(tile - full_tiles) * split + part) * (kGemmBM * kGemmBN);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ml = wave_m * 128 + u * 32 + l32;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = wave_n * 64 + t * 32 + 8 * q + 4 * h;
          *reinterpret_cast<float4*>(pp + ml * kGemmBN + nl) =
              make_float4(acc[t][u][4 * q], acc[t][u][4 * q + 1], acc[t][u][4 * q + 2], acc[t][u][4 * q + 3]);
        }
    }
    return;
  }
  const float scale = kA16 ? *gsw_p : (*gsx_p) * (*gsw_p);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int m = m0 + wave_m * 128 + u * 32 + l32;
    if (m >= M) continue;
    uint8_t* yrow = y + (size_t)m * ld_y_bytes;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nn = n0 + wave_n * 64 + t * 32 + 8 * q + 4 * h;
        store4<kYBf16>(yrow, nn, N, acc[t][u][4 * q] * scale, acc[t][u][4 * q + 1] * scale,
                       acc[t][u][4 * q + 2] * scale, acc[t][u][4 * q + 3] * scale);
      }
    }
  }
}

// Adds the K parts of every split tile in part order, applies the scales
// and stores Y.  One thread per 4 consecutive outputs of a tile row.
template <bool kA16, bool kYBf16>
__global__ __launch_bounds__(256) void gemm_split_reduce_kernel(const float* __restrict__ partials, int full_tiles,
                                                                 int split, int tiles_n, int M, int N,
                                                                 const float* __restrict__ gsx_p,
                                                                 const float* __restrict__ gsw_p,
                                                                 uint8_t* __restrict__ y, size_t ld_y_bytes) {
  const int r = blockIdx.y;                        // remaining tile index
  const int tile = full_tiles + r;
  const int tn = tile % tiles_n, tm = tile / tiles_n;
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;  // element in the tile
  const int ml = e / kGemmBN, nl = e % kGemmBN;
  const int m = tm * kGemmBM + ml, n = tn * kGemmBN + nl;
  if (m >= M || n >= N) return;
  const float* pp = partials + (size_t)r * split * (kGemmBM * kGemmBN) + e;
  float4 a = *reinterpret_cast<const float4*>(pp);
  for (int s = 1; s < split; ++s) {
    const float4 b = *reinterpret_cast<const float4*>(pp + (size_t)s * (kGemmBM * kGemmBN));
    a.x += b.x;
    a.y += b.y;
    a.z += b.z;
    a.w += b.w;
  }
  const float scale = kA16 ? *gsw_p : (*gsx_p) * (*gsw_p);
  store4<kYBf16>(y + (size_t)m * ld_y_bytes, n, N, a.x * scale, a.y * scale, a.z * scale, a.w * scale);
}

// ================================================================ FP8 weights
// W8A16 and W8A8 (model card "Gemma-4-31B-IT-NVFP4-FP8attn-text", section
// "What was quantized, exactly": float8_e4m3 weights with one per-tensor
// scale, served against bf16 activations; W8A8 with FP8 activations): W is
// [N, K] E4M3 bytes.  The tile, the wave grid, the three-buffer ring of
// direct transfers and the split-K tail are those of the kernel above.
//   kA8 = false: X bf16 as given; each W byte pair becomes a bf16 pair
//     (exact, one conversion) and the MFMA is 32x32x16 bf16.
//   kA8 = true: X is E4M3 bytes; both operands go to the 32x32x64 FP8 MFMA
//     unconverted (unit block scales), 32 consecutive k per lane.
// Epilogue: y = acc * s_w (W8A16) or acc * RN(s_x * s_w) (W8A8).
//
// LDS rows of 64 bytes (W, and X in FP8) hold chunk c of row r in 16-byte
// slot c ^ ((r >> 2) & 3), so 16 consecutive rows read at one chunk hit 16
// distinct 16-byte bank groups.
typedef int i32x8 __attribute__((ext_vector_type(8)));

template <bool kA8>
struct Fp8wBuf {
  uint4 x[kGemmBM * (kA8 ? 4 : 8)];  // X: 256 rows x 64 k (fp8: 16 KB, bf16: 32 KB)
  uint4 w[kGemmBN * 4];              // W: 256 rows x 64 k fp8 (16 KB)
};

__device__ __forceinline__ uint32_t row64_slot(int row, int chunk) { return (uint32_t)(chunk ^ ((row >> 2) & 3)); }

template <bool kA8, bool kYBf16>
__global__ __launch_bounds__(512, 1) void gemm_fp8w_kernel(const uint8_t* __restrict__ x, uint32_t ld_x_bytes,
                                                            const uint8_t* __restrict__ wq, int N, int K, int M,
                                                            const float* __restrict__ sx_p,
                                                            const float* __restrict__ sw_p,
                                                            uint8_t* __restrict__ y, size_t ld_y_bytes, int tiles_n,
                                                            int nk, int full_tiles, int split,
                                                            float* __restrict__ partials) {
  using B = Fp8wBuf<kA8>;
  __shared__ B b0, b1, b2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_n = wave >> 1, wave_m = wave & 1;  // W rows 64 wave_n.., X rows 128 wave_m..
  int tile = blockIdx.x, part = -1, kb = 0, ke = nk;
  if (tile >= full_tiles) {
    const int i = tile - full_tiles;
    tile = full_tiles + i / split;
    part = i % split;
    kb = part * nk / split;
    ke = (part + 1) * nk / split;
  }
  int tm, tn;
  tile_coords(tile, full_tiles, tiles_n, tm, tn);
  const int n0 = tn * kGemmBN, m0 = tm * kGemmBM;
  const int l32 = lane & 31, h = lane >> 5;

  // ---- transfers: per step W 2 x 1 KB and X 2 x 1 KB (fp8) or 4 x 1 KB
  // (bf16) per wave.  64-byte rows: instruction j of wave w fills slots
  // (2w + j) * 64 + lane = row (2w + j) * 16 + lane / 4, slot lane % 4.
  const uint8_t* wbase = wq + (size_t)n0 * (size_t)K;
  const uint8_t* xbase = x + (size_t)m0 * ld_x_bytes;
  uint32_t woff[2], x8off[2], x16off[4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = (2 * wave + j) * 16 + (lane >> 2);
    const int logical = (lane & 3) ^ ((r >> 2) & 3);
    int rn = n0 + r < N ? r : N - 1 - n0;   // rows past N / M repeat the last one (not stored)
    int rm = m0 + r < M ? r : M - 1 - m0;
    woff[j] = (uint32_t)rn * (uint32_t)K + 16u * (uint32_t)logical;
    x8off[j] = (uint32_t)rm * ld_x_bytes + 16u * (uint32_t)logical;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // bf16 X: 128-byte rows, as in the NVFP4 kernel
    int r = (wave * 4 + j) * 8 + (lane >> 3);
    r = m0 + r < M ? r : M - 1 - m0;
    x16off[j] = (uint32_t)r * ld_x_bytes + ((uint32_t)((lane & 7) ^ ((lane >> 3) & 7) ^ (j & 1))) * 16u;
  }
  constexpr int kXDma = kA8 ? 2 : 4;
  auto lx = [&](const B& bf) { return lds_addr(&bf.x[wave * (kA8 ? 128 : 256)]); };
  auto lw = [&](const B& bf) { return lds_addr(&bf.w[wave * 128]); };
  const uint32_t lx0 = lx(b0), lx1 = lx(b1), lx2 = lx(b2), lw0 = lw(b0), lw1 = lw(b1), lw2 = lw(b2);
  auto issue = [&](int kt, uint32_t ldx, uint32_t ldw) {
#pragma unroll
    for (int j = 0; j < 2; ++j) lds_dma16(wbase + (size_t)kt * 64, woff[j], ldw + j * 1024);
    if constexpr (kA8) {
#pragma unroll
      for (int j = 0; j < 2; ++j) lds_dma16(xbase + (size_t)kt * 64, x8off[j], ldx + j * 1024);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) lds_dma16(xbase + (size_t)kt * 128, x16off[j], ldx + j * 1024);
    }
  };

  floatx16 acc[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][u][r] = 0.0f;

  // 32 bytes of a 64-byte row at k 32h .. 32h+31
  auto read32 = [&](const uint4* base, int row, uint4 (&v)[2]) {
    v[0] = base[row * 4 + row64_slot(row, 2 * h)];
    v[1] = base[row * 4 + row64_slot(row, 2 * h + 1)];
  };
  auto compute = [&](const B& cur) {
    uint4 w32[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) read32(cur.w, wave_n * 64 + t * 32 + l32, w32[t]);
    if constexpr (kA8) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint4 x32[2];
        read32(cur.x, wave_m * 128 + u * 32 + l32, x32);
        const i32x8 xb = __builtin_bit_cast(i32x8, x32);
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[t][u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, w32[t]), xb,
                                                                       acc[t][u], 0, 0, 0, 127, 0, 127);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 aw[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint32_t d0 = dword_of(w32[t][j >> 1], 2 * (j & 1)), d1 = dword_of(w32[t][j >> 1], 2 * (j & 1) + 1);
          const uint4 e = make_uint4(
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true)));
          aw[t] = __builtin_bit_cast(bf16x8, e);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int row = wave_m * 128 + u * 32 + l32;
          const bf16x8 bx = __builtin_bit_cast(bf16x8, cur.x[row * 8 + ((4 * h + j) ^ (row & 7) ^ ((row >> 3) & 1))]);
#pragma unroll
          for (int t = 0; t < 2; ++t)
            acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw[t], bx, acc[t][u], 0, 0, 0);
        }
      }
    }
  };
  constexpr int kDma = 2 + kXDma;
  // Step kt computes buffer kt % 3 while the transfers of kt + 1 and kt + 2
  // fly; the wait before the barrier leaves only kt + 2's (kDma) in flight.
  auto step = [&](int kt, const B& cur, uint32_t ldx, uint32_t ldw) {
    if constexpr (kA8)
      asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int last = ke - 1;
    issue(kt + 2 < last ? kt + 2 : last, ldx, ldw);
    compute(cur);
  };
  static_assert(kDma == (kA8 ? 4 : 6), "the wait counts above must match the transfers per step");

  if (ke > kb) {
    issue(kb, lx0, lw0);
    issue(kb + 1 < ke ? kb + 1 : kb, lx1, lw1);
    for (int kt = kb; kt < ke; kt += 3) {
      step(kt, b0, lx2, lw2);
      if (kt + 1 < ke) step(kt + 1, b1, lx0, lw0);
      if (kt + 2 < ke) step(kt + 2, b2, lx1, lw1);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  if (part >= 0) {
    float* pp = partials + ((size_t)(tile - full_tiles) * split + part) * (kGemmBM * kGemmBN);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ml = wave_m * 128 + u * 32 + l32;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = wave_n * 64 + t * 32 + 8 * q + 4 * h;
          *reinterpret_cast<float4*>(pp + ml * kGemmBN + nl) =
              make_float4(acc[t][u][4 * q], acc[t][u][4 * q + 1], acc[t][u][4 * q + 2], acc[t][u][4 * q + 3]);
        }
    }
    return;
  }
  const float scale = kA8 ? (*sx_p) * (*sw_p) : *sw_p;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int m = m0 + wave_m * 128 + u * 32 + l32;
    if (m >= M) continue;
    uint8_t* yrow = y + (size_t)m * ld_y_bytes;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wave_n * 64 + t * 32 + 8 * q + 4 * h;
        store4<kYBf16>(yrow, n, N, acc[t][u][4 * q] * scale, acc[t][u][4 * q + 1] * scale,
                       acc[t][u][4 * q + 2] * scale, acc[t][u][4 * q + 3] * scale);
      }
    }
  }
}

// ====================================================================== launch
template <bool kA16>
static void gemm_go(const void* x, uint32_t ld_x_chunks, int64_t M, int64_t K, const uint8_t* wc, const uint8_t* ws,
                    int64_t N, const float* gsx, const float* gsw, void* y, bool y_bf16, int64_t ld_y,
                    float* partials, hipStream_t s) {
  const GemmPlan p = plan_gemm(M, N, K);
  const int rem = p.tiles_m * p.tiles_n - p.full_tiles;
  const size_t ldb = (size_t)ld_y * (y_bf16 ? 2u : 4u);
  dim3 grid(p.full_tiles + rem * p.split);
  if (y_bf16)
    gemm_kernel<kA16, true><<<grid, kGemmWaves * 64, 0, s>>>((const uint4*)x, ld_x_chunks, wc, ws, (int)N, (int)K,
                                                            (int)M, gsx, gsw, (uint8_t*)y, ldb, p.tiles_n, p.nk,
                                                            p.full_tiles, p.split, partials);
  else
    gemm_kernel<kA16, false><<<grid, kGemmWaves * 64, 0, s>>>((const uint4*)x, ld_x_chunks, wc, ws, (int)N, (int)K,
                                                             (int)M, gsx, gsw, (uint8_t*)y, ldb, p.tiles_n, p.nk,
                                                             p.full_tiles, p.split, partials);
  if (p.split > 1) {
    dim3 rgrid(kGemmBM * kGemmBN / 4 / 256, rem);
    if (y_bf16)
      gemm_split_reduce_kernel<kA16, true><<<rgrid, 256, 0, s>>>(partials, p.full_tiles, p.split, p.tiles_n, (int)M,
                                                                 (int)N, gsx, gsw, (uint8_t*)y, ldb);
    else
      gemm_split_reduce_kernel<kA16, false><<<rgrid, 256, 0, s>>>(partials, p.full_tiles, p.split, p.tiles_n,
                                                                  (int)M, (int)N, gsx, gsw, (uint8_t*)y, ldb);
  }
}

template <bool kA8>
static void gemm_fp8w_go(const void* x, uint32_t ld_x_bytes, int64_t M, int64_t K, const uint8_t* wq, int64_t N,
                         const float* sx, const float* sw, void* y, bool y_bf16, int64_t ld_y, float* partials,
                         hipStream_t s) {
  const GemmPlan p = plan_gemm(M, N, K);
  const int rem = p.tiles_m * p.tiles_n - p.full_tiles;
  const size_t ldb = (size_t)ld_y * (y_bf16 ? 2u : 4u);
  dim3 grid(p.full_tiles + rem * p.split);
  if (y_bf16)
    gemm_fp8w_kernel<kA8, true><<<grid, kGemmWaves * 64, 0, s>>>((const uint8_t*)x, ld_x_bytes, wq, (int)N, (int)K,
                                                                (int)M, sx, sw, (uint8_t*)y, ldb, p.tiles_n, p.nk,
                                                                p.full_tiles, p.split, partials);
  else
    gemm_fp8w_kernel<kA8, false><<<grid, kGemmWaves * 64, 0, s>>>((const uint8_t*)x, ld_x_bytes, wq, (int)N, (int)K,
                                                                 (int)M, sx, sw, (uint8_t*)y, ldb, p.tiles_n, p.nk,
                                                                 p.full_tiles, p.split, partials);
  if (p.split > 1) {
    // the reduce applies s_w (W8A16: kA16 form) or s_x * s_w (W8A8: W4A4 form)
    dim3 rgrid(kGemmBM * kGemmBN / 4 / 256, rem);
    if (y_bf16)
      gemm_split_reduce_kernel<!kA8, true><<<rgrid, 256, 0, s>>>(partials, p.full_tiles, p.split, p.tiles_n, (int)M,
                                                                 (int)N, sx, sw, (uint8_t*)y, ldb);
    else
      gemm_split_reduce_kernel<!kA8, false><<<rgrid, 256, 0, s>>>(partials, p.full_tiles, p.split, p.tiles_n,
                                                                  (int)M, (int)N, sx, sw, (uint8_t*)y, ldb);
  }
}

void launch_gemm_fp8w(bool a8, const void* x, size_t ld_x_bytes, int64_t M, int64_t K, const uint8_t* wq, int64_t N,
                      const float* sx, const float* sw, void* y, bool y_bf16, int64_t ld_y, float* partials,
                      hipStream_t s) {
  if (a8)
    gemm_fp8w_go<true>(x, (uint32_t)ld_x_bytes, M, K, wq, N, sx, sw, y, y_bf16, ld_y, partials, s);
  else
    gemm_fp8w_go<false>(x, (uint32_t)ld_x_bytes, M, K, wq, N, sx, sw, y, y_bf16, ld_y, partials, s);
}

void launch_gemm(bool a16, const void* x, size_t ld_x_bytes, int64_t M, int64_t K, const uint8_t* wc,
                 const uint8_t* ws, int64_t N, const float* gsx, const float* gsw, void* y, bool y_bf16,
                 int64_t ld_y, float* partials, hipStream_t s) {
  const uint32_t ldc = (uint32_t)(ld_x_bytes / 16);
  if (a16)
    gemm_go<true>(x, ldc, M, K, wc, ws, N, gsx, gsw, y, y_bf16, ld_y, partials, s);
  else
    gemm_go<false>(x, ldc, M, K, wc, ws, N, gsx, gsw, y, y_bf16, ld_y, partials, s);
}

}  // namespace nvfp4
