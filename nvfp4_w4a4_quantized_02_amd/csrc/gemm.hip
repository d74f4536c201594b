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
// Inside one MFMA the order of K is free as long as both operands agree.
// Each lane loads 16 bytes of W codes (32 consecutive k) and feeds dword j
// of them to sub-step j; the X operand is read with the same k permutation.
#include "encode.h"
#include "launch.h"

namespace nvfp4 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f16x8 u4_as_f16x8(uint4 v) { return __builtin_bit_cast(f16x8, v); }

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int j) {
  return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

// Store 4 consecutive outputs y[m, n .. n+3] (n + 3 may pass N on the last tile).
template <bool kYBf16>
__device__ __forceinline__ void store4(uint8_t* __restrict__ yrow, int n, int N, float v0, float v1, float v2,
                                       float v3) {
  if (kYBf16) {
    uint32_t b0 = f32_to_bf16_rne(v0), b1 = f32_to_bf16_rne(v1), b2 = f32_to_bf16_rne(v2),
             b3 = f32_to_bf16_rne(v3);
    uint16_t* p = reinterpret_cast<uint16_t*>(yrow) + n;
    if (n + 3 < N) {
      *reinterpret_cast<uint2*>(p) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
    } else {
      if (n < N) p[0] = (uint16_t)b0;
      if (n + 1 < N) p[1] = (uint16_t)b1;
      if (n + 2 < N) p[2] = (uint16_t)b2;
    }
  } else {
    float* p = reinterpret_cast<float*>(yrow) + n;
    if (n + 3 < N) {
      *reinterpret_cast<float4*>(p) = make_float4(v0, v1, v2, v3);
    } else {
      if (n < N) p[0] = v0;
      if (n + 1 < N) p[1] = v1;
      if (n + 2 < N) p[2] = v2;
    }
  }
}

// ====================================================================== GEMM
// Workgroup tile 256 (W rows) x 256 (X rows), 4 waves in a 2 x 2 grid, each
// wave 128 x 128 = 4 x 4 MFMA 32x32x16 tiles (256 fp32 accumulators per lane,
// held in the accumulation registers).  K advances 64 per step.
//
// Every operand byte reaches LDS by direct global->LDS transfers
// (global_load_lds): the X tile (256 rows x 64 k fp16 = 32 KB), the W codes
// (256 rows x 32 B) and the W scale bytes (256 rows x 4 B).  Three buffers
// form a ring: step kt computes from buffer kt%3 while the transfers of step
// kt+2 are in flight, so one barrier per step suffices and no staging
// registers are needed.  Because all memory traffic is of this one kind and
// completes in issue order, the wait before each barrier is exact.
//
// LDS layouts (16-byte slots): X chunk (row, c) sits in slot
// c ^ (row & 7) ^ ((row >> 3) & 1) of its row; W code half (row, h) in slot
// h ^ (((row >> 2) ^ (row >> 3)) & 1).  Any 8 or 16 consecutive rows then hit
// distinct 16-byte bank groups, so the 128-bit operand reads are free of
// bank conflicts whether the LDS serves 8 or 16 lanes per pass.
typedef __attribute__((address_space(3))) void lds_void_t;

// Direct global->LDS transfers from a wave-uniform base (scalar registers)
// plus a 32-bit per-lane byte offset.  Lane i of the wave writes `size` bytes
// at LDS byte address `lds` + i * size; `lds` is wave-uniform and goes
// through M0 (one wait state after the SALU write of M0).  The transfers have no
// destination registers, and the compiler is not told about them: every wait
// on them is an explicit s_waitcnt below, which lets the main loop keep two
// steps in flight where the compiler's own bookkeeping would drain them.
// M0 is written only here; nothing else in these kernels uses it.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(const lds_void_t*)p);
}

struct GemmBuf {
  uint4 x[kGemmBM * 8];        // 32 KB
  uint4 wc[kGemmBN * 2];       // 8 KB
  uint32_t ws[kGemmBN];        // 1 KB
};

constexpr int kDmaPerStep = 11;  // per wave: 8 (X) + 2 (W codes) + 1 (W scales)

template <bool kYBf16>
__global__ __launch_bounds__(256, 1) void gemm_kernel(const uint4* __restrict__ x16, uint32_t kp_chunks,
                                                       const uint8_t* __restrict__ wc,
                                                       const uint8_t* __restrict__ ws, int N, int K, int M,
                                                       const float* __restrict__ gsx_p,
                                                       const float* __restrict__ gsw_p, uint8_t* __restrict__ y,
                                                       size_t ld_y_bytes, int tiles_n, int nk) {
  // Three distinct buffers (not one indexed array) so the compiler can see
  // that a transfer into one buffer never feeds reads of another.
  __shared__ GemmBuf b0, b1, b2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_n = wave >> 1, wave_m = wave & 1;
  const int tn = blockIdx.x % tiles_n, tm = blockIdx.x / tiles_n;
  const int n0 = tn * kGemmBN, m0 = tm * kGemmBM;
  const int l32 = lane & 31, h = lane >> 5;
  const size_t kh = (size_t)K / 2, ks = (size_t)K / 16;

  // ---- transfer sources: a wave-uniform base per step plus per-lane byte
  // offsets fixed for the whole loop.
  const uint8_t* xbase = reinterpret_cast<const uint8_t*>(x16 + (size_t)m0 * kp_chunks);  // + 128 B per step
  const uint8_t* wcbase = wc + (size_t)n0 * kh;                                          // + 32 B per step
  const uint8_t* wsbase = ws + (size_t)n0 * ks;                                          // + 4 B per step
  uint32_t xoff[8];  // X: instruction j fills slots (wave*8+j)*64 + lane (row wave*64+8j+lane/8)
#pragma unroll
  for (int j = 0; j < 8; ++j)
    xoff[j] = ((uint32_t)(wave * 64 + 8 * j + (lane >> 3)) * kp_chunks +
               ((lane & 7) ^ ((lane >> 3) & 7) ^ (j & 1))) * 16u;
  uint32_t wcoff[2];  // W codes: instruction j fills slots (wave*2+j)*64 + lane = row*2 + physical half
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int row = (wave * 2 + j) * 32 + (lane >> 1);
    row = n0 + row < N ? row : N - 1 - n0;   // rows past N repeat the last one (not stored)
    wcoff[j] = (uint32_t)row * (uint32_t)kh + (uint32_t)(((lane & 1) ^ (((lane >> 3) ^ (lane >> 4)) & 1)) * 16);
  }
  uint32_t wsoff;  // W scales: one dword (4 blocks) per row
  {
    int row = wave * 64 + lane;
    row = n0 + row < N ? row : N - 1 - n0;
    wsoff = (uint32_t)row * (uint32_t)ks;
  }
  // LDS byte addresses of this wave's transfer slots in each buffer
  const uint32_t lx0 = lds_addr(&b0.x[wave * 512]), lx1 = lds_addr(&b1.x[wave * 512]),
                 lx2 = lds_addr(&b2.x[wave * 512]);
  const uint32_t lc0 = lds_addr(&b0.wc[wave * 128]), lc1 = lds_addr(&b1.wc[wave * 128]),
                 lc2 = lds_addr(&b2.wc[wave * 128]);
  const uint32_t ls0 = lds_addr(&b0.ws[wave * 64]), ls1 = lds_addr(&b1.ws[wave * 64]),
                 ls2 = lds_addr(&b2.ws[wave * 64]);

  auto issue = [&](int kt, uint32_t lx, uint32_t lc, uint32_t ls) {
    const uint8_t* xb = xbase + (size_t)kt * 128;
#pragma unroll
    for (int j = 0; j < 8; ++j) lds_dma16(xb, xoff[j], lx + j * 1024);
    const uint8_t* cb = wcbase + (size_t)kt * 32;
#pragma unroll
    for (int j = 0; j < 2; ++j) lds_dma16(cb, wcoff[j], lc + j * 1024);
    lds_dma4(wsbase + (size_t)kt * 4, wsoff, ls);
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][u][r] = 0.0f;

  // Operand fragments of sub-step j from buffer `cur`.
  auto read_x = [&](const GemmBuf& cur, int j, f16x8 (&bx)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = wave_m * 128 + u * 32 + l32;
      bx[u] = u4_as_f16x8(cur.x[row * 8 + ((4 * h + j) ^ (row & 7) ^ ((row >> 3) & 1))]);
    }
  };
  auto expand_w = [&](const uint4 (&wv)[4], const ScaleSplit (&sp)[4][2], int j, f16x8 (&aw)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t e[4];
      expand8(dword_of(wv[t], j), sp[t][j >> 1], e);
      aw[t] = u4_as_f16x8(make_uint4(e[0], e[1], e[2], e[3]));
    }
  };

  // One main-loop step: compute step kt from `cur` while the transfers of
  // step kt+2 are in flight.  Every step issues the same transfers (near the
  // end they repeat the last step into a buffer that is no longer read), so
  // the wait count is the same in every step.  Within the step, the LDS
  // reads and the W expansion of sub-step j+1 are issued ahead of the MFMAs
  // of sub-step j.
  auto step = [&](int kt, const GemmBuf& cur, uint32_t lx, uint32_t lc, uint32_t ls) {
    const int last = nk - 1;
    uint4 wv[4];
    uint32_t sw[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = wave_n * 128 + t * 32 + l32;
      wv[t] = cur.wc[row * 2 + (h ^ (((row >> 2) ^ (row >> 3)) & 1))];
      sw[t] = cur.ws[row] >> (16 * h);
    }
    f16x8 bx[4], aw[4];
    read_x(cur, 0, bx);
    issue(kt + 2 < last ? kt + 2 : last, lx, lc, ls);
    ScaleSplit sp[4][2];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sp[t][0] = split_scale(sw[t] & 0xFFu);
      sp[t][1] = split_scale((sw[t] >> 8) & 0xFFu);
    }
    expand_w(wv, sp, 0, aw);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f16x8 bxn[4], awn[4];
      if (j < 3) read_x(cur, j + 1, bxn);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aw[t], bx[u], acc[t][u], 0, 0, 0);
      if (j < 3) {
        expand_w(wv, sp, j + 1, awn);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bx[q] = bxn[q];
          aw[q] = awn[q];
        }
      }
    }
    // The transfers of step kt+1 must have landed before the barrier; only
    // this step's (kt+2) may still be in flight.  The barrier is a bare
    // s_barrier: a workgroup fence would also wait for those.  The LDS reads
    // of `cur` are complete here (their values fed the MFMAs above), so `cur`
    // may be refilled after it.
    asm volatile("s_waitcnt vmcnt(11)\n\ts_barrier" ::: "memory");
  };
  static_assert(kDmaPerStep == 11, "the wait count above must match the transfers per step");

  if (nk > 0) {
    issue(0, lx0, lc0, ls0);
    issue(nk > 1 ? 1 : 0, lx1, lc1, ls1);
    asm volatile("s_waitcnt vmcnt(11)\n\ts_barrier" ::: "memory");
    for (int kt = 0; kt < nk; kt += 3) {
      step(kt, b0, lx2, lc2, ls2);
      if (kt + 1 < nk) step(kt + 1, b1, lx0, lc0, ls0);
      if (kt + 2 < nk) step(kt + 2, b2, lx1, lc1, ls1);
    }
    // drain the repeated transfers before the workgroup can exit
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  const float scale = (*gsx_p) * (*gsw_p);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int m = m0 + wave_m * 128 + u * 32 + l32;
    if (m >= M) continue;
    uint8_t* yrow = y + (size_t)m * ld_y_bytes;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wave_n * 128 + t * 32 + 8 * q + 4 * h;
        store4<kYBf16>(yrow, n, N, acc[t][u][4 * q] * scale, acc[t][u][4 * q + 1] * scale,
                       acc[t][u][4 * q + 2] * scale, acc[t][u][4 * q + 3] * scale);
      }
    }
  }
}

// ====================================================================== GEMV
// M <= 16 (decode).  MFMA 16x16x32 with W as the 16-row A operand and the
// (zero-padded) activations as the 16-column B operand.  A workgroup owns
// NT*16 rows of W; its 4 waves split K round-robin in 128-k chunks and their
// partial sums are added in a fixed order through LDS, so the result does
// not depend on scheduling.
template <int NT, bool kYBf16>
__global__ __launch_bounds__(256) void gemv_kernel(const uint4* __restrict__ x16, uint32_t kp_chunks, int M,
                                                    const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws,
                                                    int N, int K, const float* __restrict__ gsx_p,
                                                    const float* __restrict__ gsw_p, uint8_t* __restrict__ y,
                                                    size_t ld_y_bytes) {
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
      ScaleSplit s0 = split_scale(sv[t] & 0xFFu), s1 = split_scale(sv[t] >> 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t e[4];
        expand8(dword_of(wv[t], j), j < 2 ? s0 : s1, e);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(u4_as_f16x8(make_uint4(e[0], e[1], e[2], e[3])),
                                                        u4_as_f16x8(xv[j]), acc[t], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int t = 0; t < NT; ++t) part[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave != 0) return;
  const float scale = (*gsx_p) * (*gsw_p);
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

// ====================================================================== launch
void launch_gemm(const void* x16, int64_t M, int64_t Kp, const uint8_t* wc, const uint8_t* ws, int64_t N, int64_t K,
                 const float* gsx, const float* gsw, void* y, bool y_bf16, int64_t ld_y, hipStream_t s) {
  const int tiles_n = (int)((N + kGemmBN - 1) / kGemmBN);
  const int tiles_m = (int)((M + kGemmBM - 1) / kGemmBM);
  const int nk = (int)(Kp / kGemmBK);
  const size_t ldb = (size_t)ld_y * (y_bf16 ? 2u : 4u);
  const uint32_t kpc = (uint32_t)(Kp / 8);
  dim3 grid(tiles_n * tiles_m);
  if (y_bf16)
    gemm_kernel<true><<<grid, 256, 0, s>>>((const uint4*)x16, kpc, wc, ws, (int)N, (int)K, (int)M, gsx, gsw,
                                           (uint8_t*)y, ldb, tiles_n, nk);
  else
    gemm_kernel<false><<<grid, 256, 0, s>>>((const uint4*)x16, kpc, wc, ws, (int)N, (int)K, (int)M, gsx, gsw,
                                            (uint8_t*)y, ldb, tiles_n, nk);
}

template <int NT>
static void gemv_nt(const void* x16, int64_t M, int64_t Kp, const uint8_t* wc, const uint8_t* ws, int64_t N,
                    int64_t K, const float* gsx, const float* gsw, void* y, bool y_bf16, int64_t ld_y,
                    hipStream_t s) {
  const int grid = (int)((N + NT * 16 - 1) / (NT * 16));
  const size_t ldb = (size_t)ld_y * (y_bf16 ? 2u : 4u);
  const uint32_t kpc = (uint32_t)(Kp / 8);
  if (y_bf16)
    gemv_kernel<NT, true><<<grid, 256, 0, s>>>((const uint4*)x16, kpc, (int)M, wc, ws, (int)N, (int)K, gsx, gsw,
                                               (uint8_t*)y, ldb);
  else
    gemv_kernel<NT, false><<<grid, 256, 0, s>>>((const uint4*)x16, kpc, (int)M, wc, ws, (int)N, (int)K, gsx, gsw,
                                                (uint8_t*)y, ldb);
}

void launch_gemv(const void* x16, int64_t M, int64_t Kp, const uint8_t* wc, const uint8_t* ws, int64_t N, int64_t K,
                 const float* gsx, const float* gsw, void* y, bool y_bf16, int64_t ld_y, hipStream_t s) {
  // One 16-row tile per workgroup keeps the grid fine-grained when the
  // activations are few; more rows per workgroup amortise the activation
  // reads when M is larger.
  if (M <= 4)
    gemv_nt<1>(x16, M, Kp, wc, ws, N, K, gsx, gsw, y, y_bf16, ld_y, s);
  else
    gemv_nt<4>(x16, M, Kp, wc, ws, N, K, gsx, gsw, y, y_bf16, ld_y, s);
}

}  // namespace nvfp4
