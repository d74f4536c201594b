// Quantize-side kernels: tensor absmax, NVFP4 encode (packed codes or fp16
// expansion for the GEMM), dequant and the fused-group scale repair.
//
// Paper "Why Gated DeltaNet Survives 4-Bit Quantization", section 2 "NVFP4"
// (E2M1 values, E4M3 scale per 16-element block, FP32 tensor scale) and
// section 6 "Per-module calibration vs. fused-GEMM scaling" (the repair).
#include "encode.h"
#include "launch.h"

#include <type_traits>

namespace nvfp4 {

// ------------------------------------------------------------------ amax
// The tensor absmax is a max over fp32 bit patterns of |x| (integer order
// equals float order for non-negative values), so it is exact and does not
// depend on the reduction order.  Each workgroup writes one partial; the
// consumers reduce the partials themselves, so no atomics, no memset.
template <bool kBf16>
__global__ __launch_bounds__(256) void amax_partials_kernel(const uint4* __restrict__ x, uint32_t chunks_per_row,
                                                             uint32_t ld_chunks, uint32_t total_chunks, FastDiv fd,
                                                             uint32_t* __restrict__ partials) {
  __shared__ uint32_t red[4];
  uint32_t m = 0;
  const uint32_t stride = gridDim.x * 256u;
  // Eight 16-byte loads in flight per lane; lanes past the end re-read the
  // last chunk, which cannot change a max, so every load is unconditional.
  for (uint32_t c0 = blockIdx.x * 256u + threadIdx.x; c0 < total_chunks; c0 += 8u * stride) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      uint32_t c = c0 + (uint32_t)u * stride;
      c = c < total_chunks ? c : total_chunks - 1u;
      const uint32_t r = fastdiv(c, fd);
      v[u] = x[(size_t)r * ld_chunks + (c - r * chunks_per_row)];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (kBf16) {
          uint32_t lo = (w[i] & 0x7FFFu) << 16, hi = w[i] & 0x7FFF0000u;
          m = m > lo ? m : lo;
          m = m > hi ? m : hi;
        } else {
          uint32_t a = w[i] & 0x7FFFFFFFu;
          m = m > a ? m : a;
        }
      }
    }
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
    for (int i = 1; i < 4; ++i) r = r > red[i] ? r : red[i];
    partials[blockIdx.x] = r;
  }
}

// All threads of the workgroup return the tensor scale RN(amax / 2688).
__device__ __forceinline__ float reduce_partials_to_gs(const uint32_t* __restrict__ partials, int n,
                                                       uint32_t* red4) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    uint32_t p = partials[i];
    m = m > p ? m : p;
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t r = red4[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = r > red4[i] ? r : red4[i];
  return tensor_scale(__uint_as_float(r));
}

// Load one 16-element block as fp32 (bf16: two 16-byte chunks widened
// exactly; fp32: four chunks).
template <bool kBf16>
__device__ __forceinline__ void load_block(const uint8_t* __restrict__ p, float (&x)[16]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  if (kBf16) {
    uint4 a = q[0], b = q[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 a = q[c];
      x[4 * c] = __uint_as_float(a.x);
      x[4 * c + 1] = __uint_as_float(a.y);
      x[4 * c + 2] = __uint_as_float(a.z);
      x[4 * c + 3] = __uint_as_float(a.w);
    }
  }
}

// ------------------------------------------------------------------ encode
// One lane per 16-element block, 64 consecutive blocks per wave and step.
// The fast encoder settles every block whose scale is in its range,
// rounding ties included; the rest (a subnormal es, a reciprocal that
// overflows, a tensor scale out of range) are queued in the wave's slice of
// LDS and encoded exactly in batches of up to 64, so the exact path runs
// with full waves instead of stalling the fast path of every wave that
// holds one such block.
//
// The steps walk the tensor from its end back to its start, the reverse of
// the absmax pass, so the part read last by that pass is read first here,
// while it may still sit in the last-level cache.
//
// kF16 = false: packed codes [rows, K/2] and scale bytes [rows, K/16].
// kF16 = true: the fp16 values E2M1(code) * E4M3(scale) (the tensor scale
// stays separate) laid out [rows, out_kblocks * 16] with zero blocks beyond
// K: the A-side operand of the GEMM.
constexpr uint32_t kDeferCap = 128;  // queued blocks per wave

// kGiven: the tensor scale is *gs_in (a calibrated, static scale) and the
// partials are not read.  gs_out may be nullptr.
template <bool kBf16, bool kF16, bool kGiven>
__global__ __launch_bounds__(256) void quantize_kernel(const uint8_t* __restrict__ x, size_t ld_bytes,
                                                        uint32_t kblocks, uint32_t out_kblocks,
                                                        uint32_t total_blocks, FastDiv fd,
                                                        const uint32_t* __restrict__ partials, int npartials,
                                                        const float* __restrict__ gs_in,
                                                        uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                        uint4* __restrict__ x16, float* __restrict__ gs_out) {
  constexpr int kWaves = 4;
  __shared__ uint32_t red[kWaves];
  __shared__ uint32_t deferred[kWaves][kDeferCap];
  const float gs = kGiven ? *gs_in : reduce_partials_to_gs(partials, npartials, red);
  if (gs_out && blockIdx.x == 0 && threadIdx.x == 0) *gs_out = gs;
  const FastScale fsc = fast_scale(gs);
  const uint32_t lane = threadIdx.x & 63u;
  uint32_t* queue = deferred[threadIdx.x >> 6];
  const uint32_t waves = gridDim.x * (uint32_t)kWaves;
  const uint32_t wave_id = blockIdx.x * (uint32_t)kWaves + (threadIdx.x >> 6);
  const uint32_t chunks = (total_blocks + 63u) >> 6;
  if (wave_id >= chunks) return;

  auto load = [&](uint32_t b, uint32_t r, float (&xv)[16]) {
    const uint32_t kb = b - r * out_kblocks;
    load_block<kBf16>(x + (size_t)r * ld_bytes + (size_t)kb * (kBf16 ? 32u : 64u), xv);
  };
  auto store = [&](uint32_t b, uint32_t sb, uint32_t lo, uint32_t hi) {
    if (kF16) {
      const half2_t q2 = scale_f16x2(sb);
      uint32_t e0[4], e1[4];
      expand8(lo, q2, e0);
      expand8(hi, q2, e1);
      x16[(size_t)b * 2u] = make_uint4(e0[0], e0[1], e0[2], e0[3]);
      x16[(size_t)b * 2u + 1u] = make_uint4(e1[0], e1[1], e1[2], e1[3]);
    } else {
      *reinterpret_cast<uint2*>(codes + (size_t)b * 8u) = make_uint2(lo, hi);
      scales[b] = (uint8_t)sb;
    }
  };
  auto flush = [&](uint32_t n) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (uint32_t base = 0; base < n; base += 64u) {
      if (base + lane < n) {
        const uint32_t b = queue[base + lane];
        float xv[16];
        load(b, fastdiv(b, fd), xv);
        uint32_t lo, hi;
        const uint32_t sb = encode_block_exact(xv, gs, lo, hi);
        store(b, sb, lo, hi);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // Raw input words of the block at row r, block kb of the row.  Blocks in
  // the padding (kb >= kblocks) read the row's last real block instead,
  // which is never encoded, so every load is unconditional.
  constexpr int kWords = kBf16 ? 8 : 16;
  auto load_at = [&](uint32_t r, uint32_t kb, uint32_t (&w)[kWords]) {
    kb = kb < kblocks ? kb : kblocks - 1u;
    const uint4* q = reinterpret_cast<const uint4*>(x + (size_t)r * ld_bytes + (size_t)kb * (kBf16 ? 32u : 64u));
#pragma unroll
    for (int c = 0; c < kWords / 4; ++c) {
      const uint4 v = q[c];
      w[4 * c] = v.x;
      w[4 * c + 1] = v.y;
      w[4 * c + 2] = v.z;
      w[4 * c + 3] = v.w;
    }
  };
  const int32_t last = (int32_t)((chunks - 1u - wave_id) / waves);
  auto block_of = [&](int32_t it) { return (wave_id + (uint32_t)it * waves) * 64u + lane; };
  // A lane visits blocks b, b - stride, b - 2 stride, ... (stride = the
  // wave's chunk step).  Their (row, block-in-row) positions are stepped down
  // by the stride's quotient and remainder rather than divided out per block.
  const uint32_t stride = waves * 64u;
  const uint32_t sq = fastdiv(stride, fd), sr = stride - sq * out_kblocks;
  uint32_t pr, pk;  // position of the block fetched last
  {
    const uint32_t b = block_of(last);
    pr = fastdiv(b, fd);
    pk = b - pr * out_kblocks;
  }
  auto step_back = [&]() {
    const bool borrow = pk < sr;
    pk = pk - sr + (borrow ? out_kblocks : 0u);
    pr = pr - sq - (borrow ? 1u : 0u);
  };

  uint32_t queued = 0;  // wave-uniform
  // kb: the block's position in its row.
  auto encode = [&](uint32_t b, uint32_t kb, const uint32_t (&w)[kWords]) {
    bool settled = true;
    if (b < total_blocks) {
      if (kF16 && kb >= kblocks) {
        x16[(size_t)b * 2u] = make_uint4(0, 0, 0, 0);
        x16[(size_t)b * 2u + 1u] = make_uint4(0, 0, 0, 0);
      } else {
        float xv[16];
        words_to_floats<kBf16>(w, xv);
        uint32_t sb, lo, hi;
        settled = encode_block_fast(xv, words_absmax_bits<kBf16>(w), fsc, sb, lo, hi);
        if (settled) store(b, sb, lo, hi);
      }
    }
    const uint64_t pending = __ballot(!settled);
    if (pending) {
      const uint32_t pos =
          queued + __builtin_amdgcn_mbcnt_hi((uint32_t)(pending >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)pending, 0u));
      if (!settled) queue[pos] = b;
      queued += (uint32_t)__popcll(pending);
      if (queued > kDeferCap - 64u) {
        flush(queued);
        queued = 0;
      }
    }
  };

  // Two register sets alternate (no copies, which would wait for the fetch):
  // the next block's words are fetched before the current block is encoded,
  // so every wave keeps two blocks in flight.  The first block of the last
  // chunk may lie past the end; it then reads the tensor's last block.
  uint32_t wa[kWords], wb[kWords];
  uint32_t ka = pk, kbb = 0;  // positions of the blocks held in wa, wb
  {
    const bool in = block_of(last) < total_blocks;
    const uint32_t rl = fastdiv(total_blocks - 1u, fd);
    load_at(in ? pr : rl, in ? pk : total_blocks - 1u - rl * out_kblocks, wa);
  }
  // Past the wave's first block the position stays put, so the surplus
  // loads at the end re-read a valid block.
  for (int32_t it = last;; it -= 2) {
    if (it >= 1) step_back();
    load_at(pr, pk, wb);
    kbb = pk;
    encode(block_of(it), ka, wa);
    if (it < 1) break;
    if (it >= 2) step_back();
    load_at(pr, pk, wa);
    ka = pk;
    encode(block_of(it - 1), kbb, wb);
    if (it < 2) break;
  }
  if (queued) flush(queued);
}

// Small tensors (decode-sized activations): one launch instead of the
// absmax + encode pair, which is what decides the time at this size.  Each
// thread encodes one block, the rare bracket misses inline.  The encode is
// VALU work, so the blocks are spread over several compute units, and with
// a dynamic scale each workgroup also takes the absmax of the whole tensor
// itself (it is at most 256 KB and sits in cache after the first workgroup
// reads it; surplus lanes re-read the last block, which cannot change a max,
// so every load is unconditional): the more workgroups, the more compute
// units share the encode, but the more times the tensor is read.  Sizes:
//   * at most kSmallOneWg blocks, dynamic scale: one workgroup of that many
//     threads, whose own blocks are the whole tensor, so the absmax comes
//     from the blocks already in registers, with no second read;
//   * given scale (no absmax), or at most 16 * 256 blocks: workgroups of
//     kSmallThreads = 256 threads (one wave per SIMD);
//   * larger: workgroups of kSmallThreadsLarge = 512 threads (half as many
//     reads of the tensor per block encoded).
constexpr int kSmallThreads = 256;
constexpr int kSmallThreadsLarge = 512;
constexpr int kSmallOneWg = 1024;

// Tensors of at most this many blocks take the one-launch kernel.
static inline uint32_t small_block_limit(bool) { return 32u * kSmallThreads; }

// kGiven: the tensor scale is *gs_in and no absmax is taken.  gs_out may be
// nullptr.  With several workgroups, each takes the absmax of the whole
// tensor itself: thread t reads blocks t, t + kThreads, ... (kRounds of
// them, indices past the end clamped onto the last block), in batches whose
// loads are issued together.
template <int kThreads, bool kBf16, bool kF16, bool kGiven, int kRounds>
__global__ __launch_bounds__(kThreads) void quantize_small_kernel(const uint8_t* __restrict__ x, size_t ld_bytes,
                                                               uint32_t kblocks, uint32_t out_kblocks,
                                                               uint32_t total_blocks, FastDiv fd,
                                                               const float* __restrict__ gs_in,
                                                               uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales,
                                                               uint4* __restrict__ x16, float* __restrict__ gs_out) {
  __shared__ uint32_t red[kThreads / 64];
  if (total_blocks == 0) {  // (the launcher never sends one) no element to clamp onto
    if (gs_out && blockIdx.x == 0 && threadIdx.x == 0) *gs_out = kGiven ? *gs_in : 0.0f;
    return;
  }
  auto block_ptr = [&](uint32_t b, uint32_t& kb) {
    const uint32_t r = fastdiv(b, fd);
    kb = b - r * out_kblocks;
    const uint32_t kc = kb < kblocks ? kb : kblocks - 1u;
    return x + (size_t)r * ld_bytes + (size_t)kc * (kBf16 ? 32u : 64u);
  };

  // This thread's own block, fetched first so that it is in registers by
  // the time the tensor scale is known (lanes past the end fetch the last
  // block and encode nothing).
  const uint32_t b = blockIdx.x * kThreads + threadIdx.x;
  uint32_t kb_own;
  uint32_t own[BlockWords<kBf16>::n];
  load_words<kBf16>(block_ptr(b < total_blocks ? b : total_blocks - 1u, kb_own), own);

  float gs;
  if constexpr (kGiven) {
    gs = *gs_in;
  } else {
    uint32_t m = 0;
    if (gridDim.x == 1) {
      // One workgroup: the threads' own blocks are the whole tensor, and
      // they are already in registers (padding blocks count as zeros).
      if (b < total_blocks && kb_own < kblocks) m = words_absmax_bits<kBf16>(own);
    } else {
      // at most 16 bf16 blocks (128 registers) in flight, 4 fp32 ones
      constexpr int kCap = kBf16 ? 16 : 4;
      constexpr int kBatch = kRounds < kCap ? kRounds : kCap;
#pragma unroll
      for (int r0 = 0; r0 < kRounds; r0 += kBatch) {
        uint32_t wv[kBatch][BlockWords<kBf16>::n];
        uint32_t kb[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          uint32_t bu = threadIdx.x + (uint32_t)(r0 + u) * kThreads;
          bu = bu < total_blocks ? bu : total_blocks - 1u;
          load_words<kBf16>(block_ptr(bu, kb[u]), wv[u]);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const uint32_t a = kb[u] < kblocks ? words_absmax_bits<kBf16>(wv[u]) : 0u;  // padding blocks are zeros
          m = m > a ? m : a;
        }
      }
    }
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    uint32_t amax = red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) amax = amax > red[i] ? amax : red[i];
    gs = tensor_scale(__uint_as_float(amax));
  }
  if (gs_out && blockIdx.x == 0 && threadIdx.x == 0) *gs_out = gs;

  if (b >= total_blocks) return;
  if (kF16 && kb_own >= kblocks) {
    x16[(size_t)b * 2u] = make_uint4(0, 0, 0, 0);
    x16[(size_t)b * 2u + 1u] = make_uint4(0, 0, 0, 0);
    return;
  }
  float xv[16];
  words_to_floats<kBf16>(own, xv);
  uint32_t sb, lo, hi;
  if (!encode_block_fast(xv, words_absmax_bits<kBf16>(own), fast_scale(gs), sb, lo, hi))
    sb = encode_block_exact(xv, gs, lo, hi);
  if (kF16) {
    const half2_t q2 = scale_f16x2(sb);
    uint32_t e0[4], e1[4];
    expand8(lo, q2, e0);
    expand8(hi, q2, e1);
    x16[(size_t)b * 2u] = make_uint4(e0[0], e0[1], e0[2], e0[3]);
    x16[(size_t)b * 2u + 1u] = make_uint4(e1[0], e1[1], e1[2], e1[3]);
  }
  if (!kF16 || codes) {  // the fp16 form may also keep the packed codes and scale bytes
    *reinterpret_cast<uint2*>(codes + (size_t)b * 8u) = make_uint2(lo, hi);
    scales[b] = (uint8_t)sb;
  }
}

__global__ void fill_f32_kernel(float* p, float v) { *p = v; }
__global__ void copy_f32_kernel(float* p, const float* v) { *p = *v; }

// ------------------------------------------------------------------ dequant
// out = RN_fp32(E2M1(code) * E4M3(scale) * gs); the first product is exact.
template <bool kOutBf16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ scales,
                                                       const float* __restrict__ gs_p, uint32_t k8,
                                                       uint32_t total, FastDiv fd, uint8_t* __restrict__ out,
                                                       size_t ld_out_bytes) {
  const float gs = *gs_p;
  for (uint32_t c = blockIdx.x * 256u + threadIdx.x; c < total; c += gridDim.x * 256u) {
    uint32_t r = fastdiv(c, fd);
    uint32_t kc = c - r * k8;  // 8-element chunk within the row
    uint32_t w = codes[c];
    float sv = e4m3_value(scales[(size_t)r * (k8 >> 1) + (kc >> 1)]);
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t code = (w >> (4 * j)) & 15u;
      uint32_t mag = code & 7u, e = mag >> 1, m = mag & 1u;
      float cv = e ? __uint_as_float(((e + 126u) << 23) | (m << 22)) : (m ? 0.5f : 0.0f);
      float p = (cv * sv) * gs;
      v[j] = (code & 8u) ? -p : p;
    }
    uint8_t* o = out + (size_t)r * ld_out_bytes + (size_t)kc * (kOutBf16 ? 16u : 32u);
    if (kOutBf16) {
      uint4 q;
      q.x = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
      q.y = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
      q.z = f32_to_bf16_rne(v[4]) | (f32_to_bf16_rne(v[5]) << 16);
      q.w = f32_to_bf16_rne(v[6]) | (f32_to_bf16_rne(v[7]) << 16);
      *reinterpret_cast<uint4*>(o) = q;
    } else {
      reinterpret_cast<float4*>(o)[0] = make_float4(v[0], v[1], v[2], v[3]);
      reinterpret_cast<float4*>(o)[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

// ------------------------------------------------------------------ repair
__global__ __launch_bounds__(256) void fuse_rescale_kernel(RescaleArgs a) {
  __shared__ float rho_s[kMaxFused];
  __shared__ float S_s;
  if (threadIdx.x == 0) {
    float S = 0.0f;
    for (int i = 0; i < a.n; ++i) {
      float g = *a.gs[i];
      S = g > S ? g : S;
    }
    S_s = S;
  }
  __syncthreads();
  const float S = S_s;
  if (threadIdx.x < (unsigned)a.n) {
    float g = *a.gs[threadIdx.x];
    rho_s[threadIdx.x] = (S == 0.0f) ? 1.0f : __fdiv_rn(g, S);
  }
  __syncthreads();
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.gs_shared = S;
  for (uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x; i < a.total; i += (uint64_t)gridDim.x * 256u) {
    int mbr = 0;
    while (mbr + 1 < a.n && i >= a.offset[mbr + 1]) ++mbr;
    uint8_t* p = a.scales[mbr] + (i - a.offset[mbr]);
    uint32_t b = *p;
    if ((b & 0x7Fu) == 0x7Fu) continue;  // NaN bytes are kept
    float v = e4m3_value(b & 0x7Fu) * rho_s[mbr];
    *p = (uint8_t)((b & 0x80u) | e4m3_encode_sat(v));
  }
}

// ------------------------------------------------------------------ launchers
static inline int grid_for(uint64_t work, uint64_t per_wg, int cap) {
  uint64_t g = (work + per_wg - 1) / per_wg;
  if (g < 1) g = 1;
  if (g > (uint64_t)cap) g = cap;
  return (int)g;
}

int launch_amax(const void* x, bool bf16, int64_t rows, int64_t K, int64_t ld, uint32_t* partials,
                hipStream_t s) {
  if (rows * (K / 16) <= (int64_t)small_block_limit(bf16)) return 0;  // one-launch quantize instead
  uint32_t esize = bf16 ? 2u : 4u;
  uint32_t cpr = (uint32_t)(K * esize / 16);
  uint32_t ldc = (uint32_t)(ld * esize / 16);
  uint32_t total = (uint32_t)(rows * (int64_t)cpr);
  // 512 workgroups keep 16 MB in flight, enough for full bandwidth, and
  // give the encode kernel few partials to reduce.
  int grid = grid_for(total, 256 * 8, 512);
  FastDiv fd = make_fastdiv(cpr ? cpr : 1u);
  if (bf16)
    amax_partials_kernel<true><<<grid, 256, 0, s>>>((const uint4*)x, cpr, ldc, total, fd, partials);
  else
    amax_partials_kernel<false><<<grid, 256, 0, s>>>((const uint4*)x, cpr, ldc, total, fd, partials);
  return grid;
}

template <bool kBf16, bool kF16, bool kGiven>
static void launch_encode(bool small, const uint8_t* xb, size_t ld_bytes, uint32_t kb, uint32_t okb, uint32_t total,
                          FastDiv fd, const uint32_t* partials, int npartials, const float* gs_in, uint8_t* codes,
                          uint8_t* scales, uint4* xo, float* gs, hipStream_t s) {
  if (small) {
    if (!kGiven && total <= (uint32_t)kSmallOneWg) {
      quantize_small_kernel<kSmallOneWg, kBf16, kF16, false, 1>
          <<<1, kSmallOneWg, 0, s>>>(xb, ld_bytes, kb, okb, total, fd, gs_in, codes, scales, xo, gs);
      return;
    }
    // the absmax reads every block: kRounds * threads >= total
    if (kGiven || total <= 16u * kSmallThreads) {
      const int grid = (int)((total + kSmallThreads - 1) / kSmallThreads);
      auto go = [&](auto rounds) {
        quantize_small_kernel<kSmallThreads, kBf16, kF16, kGiven, decltype(rounds)::value>
            <<<grid, kSmallThreads, 0, s>>>(xb, ld_bytes, kb, okb, total, fd, gs_in, codes, scales, xo, gs);
      };
      if (kGiven) go(std::integral_constant<int, 1>());
      else if (grid <= 8) go(std::integral_constant<int, 8>());
      else go(std::integral_constant<int, 16>());
      return;
    }
    const int grid = (int)((total + kSmallThreadsLarge - 1) / kSmallThreadsLarge);  // at most 16
    auto go = [&](auto rounds) {
      quantize_small_kernel<kSmallThreadsLarge, kBf16, kF16, false, decltype(rounds)::value>
          <<<grid, kSmallThreadsLarge, 0, s>>>(xb, ld_bytes, kb, okb, total, fd, gs_in, codes, scales, xo, gs);
    };
    if (grid <= 12) go(std::integral_constant<int, 12>());
    else go(std::integral_constant<int, 16>());
    return;
  }
  // Four workgroups per compute unit, all resident at once:
  // each wave then walks several chunks and every workgroup reduces the
  // partials once.
  const int grid = grid_for(total, 256, 1024);
  quantize_kernel<kBf16, kF16, kGiven><<<grid, 256, 0, s>>>(xb, ld_bytes, kb, okb, total, fd, partials, npartials,
                                                            gs_in, codes, scales, xo, gs);
}

// npartials == 0 (launch_amax launched nothing): one workgroup does it all.
// gs_in != nullptr: the tensor scale is given; no absmax is taken (and
// partials/npartials are ignored): small tensors take the one-launch kernel,
// large ones the encode kernel alone.
template <bool kF16>
static void launch_quantize(const void* x, bool bf16, int64_t rows, int64_t K, int64_t ld, int64_t Kp,
                            const uint32_t* partials, int npartials, const float* gs_in, uint8_t* codes,
                            uint8_t* scales, void* x16, float* gs, hipStream_t s) {
  const uint32_t kb = (uint32_t)(K / 16), okb = (uint32_t)(Kp / 16);
  const uint32_t total = (uint32_t)(rows * (int64_t)okb);
  const size_t ld_bytes = (size_t)ld * (bf16 ? 2u : 4u);
  const FastDiv fd = make_fastdiv(okb ? okb : 1u);
  const uint8_t* xb = (const uint8_t*)x;
  uint4* xo = (uint4*)x16;
  if (total == 0) {  // nothing to encode; the absmax of no elements is 0
    if (gs && !gs_in) launch_fill_f32(gs, 0.0f, s);
    if (gs && gs_in) launch_copy_f32(gs, gs_in, s);
    return;
  }
  const bool small = gs_in ? total <= small_block_limit(bf16) : npartials == 0;
  if (bf16 && gs_in)
    launch_encode<true, kF16, true>(small, xb, ld_bytes, kb, okb, total, fd, partials, npartials, gs_in, codes,
                                    scales, xo, gs, s);
  else if (bf16)
    launch_encode<true, kF16, false>(small, xb, ld_bytes, kb, okb, total, fd, partials, npartials, gs_in, codes,
                                     scales, xo, gs, s);
  else if (gs_in)
    launch_encode<false, kF16, true>(small, xb, ld_bytes, kb, okb, total, fd, partials, npartials, gs_in, codes,
                                     scales, xo, gs, s);
  else
    launch_encode<false, kF16, false>(small, xb, ld_bytes, kb, okb, total, fd, partials, npartials, gs_in, codes,
                                      scales, xo, gs, s);
}

void launch_quantize_packed(const void* x, bool bf16, int64_t rows, int64_t K, int64_t ld,
                            const uint32_t* partials, int npartials, const float* gs_in, uint8_t* codes,
                            uint8_t* scales, float* gs, hipStream_t s) {
  launch_quantize<false>(x, bf16, rows, K, ld, K, partials, npartials, gs_in, codes, scales, nullptr, gs, s);
}

void launch_quantize_f16(const void* x, bool bf16, int64_t rows, int64_t K, int64_t ld, int64_t Kp,
                         const uint32_t* partials, int npartials, const float* gs_in, void* x16, float* gs,
                         uint8_t* codes, uint8_t* scales, hipStream_t s) {
  launch_quantize<true>(x, bf16, rows, K, ld, Kp, partials, npartials, gs_in, codes, scales, x16, gs, s);
}

void launch_fill_f32(float* p, float v, hipStream_t s) { fill_f32_kernel<<<1, 1, 0, s>>>(p, v); }
void launch_copy_f32(float* p, const float* v, hipStream_t s) { copy_f32_kernel<<<1, 1, 0, s>>>(p, v); }

void launch_dequant(const uint8_t* codes, const uint8_t* scales, const float* gs, int64_t rows, int64_t K,
                    void* out, bool out_bf16, int64_t ld_out, hipStream_t s) {
  uint32_t k8 = (uint32_t)(K / 8);
  uint32_t total = (uint32_t)(rows * (int64_t)k8);
  int grid = grid_for(total, 256, 8192);
  FastDiv fd = make_fastdiv(k8 ? k8 : 1u);
  size_t ldb = (size_t)ld_out * (out_bf16 ? 2u : 4u);
  if (out_bf16)
    dequant_kernel<true><<<grid, 256, 0, s>>>((const uint32_t*)codes, scales, gs, k8, total, fd, (uint8_t*)out, ldb);
  else
    dequant_kernel<false><<<grid, 256, 0, s>>>((const uint32_t*)codes, scales, gs, k8, total, fd, (uint8_t*)out,
                                               ldb);
}

void launch_fuse_rescale(const RescaleArgs& a, hipStream_t s) {
  int grid = grid_for(a.total, 256, 4096);
  fuse_rescale_kernel<<<grid, 256, 0, s>>>(a);
}

}  // namespace nvfp4
