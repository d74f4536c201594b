// FP8 E4M3 with one per-tensor scale: quantize and dequantize.
//
// Model card "Gemma-4-31B-IT-NVFP4-FP8attn-text", section "What was
// quantized, exactly" (per-tensor scale, float8_e4m3) and paper "Why Gated
// DeltaNet Survives 4-Bit Quantization", section 7 "KV-cache precision" (FP8
// KV cache with static per-tensor scales).  Byte = sign(x) << 7 |
// E4M3_RNE_sat(RN(|x| / s)); s = RN(amax / 448) unless given; dequant
// RN(E4M3(byte) * s).
//
// The rounding is decided exactly with a bracket, as for the NVFP4 encoder:
// with r = RN(1 / s) and r (1 -/+ 2^-20), the products x * r_lo and x * r_hi
// lie on either side of RN(x / s) (each rounding moves a value by at most
// 2^-24 relative), and the hardware FP8 conversion (round to nearest even;
// inputs clamped to +-448 first, which only turns larger magnitudes into the
// saturated byte the rule gives) is monotone, so equal bytes at both ends are
// the exact byte.  The rare element whose ends differ takes the correctly
// rounded quotient.  A scale whose reciprocal leaves the normal range takes
// the correctly rounded quotient for every element.
#include "launch.h"
#include "mfma_util.h"

namespace nvfp4 {

struct Fp8Scale {
  float s, rlo, rhi;
  bool fast;  // the bracket applies
};

__device__ __forceinline__ Fp8Scale fp8_scale(float s) {
  Fp8Scale f;
  f.s = s;
  const float r = s == 0.0f ? 0.0f : __fdiv_rn(1.0f, s);
  f.rlo = r * 0.99999904632568359375f;  // 1 - 2^-20
  f.rhi = r * 1.00000095367431640625f;  // 1 + 2^-20
  f.fast = s != 0.0f && s >= 0x1p-126f && r < 0x1p+126f;
  return f;
}

__device__ __forceinline__ float clamp448(float v) { return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f); }

// Bytes of four elements (element i in byte i).
__device__ __forceinline__ uint32_t fp8_pack4(float a, float b, float c, float d) {
  uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), (int)r, true);
}

__device__ __forceinline__ uint32_t fp8_exact1(float x, float s) {
  if (s == 0.0f) return (__float_as_uint(x) >> 24) & 0x80u;
  const uint32_t b = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(__fdiv_rn(x, s)), 0.0f, 0, false);
  return b & 0xFFu;
}

// Four elements -> four bytes, exactly.
__device__ __forceinline__ uint32_t fp8_encode4(const float (&x)[4], const Fp8Scale& f) {
  if (f.fast) {
    const uint32_t lo = fp8_pack4(x[0] * f.rlo, x[1] * f.rlo, x[2] * f.rlo, x[3] * f.rlo);
    const uint32_t hi = fp8_pack4(x[0] * f.rhi, x[1] * f.rhi, x[2] * f.rhi, x[3] * f.rhi);
    if (__builtin_expect(lo == hi, 1)) return lo;
    uint32_t r = lo;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (((lo ^ hi) >> (8 * i)) & 0xFFu) r = (r & ~(0xFFu << (8 * i))) | (fp8_exact1(x[i], f.s) << (8 * i));
    return r;
  }
  return fp8_exact1(x[0], f.s) | (fp8_exact1(x[1], f.s) << 8) | (fp8_exact1(x[2], f.s) << 16) |
         (fp8_exact1(x[3], f.s) << 24);
}

// 16 elements of a row as fp32 (bf16 widened exactly).
template <bool kBf16>
__device__ __forceinline__ void load16(const uint8_t* __restrict__ p, float (&x)[16]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  if (kBf16) {
    const uint4 a = q[0], b = q[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 a = q[c];
      x[4 * c] = __uint_as_float(a.x);
      x[4 * c + 1] = __uint_as_float(a.y);
      x[4 * c + 2] = __uint_as_float(a.z);
      x[4 * c + 3] = __uint_as_float(a.w);
    }
  }
}

__device__ __forceinline__ uint32_t absmax16(const float (&x)[16]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t a = __float_as_uint(x[i]) & 0x7FFFFFFFu;
    m = m > a ? m : a;
  }
  return m;
}

// kMode 0: the scale is *s_in.  1: the scale comes from the absmax partials
// of a preceding pass.  2 (small tensors): every workgroup takes the absmax
// of the whole tensor itself, then quantizes its share.  One thread per 16
// consecutive elements of a row and step, grid-stride; s_out (may be null)
// receives the scale from workgroup 0.
constexpr int kFp8Threads = 256;

template <bool kBf16, int kMode>
__global__ __launch_bounds__(256) void fp8_quantize_kernel(const uint8_t* __restrict__ x, size_t ld_bytes,
                                                            uint32_t groups_per_row, uint32_t total, FastDiv fd,
                                                            const uint32_t* __restrict__ partials, int npartials,
                                                            const float* __restrict__ s_in,
                                                            uint8_t* __restrict__ q, float* __restrict__ s_out) {
  __shared__ uint32_t red[kFp8Threads / 64];
  constexpr uint32_t kGroupBytes = kBf16 ? 32u : 64u;
  auto group_ptr = [&](uint32_t g) {
    const uint32_t r = fastdiv(g, fd);
    return x + (size_t)r * ld_bytes + (size_t)(g - r * groups_per_row) * kGroupBytes;
  };
  float s;
  if constexpr (kMode == 0) {
    s = *s_in;
  } else {
    uint32_t m = 0;
    if constexpr (kMode == 1) {
      for (int i = threadIdx.x; i < npartials; i += kFp8Threads) m = m > partials[i] ? m : partials[i];
    } else {
      for (uint32_t g = threadIdx.x; g < total; g += kFp8Threads) {
        float v[16];
        load16<kBf16>(group_ptr(g), v);
        const uint32_t a = absmax16(v);
        m = m > a ? m : a;
      }
    }
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    uint32_t amax = red[0];
#pragma unroll
    for (int i = 1; i < kFp8Threads / 64; ++i) amax = amax > red[i] ? amax : red[i];
    s = __fdiv_rn(__uint_as_float(amax), 448.0f);
  }
  if (s_out && blockIdx.x == 0 && threadIdx.x == 0) *s_out = s;
  const Fp8Scale f = fp8_scale(s);
  const uint32_t stride = gridDim.x * kFp8Threads;
  for (uint32_t g = blockIdx.x * kFp8Threads + threadIdx.x; g < total; g += stride) {
    float v[16];
    load16<kBf16>(group_ptr(g), v);
    uint32_t o[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float e[4] = {v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]};
      o[c] = fp8_encode4(e, f);
    }
    reinterpret_cast<uint4*>(q)[g] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// out = RN(E4M3(byte) * s); bf16 output is the RNE of that fp32.  One thread
// per 16 bytes.
template <bool kOutBf16>
__global__ __launch_bounds__(256) void fp8_dequant_kernel(const uint4* __restrict__ q, const float* __restrict__ s_p,
                                                           uint32_t groups_per_row, uint32_t total, FastDiv fd,
                                                           uint8_t* __restrict__ out, size_t ld_out_bytes) {
  const float s = *s_p;
  for (uint32_t g = blockIdx.x * 256u + threadIdx.x; g < total; g += gridDim.x * 256u) {
    const uint4 b = q[g];
    const uint32_t w[4] = {b.x, b.y, b.z, b.w};
    float v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
      v[4 * i] = lo[0] * s;
      v[4 * i + 1] = lo[1] * s;
      v[4 * i + 2] = hi[0] * s;
      v[4 * i + 3] = hi[1] * s;
    }
    const uint32_t r = fastdiv(g, fd);
    uint8_t* o = out + (size_t)r * ld_out_bytes + (size_t)(g - r * groups_per_row) * (kOutBf16 ? 32u : 64u);
    if (kOutBf16) {
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = f32_to_bf16_rne(v[2 * i]) | (f32_to_bf16_rne(v[2 * i + 1]) << 16);
      reinterpret_cast<uint4*>(o)[0] = make_uint4(h[0], h[1], h[2], h[3]);
      reinterpret_cast<uint4*>(o)[1] = make_uint4(h[4], h[5], h[6], h[7]);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        reinterpret_cast<float4*>(o)[c] = make_float4(v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]);
    }
  }
}

static int fp8_grid(uint32_t total) {
  uint32_t g = (total + kFp8Threads - 1) / kFp8Threads;
  return (int)(g < 1 ? 1 : (g > 2048 ? 2048 : g));
}

template <bool kBf16>
static void fp8_quantize_go(int mode, const uint8_t* x, size_t ld_bytes, uint32_t gpr, uint32_t total, FastDiv fd,
                            const uint32_t* partials, int np, const float* s_in, uint8_t* q, float* s_out,
                            hipStream_t st) {
  const int grid = fp8_grid(total);
  if (mode == 0)
    fp8_quantize_kernel<kBf16, 0><<<grid, kFp8Threads, 0, st>>>(x, ld_bytes, gpr, total, fd, partials, np, s_in, q,
                                                                s_out);
  else if (mode == 1)
    fp8_quantize_kernel<kBf16, 1><<<grid, kFp8Threads, 0, st>>>(x, ld_bytes, gpr, total, fd, partials, np, s_in, q,
                                                                s_out);
  else
    fp8_quantize_kernel<kBf16, 2><<<grid, kFp8Threads, 0, st>>>(x, ld_bytes, gpr, total, fd, partials, np, s_in, q,
                                                                s_out);
}

void launch_fp8_quantize(const void* x, bool bf16, int64_t rows, int64_t K, int64_t ld, const uint32_t* partials,
                         int npartials, const float* s_in, uint8_t* q, float* s_out, hipStream_t st) {
  const uint32_t gpr = (uint32_t)(K / 16);
  const uint32_t total = (uint32_t)(rows * (int64_t)gpr);
  if (total == 0) {
    if (s_out && s_in) launch_copy_f32(s_out, s_in, st);
    else if (s_out) launch_fill_f32(s_out, 0.0f, st);
    return;
  }
  const size_t ld_bytes = (size_t)ld * (bf16 ? 2u : 4u);
  const FastDiv fd = make_fastdiv(gpr);
  const int mode = s_in ? 0 : (npartials > 0 ? 1 : 2);
  if (mode == 2 && total > (uint32_t)kFp8Threads * 32u) {
    // self-absmax is for small tensors only; the caller passes partials otherwise
    return;
  }
  if (bf16)
    fp8_quantize_go<true>(mode, (const uint8_t*)x, ld_bytes, gpr, total, fd, partials, npartials, s_in, q, s_out, st);
  else
    fp8_quantize_go<false>(mode, (const uint8_t*)x, ld_bytes, gpr, total, fd, partials, npartials, s_in, q, s_out,
                           st);
}

void launch_fp8_dequant(const uint8_t* q, const float* s, int64_t rows, int64_t K, void* out, bool out_bf16,
                        int64_t ld_out, hipStream_t st) {
  const uint32_t gpr = (uint32_t)(K / 16);
  const uint32_t total = (uint32_t)(rows * (int64_t)gpr);
  if (total == 0) return;
  const FastDiv fd = make_fastdiv(gpr);
  const size_t ldb = (size_t)ld_out * (out_bf16 ? 2u : 4u);
  const int grid = fp8_grid(total);
  if (out_bf16)
    fp8_dequant_kernel<true><<<grid, 256, 0, st>>>((const uint4*)q, s, gpr, total, fd, (uint8_t*)out, ldb);
  else
    fp8_dequant_kernel<false><<<grid, 256, 0, st>>>((const uint4*)q, s, gpr, total, fd, (uint8_t*)out, ldb);
}

}  // namespace nvfp4
