// Shared device-side helpers of the HIP library: NVFP4 codecs (E2M1 codes,
// E4M3 block scales), bf16 bit helpers and an exact unsigned divider.
//
// Format facts (paper "Why Gated DeltaNet Survives 4-Bit Quantization",
// section 2 "NVFP4"; model card "Gemma-4-31B-IT-NVFP4-FP8attn-text", section
// "Verification"): E2M1 magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6 (code =
// index, bit 3 = sign); E4M3 scales have bias 7, 3 mantissa bits, subnormals
// m * 2^-9 and a largest finite value 448 (byte 0x7E).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ----------------------------------------------------------------- divider
// n / d for 32-bit unsigned n and a fixed divisor 1 <= d < 2^31, by one
// high multiply (Granlund & Montgomery, "Division by invariant integers
// using multiplication", PLDI 1994, section 4): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(m, n) + n) >> l.
struct FastDiv {
  uint32_t d, m, l;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  f.d = d;
  f.l = l;
  f.m = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
  return f;
}

__device__ __forceinline__ uint32_t fastdiv(uint32_t n, FastDiv f) {
  uint32_t t = __umulhi(f.m, n);
  return (uint32_t)(((uint64_t)t + n) >> f.l);
}

// ----------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite input).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ----------------------------------------------------------------- E4M3
// Value of a non-negative finite E4M3 byte (0x00..0x7E).
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// Nearest E4M3 byte to v >= 0 (or +inf), ties to even, saturating at 448.
// Below 2^-6 the grid is m * 2^-9 (v * 512 is exact, rint rounds to even);
// above it, round the binary32 significand to 3 bits and rebias 127 -> 7.
__device__ __forceinline__ uint32_t e4m3_encode_sat(float v) {
  if (!(v < 448.0f)) return 0x7Eu;
  if (v < 0.015625f) return (uint32_t)__builtin_rintf(v * 512.0f);
  uint32_t u = __float_as_uint(v);
  uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
  return (r >> 20) - (120u << 3);
}

// ----------------------------------------------------------------- E2M1
// Nearest E2M1 magnitude code to r >= 0 (or +inf), ties to the even code,
// saturating at 6: the code counts the decision points passed, with strict
// comparison where the tie goes down and >= where it goes up.
__device__ __forceinline__ uint32_t e2m1_mag(float r) {
  return (uint32_t)(r > 0.25f) + (uint32_t)(r >= 0.75f) + (uint32_t)(r > 1.25f) +
         (uint32_t)(r >= 1.75f) + (uint32_t)(r > 2.5f) + (uint32_t)(r >= 3.5f) +
         (uint32_t)(r > 5.0f);
}

// Tensor scale from the absmax: RN(amax / 2688), 2688 = 6 * 448.
__device__ __forceinline__ float tensor_scale(float amax) { return __fdiv_rn(amax, 2688.0f); }

// Block scale byte and the effective element scale es = RN(dec(sb) * gs).
struct BlockScale {
  uint32_t sb;
  float es;
};

__device__ __forceinline__ BlockScale block_scale(float bmax, float gs) {
  BlockScale r;
  r.sb = 0u;
  if (gs != 0.0f) {
    float t = 6.0f * gs;
    r.sb = e4m3_encode_sat(__fdiv_rn(bmax, t));
  }
  r.es = e4m3_value(r.sb) * gs;
  return r;
}

// 4-bit code of x given the block's es.
__device__ __forceinline__ uint32_t elem_code(float x, float es) {
  uint32_t mag = (es != 0.0f) ? e2m1_mag(__fdiv_rn(fabsf(x), es)) : 0u;
  return ((__float_as_uint(x) >> 28) & 8u) | mag;
}

// Exact bf16 bits of E2M1(code) * E4M3value(sb) (at most 6 significant
// bits, so the fp32 product is exact and its upper half is the bf16).
__device__ __forceinline__ uint32_t code_times_scale_bf16(uint32_t code, float sv) {
  // E2M1 magnitude as fp32: code 1 -> 0.5, codes 2..7 -> (1 + m/2) 2^(e-1)
  uint32_t mag = code & 7u;
  uint32_t e = mag >> 1, m = mag & 1u;
  float v = e ? __uint_as_float(((e + 126u) << 23) | (m << 22)) : (m ? 0.5f : 0.0f);
  uint32_t p = __float_as_uint(v * sv);
  return ((p >> 16) & 0x7FFFu) | ((code & 8u) << 12);
}

// Wave-wide max of a uint32 (64 lanes).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t w = (uint32_t)__shfl_xor((int)v, o, 64);
    v = v > w ? v : w;
  }
  return v;
}

}  // namespace nvfp4
