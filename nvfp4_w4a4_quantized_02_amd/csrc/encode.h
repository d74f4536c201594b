// Block encoder shared by the quantize kernels: one lane owns one 16-element
// block, computes its E4M3 scale and the 16 E2M1 codes.
//
// The code of an element is E2M1(RN(|x| / es)) with ties to the even code
// (paper "Why Gated DeltaNet Survives 4-Bit Quantization", section 2
// "NVFP4"; the exact rounding rule is this library's reading).
//
// Two encoders give the same bytes.  The fast one (encode_block_fast) brackets
// every rounding decision between two cheap estimates and falls back to exact
// arithmetic only where the bracket straddles a decision point.  The exact
// one (encode_block, for the rare blocks the fast one cannot take) moves every
// decision point of the rule into |x|-space once per block: RN(q) > c holds
// exactly when q lies above the midpoint between c and its fp32 successor
// (c even, so a tie there rounds to c), and RN(q) >= c exactly when q
// reaches the midpoint between c's predecessor and c.  With q = |x| / es and
// es > 0 this becomes |x| > T * es or |x| >= T * es, where T (at most 25
// significant bits) times es (24 bits) is exact in fp64.  A directed rounding
// of that product to fp32 turns both forms into one strict fp32 comparison
// |x| > B, so an element's magnitude code is the number of the seven block
// bounds it exceeds.
#pragma once

#include "common.h"

namespace nvfp4 {

// Decision points of E2M1 round-to-nearest-even in quotient space:
// code >= k  <=>  q (>|>=) kT[k-1].  Odd k: strict (the tie rounds down);
// even k: inclusive (the tie rounds up).
__device__ __forceinline__ double e2m1_decision(int k) {
  switch (k) {
    case 0: return 0.25 + 0x1p-26;   // RN(q) >  0.25
    case 1: return 0.75 - 0x1p-25;   // RN(q) >= 0.75
    case 2: return 1.25 + 0x1p-24;   // RN(q) >  1.25
    case 3: return 1.75 - 0x1p-24;   // RN(q) >= 1.75
    case 4: return 2.5 + 0x1p-23;    // RN(q) >  2.5
    case 5: return 3.5 - 0x1p-23;    // RN(q) >= 3.5
    default: return 5.0 + 0x1p-22;   // RN(q) >  5
  }
}

struct Bounds {
  float b[7];  // code >= k+1  <=>  |x| > b[k]
};

// Largest fp32 <= P (strict decision) or < P (inclusive decision).
__device__ __forceinline__ float bound_from(double P, bool strict) {
  float f = (float)P;  // round to nearest
  double fd = (double)f;
  bool step_down = strict ? (fd > P) : (fd >= P);
  return step_down ? __uint_as_float(__float_as_uint(f) - 1u) : f;
}

__device__ __forceinline__ Bounds make_bounds(float es) {
  Bounds B;
  if (es == 0.0f) {
#pragma unroll
    for (int k = 0; k < 7; ++k) B.b[k] = __uint_as_float(0x7F800000u);  // nothing passes
    return B;
  }
  double e = (double)es;
#pragma unroll
  for (int k = 0; k < 7; ++k) B.b[k] = bound_from(e2m1_decision(k) * e, (k & 1) == 0);
  return B;
}

// Magnitude code of a = |x| (fp32 bits compared as integers: both are
// non-negative, so integer and float order agree): the number of bounds
// passed, the bounds being increasing.  A count rather than a binary search:
// a search picks bounds by computed index, which turns the bound array into
// addressable memory (the compiler then places it in LDS and reads the
// dispatch packet at every wave's start to index it), and this path is rare.
__device__ __forceinline__ uint32_t mag_from_bounds(uint32_t a, const uint32_t (&b)[7]) {
  uint32_t c = 0;
#pragma unroll
  for (int k = 0; k < 7; ++k) c += a > b[k] ? 1u : 0u;
  return c;
}

// Encode one block.  absbits[j] = fp32 bits of |x_j|, signs = bit j set when
// x_j has its sign bit set.  Returns the scale byte; codes in two dwords
// (element 2i -> low nibble of byte i).
__device__ __forceinline__ uint32_t encode_block(const uint32_t (&absbits)[16], uint32_t signs, float gs,
                                                 uint32_t& code_lo, uint32_t& code_hi) {
  uint32_t bm = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) bm = bm > absbits[j] ? bm : absbits[j];
  BlockScale s = block_scale(__uint_as_float(bm), gs);
  Bounds Bf = make_bounds(s.es);
  uint32_t b[7];
#pragma unroll
  for (int k = 0; k < 7; ++k) b[k] = __float_as_uint(Bf.b[k]);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t c = mag_from_bounds(absbits[j], b) | (((signs >> j) & 1u) << 3);
    lo |= c << (4 * j);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t c = mag_from_bounds(absbits[8 + j], b) | (((signs >> (8 + j)) & 1u) << 3);
    hi |= c << (4 * j);
  }
  code_lo = lo;
  code_hi = hi;
  return s.sb;
}

// fp32 bits of the largest |x| of a bf16 block from its eight raw words: the
// max runs on the packed 16-bit magnitude patterns (integer order is value
// order for non-negative floats), two per instruction.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_absmax_bits(const uint32_t (&w)[8]) {
  u16x2_t m[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) m[j] = __builtin_bit_cast(u16x2_t, w[j] & 0x7FFF7FFFu);
  const u16x2_t a = __builtin_elementwise_max(__builtin_elementwise_max(m[0], m[1]),
                                              __builtin_elementwise_max(m[2], m[3]));
  const u16x2_t b = __builtin_elementwise_max(__builtin_elementwise_max(m[4], m[5]),
                                              __builtin_elementwise_max(m[6], m[7]));
  const u16x2_t c = __builtin_elementwise_max(a, b);
  const uint32_t lo = c[0], hi = c[1];
  return (hi > lo ? hi : lo) << 16;
}

// Raw words of one block: bf16 eight dwords (two elements each), fp32
// sixteen.
template <bool kBf16>
struct BlockWords {
  static constexpr int n = kBf16 ? 8 : 16;
};

template <bool kBf16>
__device__ __forceinline__ void load_words(const uint8_t* __restrict__ p, uint32_t (&w)[BlockWords<kBf16>::n]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int c = 0; c < BlockWords<kBf16>::n / 4; ++c) {
    const uint4 v = q[c];
    w[4 * c] = v.x;
    w[4 * c + 1] = v.y;
    w[4 * c + 2] = v.z;
    w[4 * c + 3] = v.w;
  }
}

// The block as fp32 (bf16 widened exactly).
template <bool kBf16>
__device__ __forceinline__ void words_to_floats(const uint32_t (&w)[BlockWords<kBf16>::n], float (&xv)[16]) {
#pragma unroll
  for (int i = 0; i < BlockWords<kBf16>::n; ++i) {
    if (kBf16) {
      xv[2 * i] = __uint_as_float(w[i] << 16);
      xv[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    } else {
      xv[i] = __uint_as_float(w[i]);
    }
  }
}

// fp32 bits of the block's largest |x|.
template <bool kBf16>
__device__ __forceinline__ uint32_t words_absmax_bits(const uint32_t (&w)[BlockWords<kBf16>::n]) {
  if constexpr (kBf16) {
    return bf16_absmax_bits(w);
  } else {
    uint32_t bm = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t a = w[j] & 0x7FFFFFFFu;
      bm = bm > a ? bm : a;
    }
    return bm;
  }
}

// Fast block encoder.  Every rounding decision is bracketed: a decision is
// taken by the fast path only when both ends of a bracket around the exact
// operand give the same result, and a block whose bracket straddles a
// decision point is reported back (returns false) for the exact path.
//
// Scale: with r = RN(1 / RN(6 gs)), r_lo = RN(r (1 - 2^-20)) and r_hi =
// RN(r (1 + 2^-20)), the products bmax * r_lo and bmax * r_hi lie strictly
// below and above RN(bmax / RN(6 gs)) (each RN step moves a value by at most
// 2^-24 relative, so the 2^-20 margins dominate); E4M3 rounding is
// monotone, so equal bytes at both ends are the exact scale byte, and
// unequal ones are settled by the correctly rounded quotient.
//
// Codes: likewise with y = 1 / es from the hardware reciprocal (relative
// error below 2^-22) and y (1 -/+ 2^-20), the hardware FP4 conversion (round
// to nearest, ties to even, saturating, sign kept) of x * y_lo and x * y_hi
// brackets E2M1(RN(|x| / es)).  es == 0 uses y = 0, which yields the
// sign-only codes the rule gives there.  Quotients below the first decision
// point stay there at both ends, and saturation happens at both ends, so
// neither needs special handling.  A subnormal es or a reciprocal that
// overflows is reported to the exact path.
struct FastScale {
  float gs;
  float t;         // RN(6 gs)
  float rlo, rhi;  // bracket of 1 / RN(6 gs); both 0 when gs == 0
  bool ok;         // false: every block takes the exact path
};

__device__ __forceinline__ FastScale fast_scale(float gs) {
  FastScale f;
  f.gs = gs;
  const float t = 6.0f * gs;
  f.t = t;
  const float r = (gs == 0.0f) ? 0.0f : __fdiv_rn(1.0f, t);
  f.rlo = r * 0.99999904632568359375f;  // 1 - 2^-20
  f.rhi = r * 1.00000095367431640625f;  // 1 + 2^-20
  f.ok = (gs == 0.0f) || (t >= 0x1p-126f && r < 0x1p+126f);
  return f;
}

__device__ __forceinline__ uint32_t cvt_fp4x8(const float (&x)[16], int base, float y) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[base + 0] * y, x[base + 1] * y, 1.0f, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[base + 2] * y, x[base + 3] * y, 1.0f, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[base + 4] * y, x[base + 5] * y, 1.0f, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[base + 6] * y, x[base + 7] * y, 1.0f, 3);
  return r;
}

// Exact codes of 8 elements: the hardware FP4 conversion (round to nearest
// even, saturating, sign kept) of the correctly rounded quotients
// RN(x / es), which is the rule itself.  Used for a half-block whose bracket
// straddles a decision point somewhere: eight divisions, branch-free, cost
// less than settling the straddling elements one by one with their own
// bounds (a divergent loop over the nibbles).  Requires es > 0.
__device__ __forceinline__ uint32_t exact_codes8(const float (&x)[16], int base, float es) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __fdiv_rn(x[base + 0], es), __fdiv_rn(x[base + 1], es), 1.0f, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __fdiv_rn(x[base + 2], es), __fdiv_rn(x[base + 3], es), 1.0f, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __fdiv_rn(x[base + 4], es), __fdiv_rn(x[base + 5], es), 1.0f, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __fdiv_rn(x[base + 6], es), __fdiv_rn(x[base + 7], es), 1.0f, 3);
  return r;
}

// The fast encoder without its code fix-ups: writes the scale byte (settled
// by division when its bracket straddles a midpoint), es, and the codes of
// each half-block (8 elements) whose brackets agree; bit h of `straddle` is
// set for a half whose brackets differ somewhere, whose codes are then
// exact_codes8(x, 8h, es).  Returns false (outputs undefined) when the block
// takes the exact path (see encode_block_fast).
__device__ __forceinline__ bool encode_block_fast_parts(const float (&x)[16], uint32_t bm, const FastScale& f,
                                                        uint32_t& sb, uint32_t& code_lo, uint32_t& code_hi,
                                                        float& es_out, uint32_t& straddle) {
  // Both scale bracket ends in one hardware E4M3 conversion (OCP E4M3FN,
  // round to nearest even, subnormals kept; clamped first so it saturates
  // at 448 = 0x7E).  When they differ, the quotient sits on or next to an
  // E4M3 rounding midpoint, and the correctly rounded quotient RN(bmax / t)
  // itself is converted: one division on those blocks only (bf16 ratios land
  // exactly on midpoints often enough, up to a few percent of the blocks of a
  // tensor with a few outlier channels).  The byte is then decoded by the
  // hardware.
  const float bmf = __uint_as_float(bm);
  const uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(bmf * f.rlo, 448.0f),
                                                                fminf(bmf * f.rhi, 448.0f), 0, false);
  sb = pk & 0xFFu;
  if (__builtin_expect(sb != ((pk >> 8) & 0xFFu), 0))
    sb = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(__fdiv_rn(bmf, f.t), 448.0f), 0.0f, 0, false) & 0xFFu;
  const float es = __builtin_amdgcn_cvt_f32_fp8((int)sb, 0) * f.gs;
  const float y = (es == 0.0f) ? 0.0f : __builtin_amdgcn_rcpf(es);
  const float ylo = y * 0.99999904632568359375f;
  const float yhi = y * 1.00000095367431640625f;
  uint32_t lo_a = cvt_fp4x8(x, 0, ylo);
  const uint32_t lo_b = cvt_fp4x8(x, 0, yhi);
  uint32_t hi_a = cvt_fp4x8(x, 8, ylo);
  const uint32_t hi_b = cvt_fp4x8(x, 8, yhi);
  const bool es_ok = (es == 0.0f) || (es >= 0x1p-126f && y < 0x1p+126f);
  code_lo = lo_a;
  code_hi = hi_a;
  es_out = es;
  straddle = (lo_a != lo_b ? 1u : 0u) | (hi_a != hi_b ? 2u : 0u);
  return f.ok && es_ok;
}

// x: the 16 values as fp32 (bf16 widened exactly); bm: fp32 bits of the
// largest |x|.  On success writes the scale byte and the codes; a half-block
// with an element on or next to a decision point is settled by division.
// Returns false only
// for a tensor scale out of the fast range, a subnormal es or a reciprocal
// that overflows (see above); the block then takes the exact path.
__device__ __forceinline__ bool encode_block_fast(const float (&x)[16], uint32_t bm, const FastScale& f,
                                                  uint32_t& sb, uint32_t& code_lo, uint32_t& code_hi) {
  float es;
  uint32_t straddle;
  if (!encode_block_fast_parts(x, bm, f, sb, code_lo, code_hi, es, straddle)) return false;
  if (__builtin_expect(straddle & 1u, 0)) code_lo = exact_codes8(x, 0, es);
  if (__builtin_expect(straddle & 2u, 0)) code_hi = exact_codes8(x, 8, es);
  return true;
}

// Exact encoder from the fp32 values (for blocks the fast path reports).
__device__ __forceinline__ uint32_t encode_block_exact(const float (&x)[16], float gs, uint32_t& code_lo,
                                                       uint32_t& code_hi) {
  uint32_t absbits[16], signs = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    absbits[j] = __float_as_uint(x[j]) & 0x7FFFFFFFu;
    signs |= (__float_as_uint(x[j]) >> 31) << j;
  }
  return encode_block(absbits, signs, gs, code_lo, code_hi);
}

// fp16 expansion of 8 packed codes sharing one scale byte: E2M1(code) *
// E4M3value(sb), exact in fp16 (values from 2^-10 to 2688, at most 6
// significant bits).  E4M3 and fp16 share their layout below the exponent
// field's top bit: the byte's seven magnitude bits shifted left by 7 are the
// fp16 whose value is E4M3value(sb) * 2^-8, for normal and subnormal bytes
// alike (the fp16 exponent bias, 15, is the E4M3 bias, 7, plus 8).  The
// hardware FP4 conversion multiplies by 2^8 (it uses only the exponent of its
// scale operand), giving E2M1 * 2^8 in [128, 1536], and one packed fp16
// multiply by that fp16 applies the scale.  Every step is exact.
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

// Both halves = E4M3value(sb & 0x7F) * 2^-8.
__device__ __forceinline__ half2_t scale_f16x2(uint32_t sb) {
  return __builtin_bit_cast(half2_t, (sb & 0x7Fu) * 0x00800080u);
}

// out[i] = fp16 pair for codes byte i (element 2i low half).
__device__ __forceinline__ void expand8(uint32_t codes8, half2_t q2, uint32_t (&out)[4]) {
  const half2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes8, 256.0f, 0);
  const half2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes8, 256.0f, 1);
  const half2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes8, 256.0f, 2);
  const half2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes8, 256.0f, 3);
  out[0] = __builtin_bit_cast(uint32_t, v0 * q2);
  out[1] = __builtin_bit_cast(uint32_t, v1 * q2);
  out[2] = __builtin_bit_cast(uint32_t, v2 * q2);
  out[3] = __builtin_bit_cast(uint32_t, v3 * q2);
}

}  // namespace nvfp4
