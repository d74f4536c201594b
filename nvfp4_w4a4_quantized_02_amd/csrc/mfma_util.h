// Helpers shared by the MFMA kernels: operand casts and the output store.
#pragma once

#include "encode.h"

namespace nvfp4 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f16x8 u4_as_f16x8(uint4 v) { return __builtin_bit_cast(f16x8, v); }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// bf16 pairs of 8 packed codes sharing one scale: E2M1(code) * E4M3 value,
// exact (at most 6 significant bits, inside bf16's range).  The FP4
// conversion gives E2M1 as fp32, the products are exact in fp32, and the
// packing conversion to bf16 does not round.  out[i] = pair of codes byte i.
__device__ __forceinline__ void expand8_bf16(uint32_t codes8, float sv, uint32_t (&out)[4]) {
  const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes8, 1.0f, 0);
  const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes8, 1.0f, 1);
  const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes8, 1.0f, 2);
  const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes8, 1.0f, 3);
  out[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v0 * sv, bf16x2));
  out[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v1 * sv, bf16x2));
  out[2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2 * sv, bf16x2));
  out[3] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v3 * sv, bf16x2));
}

// The two operand types of the contraction kernels.  A16 = false: fp16,
// the activations being the exact fp16 expansion of their NVFP4 encoding
// (W4A4).  A16 = true: bf16, the activations being the caller's bf16 tensor
// as given (W4A16).  In both, W is expanded exactly from codes and scale
// bytes; `scale_bits` is what one scale byte (sign bit ignored) becomes for
// `expand`.
template <bool kA16>
struct Op;

template <>
struct Op<false> {
  using vec8 = f16x8;
  static __device__ __forceinline__ vec8 vec(uint4 v) { return __builtin_bit_cast(f16x8, v); }
  static __device__ __forceinline__ uint32_t scale_bits(uint32_t sb) {
    return __builtin_bit_cast(uint32_t, scale_f16x2(sb));
  }
  static __device__ __forceinline__ void expand(uint32_t codes8, uint32_t sbits, uint32_t (&out)[4]) {
    expand8(codes8, __builtin_bit_cast(half2_t, sbits), out);
  }
  static __device__ __forceinline__ floatx4 mfma16(vec8 a, vec8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ floatx16 mfma32(vec8 a, vec8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Op<true> {
  using vec8 = bf16x8;
  static __device__ __forceinline__ vec8 vec(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
  static __device__ __forceinline__ uint32_t scale_bits(uint32_t sb) {
    return __float_as_uint(e4m3_value(sb & 0x7Fu));
  }
  static __device__ __forceinline__ void expand(uint32_t codes8, uint32_t sbits, uint32_t (&out)[4]) {
    expand8_bf16(codes8, __uint_as_float(sbits), out);
  }
  static __device__ __forceinline__ floatx4 mfma16(vec8 a, vec8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ floatx16 mfma32(vec8 a, vec8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

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

typedef __attribute__((address_space(3))) void lds_void_t;

// Direct global->LDS transfers from a wave-uniform base (scalar registers)
// plus a 32-bit per-lane byte offset.  Lane i of the wave writes `size` bytes
// at LDS byte address `lds` + i * size; `lds` is wave-uniform and goes
// through M0 (one wait state after the SALU write of M0).  The transfers have no
// destination registers, and the compiler is not told about them: every wait
// on them is an explicit s_waitcnt in the kernel, which lets a main loop keep
// several steps in flight where the compiler's own bookkeeping would drain
// them.  A kernel that issues them must wait for all of them (vmcnt(0))
// before it ends, because its LDS is handed to the next workgroup.
// M0 is written only here; nothing else in these kernels uses it.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(const lds_void_t*)p);
}

}  // namespace nvfp4
