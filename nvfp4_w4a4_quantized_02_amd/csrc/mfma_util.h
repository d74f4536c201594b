// Helpers shared by the MFMA kernels: operand casts and the output store.
#pragma once

#include "common.h"

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
