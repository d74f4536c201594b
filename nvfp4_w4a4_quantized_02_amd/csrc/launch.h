// Internal launchers shared between the kernel sources and the C ABI layer.
// Every launcher assumes its arguments were validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace nvfp4 {

// Compute units and LDS bytes per compute unit of the current device, for
// launch shapes.  Each device's values are queried once and kept in atomics:
// concurrent first calls from several host threads store the same values.
// False when the runtime cannot report them.
inline bool device_caps(int& cus, int& lds_per_cu) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached_cus[kMaxDevices], cached_lds[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  const bool cache = dev >= 0 && dev < kMaxDevices;
  if (cache) {
    cus = cached_cus[dev].load(std::memory_order_relaxed);
    lds_per_cu = cached_lds[dev].load(std::memory_order_relaxed);
    if (cus > 0 && lds_per_cu > 0) return true;
  }
  int a = 0, b = 0;
  if (hipDeviceGetAttribute(&a, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(&b, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess || a <= 0 ||
      b <= 0)
    return false;
  if (cache) {
    cached_cus[dev].store(a, std::memory_order_relaxed);
    cached_lds[dev].store(b, std::memory_order_relaxed);
  }
  cus = a;
  lds_per_cu = b;
  return true;
}

constexpr int kMaxFused = 16;
constexpr int kMaxPartials = 2048;  // absmax partials (one per workgroup)

// Workspace layout shared by quantize and gemm (byte offsets, 256-aligned).
constexpr size_t kWsPartials = 0;
constexpr size_t kWsGs = kMaxPartials * sizeof(uint32_t);   // one float
constexpr size_t kWsX16 = kWsGs + 256;                       // fp16 A operand

// GEMM tiling (see gemm.hip).
constexpr int kGemmBM = 256;   // X rows per workgroup tile
constexpr int kGemmBN = 256;   // W rows per workgroup tile
constexpr int kGemmBK = 64;    // K per main-loop step
constexpr int kGemvMaxM = 16;  // M at or below this uses the GEMV kernel

// Tiling of one GEMM.  Whole 256 x 256 tiles fill complete rounds of the
// machine; when the last round would leave most compute units idle, its
// tiles are split along K into `split` parts that write fp32 partial sums,
// which a second kernel adds in a fixed order.  A round is one tile per
// compute unit of the current device (256 on a whole MI355X, the value
// taken when the runtime cannot report it).
inline int gemm_cus() {
  int cus = 0, lds = 0;
  return device_caps(cus, lds) ? cus : 256;
}

struct GemmPlan {
  int tiles_m, tiles_n, nk;
  int full_tiles;     // tiles computed whole
  int split;          // K parts of each remaining tile (1 = none)
  size_t partial_bytes;
};

// The tile GEMM takes at most this many 256 x 256 tiles (the ABI rejects
// larger problems), so tile counts and grid sizes fit an int.
constexpr int64_t kMaxGemmTiles = (int64_t)1 << 30;
inline int64_t gemm_tiles(int64_t M, int64_t N) {
  return ((M + kGemmBM - 1) / kGemmBM) * ((N + kGemmBN - 1) / kGemmBN);
}

// 0 <= M, N, K < 2^31 and gemm_tiles(M, N) <= kMaxGemmTiles.
inline GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K) {
  GemmPlan p;
  p.tiles_m = (int)((M + kGemmBM - 1) / kGemmBM);
  p.tiles_n = (int)((N + kGemmBN - 1) / kGemmBN);
  p.nk = (int)((K + kGemmBK - 1) / kGemmBK);
  const int tiles = (int)gemm_tiles(M, N);
  const int cus = gemm_cus();
  const int rem = tiles % cus;
  int split = rem ? cus / rem : 1;
  if (split > p.nk) split = p.nk;
  if (split < 2 || M <= kGemvMaxM) {
    p.full_tiles = tiles;
    p.split = 1;
    p.partial_bytes = 0;
  } else {
    p.full_tiles = tiles - rem;
    p.split = split;
    p.partial_bytes = (size_t)rem * split * kGemmBM * kGemmBN * sizeof(float);
  }
  return p;
}

struct RescaleArgs {
  int n;
  uint64_t total;
  uint8_t* scales[kMaxFused];
  uint64_t offset[kMaxFused];
  const float* gs[kMaxFused];
  float* gs_shared;
};

// Returns the number of partials written.
int launch_amax(const void* x, bool bf16, int64_t rows, int64_t K, int64_t ld, uint32_t* partials, hipStream_t s);
// gs_in != nullptr: quantize with that (calibrated) tensor scale instead of
// the absmax one; partials/npartials are then ignored and gs may be nullptr
// (otherwise *gs receives the scale used).
void launch_quantize_packed(const void* x, bool bf16, int64_t rows, int64_t K, int64_t ld,
                            const uint32_t* partials, int npartials, const float* gs_in, uint8_t* codes,
                            uint8_t* scales, float* gs, hipStream_t s);
// codes/scales (may be null): the small-tensor kernel (at most 8192 blocks)
// also writes the packed codes and scale bytes there.
void launch_quantize_f16(const void* x, bool bf16, int64_t rows, int64_t K, int64_t ld, int64_t Kp,
                         const uint32_t* partials, int npartials, const float* gs_in, void* x16, float* gs,
                         uint8_t* codes, uint8_t* scales, hipStream_t s);
void launch_fill_f32(float* p, float v, hipStream_t s);
void launch_copy_f32(float* p, const float* v, hipStream_t s);
void launch_dequant(const uint8_t* codes, const uint8_t* scales, const float* gs, int64_t rows, int64_t K,
                    void* out, bool out_bf16, int64_t ld_out, hipStream_t s);
void launch_fuse_rescale(const RescaleArgs& a, hipStream_t s);

// FP8 E4M3 per-tensor quantize: s_in given (static scale), else the absmax
// partials of launch_amax (npartials > 0) or, when that launched nothing, a
// one-launch kernel that takes the absmax itself.  s_out may be null.  K % 16
// == 0; q is [rows, K] contiguous.
void launch_fp8_quantize(const void* x, bool bf16, int64_t rows, int64_t K, int64_t ld, const uint32_t* partials,
                         int npartials, const float* s_in, uint8_t* q, float* s_out, hipStream_t s);
void launch_fp8_dequant(const uint8_t* q, const float* scale, int64_t rows, int64_t K, void* out, bool out_bf16,
                        int64_t ld_out, hipStream_t s);

// C[m, n] = (sum_k X[m, k] * W[n, k]) * scale for the prefill tile kernel
// (M > kGemvMaxM) and the small-M kernels; K % 64 == 0.  a16 = false: X is
// the fp16 expansion of the quantized activations and scale = gs_x * gs_w
// (W4A4); a16 = true: X is the caller's bf16 tensor and scale = gs_w (W4A16,
// gsx unused).  ld_x_bytes: bytes between rows of X, a multiple of 16.
void launch_gemm(bool a16, const void* x, size_t ld_x_bytes, int64_t M, int64_t K, const uint8_t* wc,
                 const uint8_t* ws, int64_t N, const float* gsx, const float* gsw, void* y, bool y_bf16,
                 int64_t ld_y, float* partials, hipStream_t s);
// FP8 E4M3 weights [N, K] with one per-tensor scale: a8 = false (W8A16): X
// bf16, y = acc * sw; a8 = true (W8A8): X E4M3 bytes, y = acc * sx * sw.
// K % 64 == 0.  The GEMV form needs M <= 16 and K <= 5120.
void launch_gemm_fp8w(bool a8, const void* x, size_t ld_x_bytes, int64_t M, int64_t K, const uint8_t* wq, int64_t N,
                      const float* sx, const float* sw, void* y, bool y_bf16, int64_t ld_y, float* partials,
                      hipStream_t s);
void launch_gemv_fp8w(bool a8, const void* x, size_t ld_x_bytes, int64_t M, int64_t K, const uint8_t* wq, int64_t N,
                      const float* sx, const float* sw, void* y, bool y_bf16, int64_t ld_y, hipStream_t s);
constexpr int64_t kFp8GemvMaxK = 5120;

// Whether the FP4-MFMA GEMV has a form for M activation rows of length K.
inline bool gemv_fp4_has_form(int64_t M, int64_t K) { return M >= 1 && M <= 4 && (K == 4096 || K == 5120); }
// The W4A4 decode step for up to four activation rows in one launch:
// quantize x ([M, K] bf16, row stride ldx_bytes; with gs_in given, that
// tensor scale) and contract with W into y (row stride ldy_bytes).  Also
// writes what nvfp4_gemm_prepare would: the fp16 operand to x16_out
// ([M, K]), the tensor scale to gsx_out, the packed codes [M][K/2] and then
// the scale bytes [M][K/16] to q_out.  Returns false (nothing launched)
// for a shape it has no form for.
bool launch_gemv_fp4(const void* x, bool x_bf16, int64_t M, int64_t K, size_t ldx_bytes, const float* gs_in,
                     const uint8_t* wc, const uint8_t* ws, int64_t N, const float* gsw, void* y, bool y_bf16,
                     size_t ldy_bytes, void* x16_out, float* gsx_out, uint8_t* q_out, hipStream_t s);
// The GEMV for up to four prepared rows: their packed codes [M][K/2] at q,
// then their scale bytes [M][K/16], the tensor scale at gsx.  Returns false
// (nothing launched) for a shape it has no form for.
bool launch_gemv_fp4_prepared(const uint8_t* q, int64_t M, int64_t K, const float* gsx, const uint8_t* wc,
                              const uint8_t* ws, int64_t N, const float* gsw, void* y, bool y_bf16,
                              size_t ldy_bytes, hipStream_t s);

void launch_gemv(bool a16, const void* x, size_t ld_x_bytes, int64_t M, int64_t K, const uint8_t* wc,
                 const uint8_t* ws, int64_t N, const float* gsx, const float* gsw, void* y, bool y_bf16,
                 int64_t ld_y, hipStream_t s);

}  // namespace nvfp4
