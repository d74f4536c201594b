// C ABI of the library (declared in include/nvfp4.h): argument checks,
// workspace carving and kernel launches.  Nothing here allocates memory or
// synchronizes; every failure is reported before anything is launched.
#include "../../include/nvfp4.h"

#include <hip/hip_runtime.h>

#include <atomic>

#include "launch.h"

using namespace nvfp4;

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;  // per-dimension limit
constexpr uint64_t kMaxBlocks = (uint64_t)1 << 31;
// Kernels that read the caller's activations tile by tile address up to 256
// rows from a tile base with 32-bit offsets.
constexpr uint64_t kMaxTileRowBytes = (uint64_t)1 << 24;

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
inline size_t esize(nvfp4_dtype_t t) { return t == NVFP4_BF16 ? 2u : 4u; }
inline bool dtype_ok(nvfp4_dtype_t t) { return t == NVFP4_F32 || t == NVFP4_BF16; }

nvfp4_status_t launched() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_DEVICE;
}

// Shared checks for a [rows, K] activation/weight input with leading dim ld.
nvfp4_status_t check_input(const void* x, nvfp4_dtype_t dt, int64_t rows, int64_t K, int64_t ld) {
  if (!dtype_ok(dt)) return NVFP4_ERR_DTYPE;
  if (rows < 0 || K < 0 || rows >= kMaxDim || K >= kMaxDim) return NVFP4_ERR_SHAPE;
  if (K % 16 != 0) return NVFP4_ERR_SHAPE;
  if (rows > 0 && K > 0) {
    if (!x) return NVFP4_ERR_NULL;
    if (ld < K) return NVFP4_ERR_SHAPE;
    if (!aligned(x, 16) || ((uint64_t)ld * esize(dt)) % 16 != 0) return NVFP4_ERR_ALIGN;
    // chunk indices (16 bytes) and block indices must fit 32 bits
    if ((uint64_t)rows * (uint64_t)(K / 16) * 4u >= kMaxBlocks) return NVFP4_ERR_SHAPE;
    if ((uint64_t)rows * (uint64_t)ld * esize(dt) / 16u >= ((uint64_t)1 << 32)) return NVFP4_ERR_SHAPE;
  }
  return NVFP4_OK;
}

}  // namespace

extern "C" {

const char* nvfp4_status_string(nvfp4_status_t s) {
  switch (s) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "invalid shape or leading dimension";
    case NVFP4_ERR_DTYPE: return "unsupported dtype";
    case NVFP4_ERR_ALIGN: return "pointer or leading dimension not 16-byte aligned";
    case NVFP4_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case NVFP4_ERR_INVALID: return "invalid argument";
    case NVFP4_ERR_DEVICE: return "HIP launch failed";
  }
  return "unknown status";
}

int nvfp4_version(void) { return 100; }

size_t nvfp4_quantize_workspace_size(int64_t rows, int64_t K) {
  (void)rows;
  (void)K;
  return kMaxPartials * sizeof(uint32_t);
}

nvfp4_status_t nvfp4_quantize(const void* x, nvfp4_dtype_t x_dtype, int64_t rows, int64_t K, int64_t ld_x,
                              uint8_t* codes, uint8_t* scales, float* gs, void* workspace, size_t workspace_bytes,
                              void* stream) {
  nvfp4_status_t st = check_input(x, x_dtype, rows, K, ld_x);
  if (st != NVFP4_OK) return st;
  if (!gs) return NVFP4_ERR_NULL;
  hipStream_t s = (hipStream_t)stream;
  if (rows == 0 || K == 0) {
    launch_fill_f32(gs, 0.0f, s);
    return launched();
  }
  if (!codes || !scales) return NVFP4_ERR_NULL;
  if (!aligned(codes, 8)) return NVFP4_ERR_ALIGN;
  if (!workspace || !aligned(workspace, 256) ||
      workspace_bytes < nvfp4_quantize_workspace_size(rows, K))
    return NVFP4_ERR_WORKSPACE;
  uint32_t* partials = (uint32_t*)((char*)workspace + kWsPartials);
  int np = launch_amax(x, x_dtype == NVFP4_BF16, rows, K, ld_x, partials, s);
  launch_quantize_packed(x, x_dtype == NVFP4_BF16, rows, K, ld_x, partials, np, nullptr, codes, scales, gs, s);
  return launched();
}

nvfp4_status_t nvfp4_quantize_static(const void* x, nvfp4_dtype_t x_dtype, int64_t rows, int64_t K, int64_t ld_x,
                                     const float* gs, uint8_t* codes, uint8_t* scales, void* stream) {
  nvfp4_status_t st = check_input(x, x_dtype, rows, K, ld_x);
  if (st != NVFP4_OK) return st;
  if (!gs) return NVFP4_ERR_NULL;
  if (rows == 0 || K == 0) return NVFP4_OK;
  if (!codes || !scales) return NVFP4_ERR_NULL;
  if (!aligned(codes, 8)) return NVFP4_ERR_ALIGN;
  launch_quantize_packed(x, x_dtype == NVFP4_BF16, rows, K, ld_x, nullptr, 0, gs, codes, scales, nullptr,
                         (hipStream_t)stream);
  return launched();
}

nvfp4_status_t nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* gs, int64_t rows,
                                int64_t K, void* out, nvfp4_dtype_t out_dtype, int64_t ld_out, void* stream) {
  if (!dtype_ok(out_dtype)) return NVFP4_ERR_DTYPE;
  if (rows < 0 || K < 0 || rows >= kMaxDim || K >= kMaxDim || K % 16 != 0) return NVFP4_ERR_SHAPE;
  if (rows == 0 || K == 0) return NVFP4_OK;
  if (!codes || !scales || !gs || !out) return NVFP4_ERR_NULL;
  if (ld_out < K) return NVFP4_ERR_SHAPE;
  if ((uint64_t)rows * (uint64_t)(K / 8) >= kMaxBlocks) return NVFP4_ERR_SHAPE;
  if (!aligned(codes, 4) || !aligned(out, 16) || ((uint64_t)ld_out * esize(out_dtype)) % 16 != 0)
    return NVFP4_ERR_ALIGN;
  launch_dequant(codes, scales, gs, rows, K, out, out_dtype == NVFP4_BF16, ld_out, (hipStream_t)stream);
  return launched();
}

nvfp4_status_t nvfp4_fuse_rescale(int n, uint8_t* const* scales, const int64_t* rows, int64_t k_blocks,
                                  const float* const* gs_in, float* gs_shared, void* stream) {
  if (n < 1 || n > NVFP4_MAX_FUSED) return NVFP4_ERR_INVALID;
  if (!scales || !rows || !gs_in || !gs_shared) return NVFP4_ERR_NULL;
  if (k_blocks < 0 || k_blocks >= kMaxDim) return NVFP4_ERR_SHAPE;
  RescaleArgs a = {};
  a.n = n;
  uint64_t off = 0;
  for (int i = 0; i < n; ++i) {
    if (rows[i] < 0 || rows[i] >= kMaxDim) return NVFP4_ERR_SHAPE;
    if (!gs_in[i]) return NVFP4_ERR_NULL;
    if (gs_in[i] == gs_shared) return NVFP4_ERR_INVALID;
    uint64_t cnt = (uint64_t)rows[i] * (uint64_t)k_blocks;
    if (cnt > 0 && !scales[i]) return NVFP4_ERR_NULL;
    a.scales[i] = scales[i];
    a.offset[i] = off;
    a.gs[i] = gs_in[i];
    off += cnt;
  }
  if (off >= ((uint64_t)1 << 40)) return NVFP4_ERR_SHAPE;
  a.total = off;
  a.gs_shared = gs_shared;
  launch_fuse_rescale(a, (hipStream_t)stream);
  return launched();
}

// The contraction kernels address up to 256 rows of the fp16 activations
// (the tile GEMM) or up to 16 (the GEMV forms) from a base with 32-bit
// offsets, so a row may not reach 2^24 bytes.
static bool tile_rows_ok(int64_t K) { return (uint64_t)round_up(K, kGemmBK) * 2u < kMaxTileRowBytes; }

// The tile GEMM (M > 16, or the FP8 weights' long-K path) needs its tile
// count in range.  Arguments already below 2^31.
static bool tiles_ok(int64_t M, int64_t N) { return gemm_tiles(M, N) <= kMaxGemmTiles; }

// Shapes every linear's size function accepts; anything else sizes to 0,
// which the entry point then rejects with its own status.
static bool dims_ok(int64_t M, int64_t N, int64_t K) {
  return M >= 0 && N >= 0 && K >= 0 && M < kMaxDim && N < kMaxDim && K < kMaxDim && tiles_ok(M, N);
}

// Workspace: absmax partials | gs_x | fp16 activations [Mp, Kp] | fp32 K-part
// sums of the split tiles (see plan_gemm).
static size_t x16_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0) return 0;
  int64_t Mp = M <= kGemvMaxM ? M : round_up(M, kGemmBM);
  return (size_t)round_up((int64_t)Mp * round_up(K, kGemmBK) * 2, 256);
}

static size_t partial_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= kGemvMaxM || N <= 0 || K <= 0) return 0;
  return plan_gemm(M, N, K).partial_bytes;
}

// Up to four prepared rows also keep their packed codes ([M][K/2]) and scale
// bytes ([M][K/16]) after the fp16 operand, for the FP4 GEMV of
// nvfp4_gemm_run, where it has a form for the shape.
static bool keeps_codes(int64_t M, int64_t K) { return gemv_fp4_has_form(M, K); }
static size_t q_offset(int64_t M, int64_t K) { return kWsX16 + x16_bytes(M, K); }
static size_t q_bytes(int64_t M, int64_t K) {
  return keeps_codes(M, K) ? (size_t)round_up(M * K / 16 * 9, 1024) : 0;
}
static size_t prepared_bytes(int64_t M, int64_t K) { return q_offset(M, K) + q_bytes(M, K); }

size_t nvfp4_gemm_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (!dims_ok(M, N, K) || !tile_rows_ok(K)) return 0;
  return prepared_bytes(M, K) + partial_bytes(M, N, K);
}

// W4A16 needs only the fp32 K-part sums of the split tiles.
size_t nvfp4_gemm_w4a16_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (!dims_ok(M, N, K)) return 0;
  return partial_bytes(M, N, round_up(K, kGemmBK));
}

nvfp4_status_t nvfp4_gemm_prepare(const void* x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  nvfp4_status_t st = check_input(x, x_dtype, M, K, ld_x);
  if (st != NVFP4_OK) return st;
  if (K % 64 != 0) return NVFP4_ERR_SHAPE;
  if (M == 0) return NVFP4_OK;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < prepared_bytes(M, K))
    return NVFP4_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const bool xb = x_dtype == NVFP4_BF16;
  uint32_t* partials = (uint32_t*)((char*)workspace + kWsPartials);
  float* gsx = (float*)((char*)workspace + kWsGs);
  void* x16 = (char*)workspace + kWsX16;
  int np = launch_amax(x, xb, M, K, ld_x, partials, s);
  uint8_t* q = keeps_codes(M, K) ? (uint8_t*)workspace + q_offset(M, K) : nullptr;
  launch_quantize_f16(x, xb, M, K, ld_x, round_up(K, kGemmBK), partials, np, nullptr, x16, gsx, q,
                      q ? q + M * K / 2 : nullptr, s);
  return launched();
}

nvfp4_status_t nvfp4_gemm_prepare_static(const void* x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                                         const float* gs_x, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  nvfp4_status_t st = check_input(x, x_dtype, M, K, ld_x);
  if (st != NVFP4_OK) return st;
  if (K % 64 != 0) return NVFP4_ERR_SHAPE;
  if (!gs_x) return NVFP4_ERR_NULL;
  if (M == 0) return NVFP4_OK;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < prepared_bytes(M, K))
    return NVFP4_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  float* gsx = (float*)((char*)workspace + kWsGs);
  void* x16 = (char*)workspace + kWsX16;
  uint8_t* q = keeps_codes(M, K) ? (uint8_t*)workspace + q_offset(M, K) : nullptr;
  launch_quantize_f16(x, x_dtype == NVFP4_BF16, M, K, ld_x, round_up(K, kGemmBK), nullptr, 0, gs_x, x16, gsx, q,
                      q ? q + M * K / 2 : nullptr, s);
  return launched();
}

nvfp4_status_t nvfp4_gemm_run(int64_t M, int64_t K, const uint8_t* w_codes, const uint8_t* w_scales,
                              const float* w_gs, int64_t N, void* y, nvfp4_dtype_t y_dtype, int64_t ld_y,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(y_dtype)) return NVFP4_ERR_DTYPE;
  if (!dims_ok(M, N, K)) return NVFP4_ERR_SHAPE;
  if (K % 64 != 0 || !tile_rows_ok(K)) return NVFP4_ERR_SHAPE;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!y || !w_gs) return NVFP4_ERR_NULL;
  if (ld_y < N) return NVFP4_ERR_SHAPE;
  if (!aligned(y, 16) || ((uint64_t)ld_y * esize(y_dtype)) % 16 != 0) return NVFP4_ERR_ALIGN;
  if (K > 0) {
    if (!w_codes || !w_scales) return NVFP4_ERR_NULL;
    if (!aligned(w_codes, 16) || !aligned(w_scales, 4)) return NVFP4_ERR_ALIGN;
  }
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < nvfp4_gemm_workspace_size(M, N, K))
    return NVFP4_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const bool yb = y_dtype == NVFP4_BF16;
  const float* gsx = (const float*)((const char*)workspace + kWsGs);
  const void* x16 = (const char*)workspace + kWsX16;
  void* wsv = workspace;
  const int64_t Kp = round_up(K, kGemmBK);
  if (keeps_codes(M, K) &&
      launch_gemv_fp4_prepared((const uint8_t*)workspace + q_offset(M, K), M, K, gsx, w_codes, w_scales, N, w_gs,
                               y, yb, (size_t)ld_y * esize(y_dtype), s))
    return launched();
  if (M <= kGemvMaxM)
    launch_gemv(false, x16, (size_t)Kp * 2, M, K, w_codes, w_scales, N, gsx, w_gs, y, yb, ld_y, s);
  else
    launch_gemm(false, x16, (size_t)Kp * 2, M, K, w_codes, w_scales, N, gsx, w_gs, y, yb, ld_y,
                (float*)((char*)wsv + kWsX16 + x16_bytes(M, K)), s);
  return launched();
}

// The checks nvfp4_gemm makes besides those of the activations and the
// workspace.
static nvfp4_status_t linear_args_ok(int64_t M, int64_t K, const uint8_t* w_codes, const uint8_t* w_scales,
                                     const float* w_gs, int64_t N, const void* y, nvfp4_dtype_t y_dtype,
                                     int64_t ld_y) {
  if (!dtype_ok(y_dtype)) return NVFP4_ERR_DTYPE;
  if (N < 0 || N >= kMaxDim || !tiles_ok(M, N)) return NVFP4_ERR_SHAPE;
  if (K % 64 != 0 || !tile_rows_ok(K)) return NVFP4_ERR_SHAPE;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!y || !w_gs) return NVFP4_ERR_NULL;
  if (ld_y < N) return NVFP4_ERR_SHAPE;
  if (!aligned(y, 16) || ((uint64_t)ld_y * esize(y_dtype)) % 16 != 0) return NVFP4_ERR_ALIGN;
  if (K > 0) {
    if (!w_codes || !w_scales) return NVFP4_ERR_NULL;
    if (!aligned(w_codes, 16) || !aligned(w_scales, 4)) return NVFP4_ERR_ALIGN;
  }
  return NVFP4_OK;
}

static nvfp4_status_t run_args_ok(int64_t M, int64_t K, const uint8_t* w_codes, const uint8_t* w_scales,
                                  const float* w_gs, int64_t N, const void* y, nvfp4_dtype_t y_dtype,
                                  int64_t ld_y, const void* workspace, size_t workspace_bytes) {
  nvfp4_status_t st = linear_args_ok(M, K, w_codes, w_scales, w_gs, N, y, y_dtype, ld_y);
  if (st != NVFP4_OK || M == 0 || N == 0) return st;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < nvfp4_gemm_workspace_size(M, N, K))
    return NVFP4_ERR_WORKSPACE;
  return NVFP4_OK;
}

// Up to four bf16 activation rows (decode): the quantize and the GEMV in one
// launch, which also leaves the quantized rows and gs_x in the workspace as
// nvfp4_gemm_prepare would.  False when the shape has no such form
// (nothing launched); arguments already validated.
static bool fused_decode(const void* x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                         const float* gs_x, const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gs,
                         int64_t N, void* y, nvfp4_dtype_t y_dtype, int64_t ld_y, void* workspace, void* stream) {
  if (x_dtype != NVFP4_BF16 || !keeps_codes(M, K)) return false;
  return launch_gemv_fp4(x, true, M, K, (size_t)ld_x * 2u, gs_x, w_codes, w_scales, N, w_gs, y,
                         y_dtype == NVFP4_BF16, (size_t)ld_y * esize(y_dtype), (char*)workspace + kWsX16,
                         (float*)((char*)workspace + kWsGs), (uint8_t*)workspace + q_offset(M, K),
                         (hipStream_t)stream);
}

nvfp4_status_t nvfp4_gemm(const void* x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                          const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gs, int64_t N, void* y,
                          nvfp4_dtype_t y_dtype, int64_t ld_y, void* workspace, size_t workspace_bytes,
                          void* stream) {
  // validate everything before the first launch
  nvfp4_status_t st = check_input(x, x_dtype, M, K, ld_x);
  if (st != NVFP4_OK) return st;
  st = run_args_ok(M, K, w_codes, w_scales, w_gs, N, y, y_dtype, ld_y, workspace, workspace_bytes);
  if (st != NVFP4_OK || M == 0 || N == 0) return st;
  if (fused_decode(x, x_dtype, M, K, ld_x, nullptr, w_codes, w_scales, w_gs, N, y, y_dtype, ld_y, workspace, stream))
    return launched();
  st = nvfp4_gemm_prepare(x, x_dtype, M, K, ld_x, workspace, workspace_bytes, stream);
  if (st != NVFP4_OK) return st;
  return nvfp4_gemm_run(M, K, w_codes, w_scales, w_gs, N, y, y_dtype, ld_y, workspace, workspace_bytes, stream);
}

nvfp4_status_t nvfp4_gemm_static(const void* x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                                 const float* gs_x, const uint8_t* w_codes, const uint8_t* w_scales,
                                 const float* w_gs, int64_t N, void* y, nvfp4_dtype_t y_dtype, int64_t ld_y,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  // validate everything before launching anything
  nvfp4_status_t st = check_input(x, x_dtype, M, K, ld_x);
  if (st != NVFP4_OK) return st;
  if (!gs_x) return NVFP4_ERR_NULL;
  st = run_args_ok(M, K, w_codes, w_scales, w_gs, N, y, y_dtype, ld_y, workspace, workspace_bytes);
  if (st != NVFP4_OK || M == 0 || N == 0) return st;
  if (fused_decode(x, x_dtype, M, K, ld_x, gs_x, w_codes, w_scales, w_gs, N, y, y_dtype, ld_y, workspace, stream))
    return launched();
  st = nvfp4_gemm_prepare_static(x, x_dtype, M, K, ld_x, gs_x, workspace, workspace_bytes, stream);
  if (st != NVFP4_OK) return st;
  return nvfp4_gemm_run(M, K, w_codes, w_scales, w_gs, N, y, y_dtype, ld_y, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------- no-alloc
// nvfp4_gemm_noalloc: nvfp4_gemm with its workspace in a fixed array of the
// library instead of a caller buffer, for callers that cannot allocate.
// Each device holds its own copy of `scratch`; host code reaches it only
// through the device address hipGetSymbolAddress returns on that device (the
// array's name is a host-side stand-in there), taken on the first call on a
// device and kept per device.
static __device__ __align__(256) uint8_t scratch[NVFP4_NOALLOC_SCRATCH_BYTES];

static void* scratch_address() {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = cached[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
  cached[dev].store(q, std::memory_order_release);  // every thread finds the same address
  return q;
}

nvfp4_status_t nvfp4_gemm_noalloc(const void* x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                                  const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gs, int64_t N,
                                  void* y, nvfp4_dtype_t y_dtype, int64_t ld_y, void* stream) {
  // the shape checks of nvfp4_gemm come first, so the workspace size below
  // is computed for a valid shape
  nvfp4_status_t st = check_input(x, x_dtype, M, K, ld_x);
  if (st != NVFP4_OK) return st;
  st = linear_args_ok(M, K, w_codes, w_scales, w_gs, N, y, y_dtype, ld_y);
  if (st != NVFP4_OK || M == 0 || N == 0) return st;
  const size_t need = nvfp4_gemm_workspace_size(M, N, K);
  if (need > (size_t)NVFP4_NOALLOC_SCRATCH_BYTES) return NVFP4_ERR_WORKSPACE;
  void* ws = scratch_address();
  if (!ws) return NVFP4_ERR_DEVICE;
  return nvfp4_gemm(x, x_dtype, M, K, ld_x, w_codes, w_scales, w_gs, N, y, y_dtype, ld_y, ws,
                    (size_t)NVFP4_NOALLOC_SCRATCH_BYTES, stream);
}

size_t nvfp4_fp8_quantize_workspace_size(int64_t rows, int64_t K) { return nvfp4_quantize_workspace_size(rows, K); }

nvfp4_status_t nvfp4_fp8_quantize(const void* x, nvfp4_dtype_t x_dtype, int64_t rows, int64_t K, int64_t ld_x,
                                  uint8_t* q, float* scale, void* workspace, size_t workspace_bytes, void* stream) {
  nvfp4_status_t st = check_input(x, x_dtype, rows, K, ld_x);
  if (st != NVFP4_OK) return st;
  if (!scale) return NVFP4_ERR_NULL;
  hipStream_t s = (hipStream_t)stream;
  if (rows == 0 || K == 0) {
    launch_fill_f32(scale, 0.0f, s);
    return launched();
  }
  if (!q) return NVFP4_ERR_NULL;
  if (!aligned(q, 16)) return NVFP4_ERR_ALIGN;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < nvfp4_fp8_quantize_workspace_size(rows, K))
    return NVFP4_ERR_WORKSPACE;
  uint32_t* partials = (uint32_t*)((char*)workspace + kWsPartials);
  const bool xb = x_dtype == NVFP4_BF16;
  const int np = launch_amax(x, xb, rows, K, ld_x, partials, s);
  launch_fp8_quantize(x, xb, rows, K, ld_x, partials, np, nullptr, q, scale, s);
  return launched();
}

nvfp4_status_t nvfp4_fp8_quantize_static(const void* x, nvfp4_dtype_t x_dtype, int64_t rows, int64_t K,
                                         int64_t ld_x, const float* scale, uint8_t* q, void* stream) {
  nvfp4_status_t st = check_input(x, x_dtype, rows, K, ld_x);
  if (st != NVFP4_OK) return st;
  if (!scale) return NVFP4_ERR_NULL;
  if (rows == 0 || K == 0) return NVFP4_OK;
  if (!q) return NVFP4_ERR_NULL;
  if (!aligned(q, 16)) return NVFP4_ERR_ALIGN;
  launch_fp8_quantize(x, x_dtype == NVFP4_BF16, rows, K, ld_x, nullptr, 0, scale, q, nullptr, (hipStream_t)stream);
  return launched();
}

nvfp4_status_t nvfp4_fp8_dequantize(const uint8_t* q, const float* scale, int64_t rows, int64_t K, void* out,
                                    nvfp4_dtype_t out_dtype, int64_t ld_out, void* stream) {
  if (!dtype_ok(out_dtype)) return NVFP4_ERR_DTYPE;
  if (rows < 0 || K < 0 || rows >= kMaxDim || K >= kMaxDim || K % 16 != 0) return NVFP4_ERR_SHAPE;
  if (rows == 0 || K == 0) return NVFP4_OK;
  if (!q || !scale || !out) return NVFP4_ERR_NULL;
  if (ld_out < K) return NVFP4_ERR_SHAPE;
  if ((uint64_t)rows * (uint64_t)(K / 16) >= kMaxBlocks) return NVFP4_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(out, 16) || ((uint64_t)ld_out * esize(out_dtype)) % 16 != 0)
    return NVFP4_ERR_ALIGN;
  launch_fp8_dequant(q, scale, rows, K, out, out_dtype == NVFP4_BF16, ld_out, (hipStream_t)stream);
  return launched();
}

// FP8-weight linears.  Workspace: absmax partials | s_x | X in E4M3 [M, K]
// (W8A8 only) | fp32 K-part sums of the split tiles.
static size_t x8_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0) return 0;
  return (size_t)round_up(M * K, 256);
}

size_t nvfp4_gemm_w8a16_workspace_size(int64_t M, int64_t N, int64_t K) {
  return nvfp4_gemm_w4a16_workspace_size(M, N, K);
}

size_t nvfp4_gemm_w8a8_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (!dims_ok(M, N, K)) return 0;
  return kWsX16 + x8_bytes(M, K) + partial_bytes(M, N, round_up(K, kGemmBK));
}

// Checks shared by the FP8-weight entry points (besides those of X).
static nvfp4_status_t fp8w_args_ok(int64_t M, int64_t K, const uint8_t* w_q, const float* w_scale, int64_t N,
                                   const void* y, nvfp4_dtype_t y_dtype, int64_t ld_y) {
  if (!dtype_ok(y_dtype)) return NVFP4_ERR_DTYPE;
  if (N < 0 || N >= kMaxDim || K % 64 != 0 || !tiles_ok(M, N)) return NVFP4_ERR_SHAPE;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!y || !w_scale) return NVFP4_ERR_NULL;
  if (ld_y < N) return NVFP4_ERR_SHAPE;
  if (!aligned(y, 16) || ((uint64_t)ld_y * esize(y_dtype)) % 16 != 0) return NVFP4_ERR_ALIGN;
  if (K > 0) {
    if (!w_q) return NVFP4_ERR_NULL;
    if (!aligned(w_q, 16)) return NVFP4_ERR_ALIGN;
    if ((uint64_t)N * (uint64_t)K >= ((uint64_t)1 << 32)) return NVFP4_ERR_SHAPE;
  }
  return NVFP4_OK;
}

static void fp8w_run(bool a8, const void* x, size_t ld_x_bytes, int64_t M, int64_t K, const uint8_t* w_q,
                     const float* sx, const float* sw, int64_t N, void* y, bool yb, int64_t ld_y, float* partials,
                     hipStream_t s) {
  if (M <= kGemvMaxM && K <= kFp8GemvMaxK && K > 0)
    launch_gemv_fp8w(a8, x, ld_x_bytes, M, K, w_q, N, sx, sw, y, yb, ld_y, s);
  else
    launch_gemm_fp8w(a8, x, ld_x_bytes, M, K, w_q, N, sx, sw, y, yb, ld_y, partials, s);
}

nvfp4_status_t nvfp4_gemm_w8a16(const void* x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                                const uint8_t* w_q, const float* w_scale, int64_t N, void* y, nvfp4_dtype_t y_dtype,
                                int64_t ld_y, void* workspace, size_t workspace_bytes, void* stream) {
  nvfp4_status_t st = check_input(x, x_dtype, M, K, ld_x);
  if (st != NVFP4_OK) return st;
  if (x_dtype != NVFP4_BF16) return NVFP4_ERR_DTYPE;
  if ((uint64_t)ld_x * 2u >= kMaxTileRowBytes) return NVFP4_ERR_SHAPE;
  st = fp8w_args_ok(M, K, w_q, w_scale, N, y, y_dtype, ld_y);
  if (st != NVFP4_OK || M == 0 || N == 0) return st;
  const size_t need = nvfp4_gemm_w8a16_workspace_size(M, N, K);
  if (need && (!workspace || !aligned(workspace, 256) || workspace_bytes < need)) return NVFP4_ERR_WORKSPACE;
  fp8w_run(false, x, (size_t)ld_x * 2, M, K, w_q, nullptr, w_scale, N, y, y_dtype == NVFP4_BF16, ld_y,
           (float*)workspace, (hipStream_t)stream);
  return launched();
}

nvfp4_status_t nvfp4_gemm_w8a8(const void* x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                               const float* x_scale, const uint8_t* w_q, const float* w_scale, int64_t N, void* y,
                               nvfp4_dtype_t y_dtype, int64_t ld_y, void* workspace, size_t workspace_bytes,
                               void* stream) {
  nvfp4_status_t st = check_input(x, x_dtype, M, K, ld_x);
  if (st != NVFP4_OK) return st;
  // the E4M3 activations (row stride K bytes) are addressed like the
  // activations of the other linears
  if ((uint64_t)K >= kMaxTileRowBytes) return NVFP4_ERR_SHAPE;
  st = fp8w_args_ok(M, K, w_q, w_scale, N, y, y_dtype, ld_y);
  if (st != NVFP4_OK || M == 0 || N == 0) return st;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < nvfp4_gemm_w8a8_workspace_size(M, N, K))
    return NVFP4_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const bool xb = x_dtype == NVFP4_BF16;
  uint32_t* amax_partials = (uint32_t*)((char*)workspace + kWsPartials);
  float* sx = (float*)((char*)workspace + kWsGs);
  uint8_t* x8 = (uint8_t*)workspace + kWsX16;
  float* split_partials = (float*)((char*)workspace + kWsX16 + x8_bytes(M, K));
  if (K > 0) {
    if (x_scale) {
      launch_fp8_quantize(x, xb, M, K, ld_x, nullptr, 0, x_scale, x8, sx, s);
    } else {
      const int np = launch_amax(x, xb, M, K, ld_x, amax_partials, s);
      launch_fp8_quantize(x, xb, M, K, ld_x, amax_partials, np, nullptr, x8, sx, s);
    }
  } else {
    launch_fill_f32(sx, 0.0f, s);
  }
  fp8w_run(true, x8, (size_t)K, M, K, w_q, sx, w_scale, N, y, y_dtype == NVFP4_BF16, ld_y, split_partials, s);
  return launched();
}

nvfp4_status_t nvfp4_gemm_w4a16(const void* x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                                const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gs, int64_t N,
                                void* y, nvfp4_dtype_t y_dtype, int64_t ld_y, void* workspace,
                                size_t workspace_bytes, void* stream) {
  nvfp4_status_t st = check_input(x, x_dtype, M, K, ld_x);
  if (st != NVFP4_OK) return st;
  if (x_dtype != NVFP4_BF16) return NVFP4_ERR_DTYPE;
  if (!dtype_ok(y_dtype)) return NVFP4_ERR_DTYPE;
  if (N < 0 || N >= kMaxDim || K % 64 != 0 || !tiles_ok(M, N)) return NVFP4_ERR_SHAPE;
  if ((uint64_t)ld_x * 2u >= kMaxTileRowBytes) return NVFP4_ERR_SHAPE;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!y || !w_gs) return NVFP4_ERR_NULL;
  if (ld_y < N) return NVFP4_ERR_SHAPE;
  if (!aligned(y, 16) || ((uint64_t)ld_y * esize(y_dtype)) % 16 != 0) return NVFP4_ERR_ALIGN;
  if (K > 0) {
    if (!w_codes || !w_scales) return NVFP4_ERR_NULL;
    if (!aligned(w_codes, 16) || !aligned(w_scales, 4)) return NVFP4_ERR_ALIGN;
  }
  const size_t need = nvfp4_gemm_w4a16_workspace_size(M, N, K);
  if (need && (!workspace || !aligned(workspace, 256) || workspace_bytes < need)) return NVFP4_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const bool yb = y_dtype == NVFP4_BF16;
  // K == 0 runs no K step (nothing of X or W is read) and stores zeros.
  const size_t ldb = (size_t)ld_x * 2;
  if (M <= kGemvMaxM)
    launch_gemv(true, x, ldb, M, K, w_codes, w_scales, N, nullptr, w_gs, y, yb, ld_y, s);
  else
    launch_gemm(true, x, ldb, M, K, w_codes, w_scales, N, nullptr, w_gs, y, yb, ld_y, (float*)workspace, s);
  return launched();
}

}  // extern "C"
