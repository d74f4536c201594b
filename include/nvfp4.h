/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 W4A4 linear-layer library.
 *
 * NVFP4 as used here (paper "Why Gated DeltaNet Survives 4-Bit Quantization:
 * NVFP4 W4A4 for the Recurrent Half of a Hybrid 27B LLM", section 2,
 * paragraph "NVFP4"): every value is an E2M1 code (4 bits), every 16
 * consecutive values along the input dimension K share one E4M3 block scale,
 * and the tensor carries one FP32 scale.  W4A4: weights and activations are
 * both quantized this way and the product is accumulated in FP32.
 *
 * Tensor layout (model card "Gemma-4-31B-IT-NVFP4-FP8attn-text", sections
 * "Verification" and "Serving the quantized weights"; blog "The winner used
 * 8-bit in the right place", section "We opened the tensors"):
 *   codes  uint8 [rows, K/2]   two E2M1 codes per byte; element 2j of a row
 *                              is the low nibble of byte j, element 2j+1 the
 *                              high nibble; bit 3 of a code is the sign.
 *   scales uint8 [rows, K/16]  E4M3 ("FN": bias 7, max 448, no infinity,
 *                              0x7F/0xFF NaN) block scales, row-major.
 *   gs     float (one)         FP32 tensor scale in dequant form:
 *                              value = E2M1(code) * E4M3(scale) * gs.
 *
 * Arithmetic of the quantizer, bit for bit (IEEE binary32, round to nearest
 * even, no fused multiply-add, subnormals kept; RN(.) = one rounding):
 *   gs  = RN(amax / 2688)                     amax = max |x| over the tensor
 *   sb  = E4M3(RN(bmax / RN(6 * gs)))         bmax = max |x| over the block;
 *                                             E4M3(.) rounds to nearest even
 *                                             and saturates at 448; sb = 0
 *                                             when gs == 0
 *   es  = RN(E4M3value(sb) * gs)
 *   mag = E2M1(RN(|x| / es)), nearest, ties to the even code, saturating at
 *         6; mag = 0 when es == 0
 *   code = signbit(x) << 3 | mag
 * 2688 = 6 * 448: the largest E2M1 magnitude times the largest E4M3 value,
 * which makes max(block scale) * gs * 6 reproduce the tensor's absmax (model
 * card, section "Verification").
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is a device pointer; every call is enqueued on
 *    `stream` (a hipStream_t, NULL = the default stream) and returns after
 *    the enqueue, without synchronizing.  Tensor scales travel as device
 *    scalars so that no call reads them on the host.
 *  - Arguments are checked on the host before anything is launched; on any
 *    error nothing is launched and a non-zero status is returned.  No call
 *    allocates device memory: scratch space comes from the caller's
 *    workspace, whose size the *_workspace_size functions give.  The library
 *    keeps no state between calls apart from a per-device cache of two device
 *    attributes (compute units, LDS per compute unit), safe to fill from
 *    several host threads at once.
 *  - The *_workspace_size functions return 0 for shapes outside the range
 *    their entry point accepts (negative sizes, a dimension of 2^31 or
 *    more, K too long, more than 2^30 256 x 256 output tiles); the entry
 *    point rejects those shapes with NVFP4_ERR_SHAPE.
 *  - Inputs must be finite (no NaN or infinity); this is not checked.
 *  - Calls that share a workspace, or whose outputs overlap their inputs,
 *    must be ordered by the caller (same stream, or events).
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nvfp4_status {
    NVFP4_OK = 0,
    NVFP4_ERR_NULL = 1,      /* a required pointer is NULL                    */
    NVFP4_ERR_SHAPE = 2,     /* negative size, K not a multiple of 16 (64 for
                                the GEMM), leading dimension too small, or a
                                size beyond 2^31 elements per dimension        */
    NVFP4_ERR_DTYPE = 3,     /* dtype argument not NVFP4_F32 / NVFP4_BF16      */
    NVFP4_ERR_ALIGN = 4,     /* pointer or leading dimension not 16-byte
                                aligned where stated                           */
    NVFP4_ERR_WORKSPACE = 5, /* workspace NULL, misaligned or too small        */
    NVFP4_ERR_INVALID = 6,   /* other invalid argument (member count out of
                                range, aliased outputs)                        */
    NVFP4_ERR_DEVICE = 7     /* the HIP runtime reported a launch error        */
} nvfp4_status_t;

/* The dtype arguments are int-sized; any int may arrive from a caller and is
 * checked (NVFP4_ERR_DTYPE).  C++ sees the int representation explicitly, so
 * that no value is outside the enumeration's range there either. */
#ifdef __cplusplus
typedef enum nvfp4_dtype : int {
#else
typedef enum nvfp4_dtype {
#endif
    NVFP4_F32 = 0,           /* IEEE binary32                                  */
    NVFP4_BF16 = 1           /* bfloat16 (upper half of a binary32)            */
} nvfp4_dtype_t;

/* Largest number of members nvfp4_fuse_rescale accepts in one group. */
#define NVFP4_MAX_FUSED 16

/* Human-readable name of a status code (static string, never NULL). */
const char *nvfp4_status_string(nvfp4_status_t status);

/* Library version, major * 10000 + minor * 100 + patch. */
int nvfp4_version(void);

/* ------------------------------------------------------------------------
 * nvfp4_quantize -- on-the-fly NVFP4 quantization of a [rows, K] tensor.
 * Paper, section 2 "NVFP4" (E2M1 values, one E4M3 scale per 16-element
 * block set to blockmax/6, one FP32 tensor scale); the arithmetic is the one
 * spelled out at the top of this header.  Used for activations at serving
 * time and, offline, for weights (one tensor scale per module, paper
 * section 3 "Checkpoints" and section 6).
 *
 *   x        device, [rows, ld_x] row-major, dtype x_dtype (F32 or BF16);
 *            16-byte aligned, ld_x * element size a multiple of 16 bytes.
 *   rows, K  rows >= 0, K >= 0, K % 16 == 0, ld_x >= K.
 *   codes    device out, [rows, K/2] uint8, dense.
 *   scales   device out, [rows, K/16] uint8, dense.
 *   gs       device out, one float: the tensor scale.
 *   workspace, workspace_bytes: device scratch of at least
 *            nvfp4_quantize_workspace_size(rows, K) bytes, 256-byte aligned.
 * rows == 0 or K == 0 writes gs = 0 and nothing else.  The result is
 * deterministic and independent of the launch configuration.
 * ---------------------------------------------------------------------- */
size_t nvfp4_quantize_workspace_size(int64_t rows, int64_t K);

nvfp4_status_t nvfp4_quantize(const void *x, nvfp4_dtype_t x_dtype, int64_t rows, int64_t K,
                              int64_t ld_x, uint8_t *codes, uint8_t *scales, float *gs,
                              void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * nvfp4_dequantize -- two-level dequant (paper section 5, "fake
 * quantization": quantize, dequantize, continue in high precision; model
 * card sections "Verification" and "Limitations": expansion to BF16).
 *   out[r, k] = RN_fp32(E2M1(code) * E4M3(scale) * gs)   for NVFP4_F32
 *   out[r, k] = RN_bf16(that fp32 value)                 for NVFP4_BF16
 * (E2M1 * E4M3 is exact; one fp32 rounding for the product with gs.)
 *   codes [rows, K/2], scales [rows, K/16], gs one device float;
 *   out   device, [rows, ld_out] row-major, 16-byte aligned,
 *         ld_out * element size a multiple of 16 bytes, ld_out >= K.
 * ---------------------------------------------------------------------- */
nvfp4_status_t nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales, const float *gs,
                                int64_t rows, int64_t K, void *out, nvfp4_dtype_t out_dtype,
                                int64_t ld_out, void *stream);

/* ------------------------------------------------------------------------
 * nvfp4_fuse_rescale -- repair of a fused group (paper section 6, paragraph
 * "Per-module calibration vs. fused-GEMM scaling"): modules calibrated with
 * their own tensor scales but served as one GEMM are moved onto the shared
 * scale S = max_i gs_i, with the ratio folded into their E4M3 block scales:
 *   rho_i = RN(gs_i / S)        (rho_i = 1 when S == 0)
 *   byte  <- sign | E4M3(RN(E4M3value(byte & 0x7F) * rho_i))
 * Bytes 0x7F / 0xFF (NaN) are left unchanged; the member with gs_i == S is
 * left byte-identical.  Codes are never touched.  After the call the fused
 * weight is the row-concatenation of the members' codes and (rewritten)
 * scales, with tensor scale *gs_shared.
 *   n          1 <= n <= NVFP4_MAX_FUSED members.
 *   scales     host array of n device pointers, member i: [rows[i], k_blocks]
 *              uint8, rewritten in place.  Members must not overlap.
 *   rows       host array of n row counts (>= 0).
 *   k_blocks   K/16 (>= 0), the same for every member.
 *   gs_in      host array of n device pointers to the members' tensor scales.
 *   gs_shared  device out, one float; must not alias any gs_in[i].
 * ---------------------------------------------------------------------- */
nvfp4_status_t nvfp4_fuse_rescale(int n, uint8_t *const *scales, const int64_t *rows,
                                  int64_t k_blocks, const float *const *gs_in, float *gs_shared,
                                  void *stream);

/* ------------------------------------------------------------------------
 * nvfp4_gemm -- the W4A4 linear layer Y = X * W^T (paper section 2: both
 * operands NVFP4, the GEMM accumulates in FP32).  X is quantized on the fly
 * exactly as nvfp4_quantize does (tensor scale gs_x from this X), W comes
 * pre-quantized (codes, scales, *w_gs).  Then
 *   y[m, n] = RN_out( RN_fp32( acc[m, n] * RN(gs_x * gs_w) ) )
 *   acc[m, n] = sum_k (E2M1 x_code * E4M3 x_scale)(E2M1 w_code * E4M3 w_scale)
 * accumulated in FP32 (the products are exact; the order of the sum is the
 * kernel's, so results match the exact sum to FP32 accumulation accuracy).
 *
 *   x        device [M, ld_x] row-major, F32 or BF16; 16-byte aligned,
 *            ld_x * element size a multiple of 16 bytes, ld_x >= K.
 *   M, K, N  >= 0; K % 64 == 0 (the GEMM advances K 64 at a time, which
 *            is 4 scale bytes, one aligned dword, per weight row); K below
 *            2^23 (the quantized activations are addressed with 32-bit
 *            offsets), else NVFP4_ERR_SHAPE.
 *   w_codes  device [N, K/2] uint8 dense, 16-byte aligned.
 *   w_scales device [N, K/16] uint8 dense, 4-byte aligned.
 *   w_gs     device, one float.  For a fused weight: the gs_shared of
 *            nvfp4_fuse_rescale.
 *   y        device out [M, ld_y] row-major, F32 or BF16; 16-byte aligned,
 *            ld_y * element size a multiple of 16 bytes, ld_y >= N.
 *   workspace: nvfp4_gemm_workspace_size(M, N, K) bytes, 256-byte aligned.
 * Empty problems (M, N == 0) launch nothing; K == 0 writes zeros.
 * ---------------------------------------------------------------------- */
size_t nvfp4_gemm_workspace_size(int64_t M, int64_t N, int64_t K);

nvfp4_status_t nvfp4_gemm(const void *x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K,
                          int64_t ld_x, const uint8_t *w_codes, const uint8_t *w_scales,
                          const float *w_gs, int64_t N, void *y, nvfp4_dtype_t y_dtype,
                          int64_t ld_y, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * nvfp4_gemm in two halves, for callers that multiply one activation by
 * several weights (unfused q/k/v or gate/up: paper section 6 describes the
 * fused alternative) or that time the contraction alone.
 *
 * nvfp4_gemm_prepare quantizes X exactly as nvfp4_gemm does and leaves the
 * quantized operand and gs_x in the workspace (arguments as in nvfp4_gemm).
 * nvfp4_gemm_run then computes Y = X W^T from that workspace; it may be
 * called any number of times with different weights (same M and K) until
 * the workspace is reused.  nvfp4_gemm_prepare needs
 * nvfp4_gemm_workspace_size(M, 0, K) bytes; nvfp4_gemm_run needs
 * nvfp4_gemm_workspace_size(M, N, K), whose part past the prepared
 * activations it uses as scratch (so runs sharing one workspace must be
 * ordered).  The pair is equivalent to one nvfp4_gemm call.
 *
 * A prepared workspace holds, at byte 8192, gs_x (one float) and, from byte
 * 8448, the quantized activations as fp16 values E2M1(code) * E4M3(scale)
 * (exact; gs_x not applied), row-major [M, K] with a row stride of 2K bytes.
 * Up to four rows with K = 4096 or 5120 also keep their packed codes
 * ([M, K/2]) and then their scale bytes ([M, K/16]) right after the fp16
 * operand (whose size is rounded up to 256 bytes), which nvfp4_gemm_run
 * contracts directly on the FP4 MFMA.  For such shapes nvfp4_gemm with bf16
 * rows does the whole step in one launch and leaves the same workspace.
 * The layout is stable, so callers and tests may inspect the operand.
 * ---------------------------------------------------------------------- */
nvfp4_status_t nvfp4_gemm_prepare(const void *x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K,
                                  int64_t ld_x, void *workspace, size_t workspace_bytes,
                                  void *stream);

nvfp4_status_t nvfp4_gemm_run(int64_t M, int64_t K, const uint8_t *w_codes,
                              const uint8_t *w_scales, const float *w_gs, int64_t N, void *y,
                              nvfp4_dtype_t y_dtype, int64_t ld_y, void *workspace,
                              size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * nvfp4_gemm_noalloc -- nvfp4_gemm for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments and result as
 * nvfp4_gemm without the workspace: its scratch (absmax partials, gs_x, the
 * quantized activations, split-K partial sums) lives in a fixed array of
 * NVFP4_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs
 * on until the process ends.  Shapes whose nvfp4_gemm_workspace_size exceeds
 * that size give NVFP4_ERR_WORKSPACE (the 4096 x 17408 x 5120 prefill needs
 * about 109 MB, most of it the split-K partial sums of its last tiles).  Every call on one device shares the array: calls that
 * overlap on a device (different streams, concurrent graphs) race and must
 * be ordered by the caller.  Nothing of the array needs to start at zero.
 * The first call on a device looks up the array's device address (no
 * allocation).
 * ---------------------------------------------------------------------- */
#define NVFP4_NOALLOC_SCRATCH_BYTES (128u << 20)

nvfp4_status_t nvfp4_gemm_noalloc(const void *x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K,
                                  int64_t ld_x, const uint8_t *w_codes, const uint8_t *w_scales,
                                  const float *w_gs, int64_t N, void *y, nvfp4_dtype_t y_dtype,
                                  int64_t ld_y, void *stream);

/* ------------------------------------------------------------------------
 * Static (calibrated) activation scale.  The checkpoints of the paper are
 * produced by a calibration tool that fixes one FP32 global scale per
 * module (paper section 3 "Checkpoints", section 6 "Per-module calibration
 * vs. fused-GEMM scaling"); served that way, the activation quantize needs
 * no absmax pass: one read of X instead of two, one launch at decode.
 *
 * nvfp4_quantize_static quantizes X with the given tensor scale *gs (a
 * device float, finite and >= 0): block scales and codes follow the same
 * rules as nvfp4_quantize with gs in place of RN(amax / 2688), saturating at
 * 448 and 6 where |x| exceeds what gs allows.  No workspace is needed and gs
 * is not written.  rows == 0 or K == 0 does nothing.
 *
 * nvfp4_gemm_prepare_static is nvfp4_gemm_prepare with the activation
 * tensor scale given by *gs_x (copied into the workspace, so nvfp4_gemm_run
 * is used unchanged); nvfp4_gemm_static is the pair in one call (arguments
 * as in nvfp4_gemm).  A negative or non-finite scale gives unspecified
 * codes.
 * ---------------------------------------------------------------------- */
nvfp4_status_t nvfp4_quantize_static(const void *x, nvfp4_dtype_t x_dtype, int64_t rows, int64_t K,
                                     int64_t ld_x, const float *gs, uint8_t *codes, uint8_t *scales,
                                     void *stream);

nvfp4_status_t nvfp4_gemm_prepare_static(const void *x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K,
                                         int64_t ld_x, const float *gs_x, void *workspace,
                                         size_t workspace_bytes, void *stream);

nvfp4_status_t nvfp4_gemm_static(const void *x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K,
                                 int64_t ld_x, const float *gs_x, const uint8_t *w_codes,
                                 const uint8_t *w_scales, const float *w_gs, int64_t N, void *y,
                                 nvfp4_dtype_t y_dtype, int64_t ld_y, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* ----------------------------------------------------------------------
 * W4A16: NVFP4 weights against 16-bit activations.  The model card
 * "Gemma-4-31B-IT-NVFP4-FP8attn-text", section "Limitations", notes that
 * without native FP4 tensor cores the NVFP4 weights are served as W4A16
 * (the activations stay in 16 bits and are never quantized); the weight
 * format is the paper's (section 2 "NVFP4").
 *
 * nvfp4_gemm_w4a16 computes Y[m, n] = gs_w * sum_k X[m, k] * E2M1(code[n, k])
 * * E4M3(scale[n, k / 16]) with FP32 accumulation, X taken as given.
 *   x        [M, ld_x] bf16 (x_dtype must be NVFP4_BF16), 16-byte aligned
 *            rows; no activation quantization, so no tensor scale for X.
 *   K        a multiple of 64.
 *   w_codes, w_scales, w_gs, N, y, y_dtype, ld_y: as in nvfp4_gemm.
 *   ld_x     below 2^23 elements (rows are addressed with 32-bit offsets).
 *   workspace: nvfp4_gemm_w4a16_workspace_size(M, N, K) bytes, 256-byte
 *            aligned; it may be NULL when that size is 0 (always for
 *            M <= 16).
 * Errors as in nvfp4_gemm; fp32 activations give NVFP4_ERR_DTYPE.  M == 0
 * or N == 0 does nothing; K == 0 stores zeros.
 * ---------------------------------------------------------------------- */
size_t nvfp4_gemm_w4a16_workspace_size(int64_t M, int64_t N, int64_t K);

nvfp4_status_t nvfp4_gemm_w4a16(const void *x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                                const uint8_t *w_codes, const uint8_t *w_scales, const float *w_gs,
                                int64_t N, void *y, nvfp4_dtype_t y_dtype, int64_t ld_y, void *workspace,
                                size_t workspace_bytes, void *stream);

/* ----------------------------------------------------------------------
 * FP8 E4M3 with one per-tensor scale.  The model card
 * "Gemma-4-31B-IT-NVFP4-FP8attn-text", section "What was quantized,
 * exactly", stores attention weights as float8_e4m3 with one scale per
 * tensor; the paper's section 7 "KV-cache precision" stores the KV cache in
 * FP8 with static (calibrated) per-tensor scales.
 *
 * Byte = sign(x) << 7 | E4M3(RN(|x| / s)), E4M3 rounding to nearest even and
 * saturating at 448 (0x7E); s == 0 keeps only sign bits.  Dequant value =
 * RN(E4M3(byte) * s).  Bytes are [rows, K] contiguous (row stride K), q
 * 16-byte aligned; K % 16 == 0.  x as in nvfp4_quantize.
 *
 * nvfp4_fp8_quantize: s = RN(amax / 448) over the whole tensor, written to
 *   *scale (device float); workspace of nvfp4_fp8_quantize_workspace_size
 *   bytes, 256-byte aligned.  rows == 0 or K == 0 writes scale 0.
 * nvfp4_fp8_quantize_static: s = *scale (device float, finite and >= 0),
 *   e.g. a calibrated KV-cache scale; no workspace, nothing else written.
 * nvfp4_fp8_dequantize: out [rows, ld_out] fp32, or bf16 (the RNE of the
 *   fp32 value), 16-byte aligned rows.
 * ---------------------------------------------------------------------- */
size_t nvfp4_fp8_quantize_workspace_size(int64_t rows, int64_t K);

nvfp4_status_t nvfp4_fp8_quantize(const void *x, nvfp4_dtype_t x_dtype, int64_t rows, int64_t K, int64_t ld_x,
                                  uint8_t *q, float *scale, void *workspace, size_t workspace_bytes,
                                  void *stream);

nvfp4_status_t nvfp4_fp8_quantize_static(const void *x, nvfp4_dtype_t x_dtype, int64_t rows, int64_t K,
                                         int64_t ld_x, const float *scale, uint8_t *q, void *stream);

nvfp4_status_t nvfp4_fp8_dequantize(const uint8_t *q, const float *scale, int64_t rows, int64_t K, void *out,
                                    nvfp4_dtype_t out_dtype, int64_t ld_out, void *stream);

/* ----------------------------------------------------------------------
 * Linears with FP8 E4M3 weights (one per-tensor scale, as produced by
 * nvfp4_fp8_quantize).  The model card "Gemma-4-31B-IT-NVFP4-FP8attn-text",
 * section "What was quantized, exactly", serves its float8_e4m3 attention
 * weights against bf16 activations (W8A16); W8A8 quantizes the activations
 * to FP8 as well, with one per-tensor scale.
 *
 *   w_q      [N, K] E4M3 bytes, row stride K, 16-byte aligned; N * K < 2^32.
 *   w_scale  device float: the weight tensor scale s_w.
 *   K        a multiple of 64.  y, y_dtype, ld_y as in nvfp4_gemm.
 *
 * nvfp4_gemm_w8a16: Y = s_w * X . E4M3(W)^T with FP32 accumulation, X
 *   [M, ld_x] bf16 as given, ld_x below 2^23.  Workspace nvfp4_gemm_w8a16_workspace_size
 *   bytes (0 for M <= 16; NULL allowed then).
 * nvfp4_gemm_w8a8: X is quantized to E4M3 with one per-tensor scale s_x
 *   (x_scale: a device float, e.g. calibrated, or NULL for RN(amax / 448),
 *   exactly as nvfp4_fp8_quantize), then Y = RN(s_x * s_w) * sum of
 *   E4M3(X) E4M3(W) products with FP32 accumulation; x bf16 or fp32;
 *   K below 2^24.
 *   Workspace nvfp4_gemm_w8a8_workspace_size bytes, 256-byte aligned.
 * Errors as in nvfp4_gemm.
 * ---------------------------------------------------------------------- */
size_t nvfp4_gemm_w8a16_workspace_size(int64_t M, int64_t N, int64_t K);
size_t nvfp4_gemm_w8a8_workspace_size(int64_t M, int64_t N, int64_t K);

nvfp4_status_t nvfp4_gemm_w8a16(const void *x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                                const uint8_t *w_q, const float *w_scale, int64_t N, void *y,
                                nvfp4_dtype_t y_dtype, int64_t ld_y, void *workspace, size_t workspace_bytes,
                                void *stream);

nvfp4_status_t nvfp4_gemm_w8a8(const void *x, nvfp4_dtype_t x_dtype, int64_t M, int64_t K, int64_t ld_x,
                               const float *x_scale, const uint8_t *w_q, const float *w_scale, int64_t N, void *y,
                               nvfp4_dtype_t y_dtype, int64_t ld_y, void *workspace, size_t workspace_bytes,
                               void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
