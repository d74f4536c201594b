/*
 * NVFP4 oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow CPU statement of what the NVFP4 W4A4 linear layer computes.
 * It exists so that tests, the smoke check and the CPU baseline of the bench
 * have an independent answer to compare the HIP library against.  Nothing in
 * the product path may load or call it, and it shares no code, header, table
 * or helper with the HIP sources.
 *
 * Source of the method: "Why Gated DeltaNet Survives 4-Bit Quantization:
 * NVFP4 W4A4 for the Recurrent Half of a Hybrid 27B LLM" (arXiv 2609.04098),
 * section 2 "Background", paragraph "NVFP4": values are E2M1 (4 bits), one
 * E4M3 scale per 16-element block set to blockmax/6 (in units of the tensor
 * scale), one FP32 scale per tensor; weights and activations are both
 * quantized this way (W4A4).  Section 6, paragraph "Per-module calibration vs.
 * fused-GEMM scaling": fused modules are repaired by moving every member onto
 * the shared global scale and folding the ratio into the per-block E4M3
 * scales.  The model card "Gemma-4-31B-IT-NVFP4-FP8attn-text", section
 * "Verification": max(block scale) x tensor scale x 6 reproduces the original
 * absmax, 6.0 being the largest E2M1 magnitude.
 *
 * Readings where the pages are silent (each stated once more where used):
 *   R1 tensor scale gs = RN(amax / 2688), 2688 = 6 * 448, 448 = largest E4M3.
 *   R2 block scale byte = E4M3(RN(bmax / RN(6 * gs))), round to nearest,
 *      ties to even, saturating at 448; if gs == 0 every scale byte is 0.
 *   R3 element code: es = RN(dec(scale) * gs); r = RN(|x| / es); magnitude =
 *      nearest E2M1 value, ties to even code, saturating at 6; es == 0 gives
 *      magnitude 0.  The sign bit is the sign bit of x (so -0.0 keeps it).
 *   R4 packing: element 2j of a row is the low nibble of byte j.
 *   R5 scales are one byte per block, row-major [rows, K/16].
 *   R6 fused repair: S = max gs_i; rho_i = RN(gs_i / S) (1 when S == 0);
 *      byte <- E4M3(RN(dec(byte) * rho_i)), sign bit and NaN bytes kept.
 *   R7 all fp32 steps are single IEEE binary32 operations rounded to nearest
 *      even, without fused multiply-add and with subnormals kept.  Build with
 *      -O2 -ffp-contract=off, never -ffast-math.
 *
 * The GEMM is computed exactly: every E2M1 x E4M3 value is an integer times
 * 2^-10 with magnitude below 2^22, so a product of two is an integer times
 * 2^-20 and a K-long sum of them is exact in int64 for K < 2^19.  The exact
 * sum is then scaled by gs_x * gs_w in fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------------- */
/* Format definitions                                                     */
/* ---------------------------------------------------------------------- */

/* E2M1 (OCP MX element format FP4): 1 sign bit, 2 exponent bits with bias
 * 1, 1 mantissa bit, no infinities or NaN.  Exponent field 0 is subnormal:
 * value m * 0.5.  Otherwise (1 + m/2) * 2^(e-1).  Largest magnitude 6.0. */
double orc_e2m1_decode(unsigned code)
{
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, (int)e - 1);
    return s ? -mag : mag;
}

/* E4M3 "FN" (OCP 8-bit floating point): 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits.  Exponent field 0 is subnormal: m * 2^-9.  The
 * all-ones pattern S.1111.111 is NaN; there is no infinity, so the largest
 * finite magnitude is 1.75 * 2^8 = 448 (byte 0x7E). */
double orc_e4m3_decode(unsigned byte)
{
    unsigned s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

/* Nearest finite non-negative E4M3 value to v >= 0, ties to the even byte
 * (the byte's lowest bit is the mantissa's lowest bit), saturating: every v
 * at or above 448 maps to 448.  Found by trying all 127 candidates.
 * Exactness: for v < 448 every distance that can decide a tie is computed
 * without rounding in fp64 (a tie needs v to sit at a midpoint of two
 * candidates, where v has few significant bits); far from midpoints a
 * rounded distance cannot change which candidate is nearer. */
unsigned orc_e4m3_encode(float v)
{
    unsigned best = 0, b;
    double bestd = INFINITY;
    if (v >= 448.0f)
        return 0x7Eu;
    for (b = 0; b <= 0x7Eu; ++b) {
        double d = fabs((double)v - orc_e4m3_decode(b));
        if (d < bestd || (d == bestd && (b & 1u) == 0)) {
            best = b;
            bestd = d;
        }
    }
    return best;
}

/* Nearest E2M1 magnitude code (0..7) to r >= 0, ties to the even code,
 * saturating at 6.0 (code 7) for every r >= 6, +inf included.  Same
 * exactness argument as the E4M3 search. */
unsigned orc_e2m1_encode_mag(float r)
{
    unsigned best = 0, c;
    double bestd = INFINITY;
    if (r >= 6.0f)
        return 7u;
    for (c = 0; c < 8u; ++c) {
        double d = fabs((double)r - orc_e2m1_decode(c));
        if (d < bestd || (d == bestd && (c & 1u) == 0)) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

void orc_e4m3_encode_many(const float *v, int64_t n, uint8_t *out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        out[i] = (uint8_t)orc_e4m3_encode(v[i]);
}

void orc_e2m1_encode_many(const float *r, int64_t n, uint8_t *out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        out[i] = (uint8_t)orc_e2m1_encode_mag(r[i]);
}

/* ---------------------------------------------------------------------- */
/* Quantize (paper section 2 "NVFP4"; readings R1-R5, R7)                 */
/* ---------------------------------------------------------------------- */

/* Widen element (r, k) to fp32.  bf16 is the upper half of an fp32, so the
 * widening is exact. */
static float load_elem(const void *x, int is_bf16, int64_t ld, int64_t r, int64_t k)
{
    if (is_bf16) {
        uint32_t bits = (uint32_t)((const uint16_t *)x)[r * ld + k] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return f;
    }
    return ((const float *)x)[r * ld + k];
}

float orc_tensor_scale(const void *x, int is_bf16, int64_t rows, int64_t K, int64_t ld)
{
    float amax = 0.0f;
    int64_t r;
#pragma omp parallel for schedule(static) reduction(max : amax)
    for (r = 0; r < rows; ++r) {
        int64_t k;
        for (k = 0; k < K; ++k) {
            float a = fabsf(load_elem(x, is_bf16, ld, r, k));
            if (a > amax)
                amax = a;
        }
    }
    return amax / 2688.0f; /* R1 */
}

/* Encode one row with a given tensor scale gs.  codes: K/2 bytes, scales:
 * K/16 bytes. */
static void quantize_row(const void *x, int is_bf16, int64_t ld, int64_t r, int64_t K,
                         float gs, uint8_t *codes, uint8_t *scales)
{
    int64_t b, j;
    for (b = 0; b < K / 16; ++b) {
        float bmax = 0.0f, es;
        unsigned sb;
        for (j = 0; j < 16; ++j) {
            float a = fabsf(load_elem(x, is_bf16, ld, r, 16 * b + j));
            if (a > bmax)
                bmax = a;
        }
        if (gs == 0.0f) {
            sb = 0; /* R2: a zero tensor scale zeroes every block scale */
        } else {
            float t = 6.0f * gs;
            float sbf = bmax / t;
            sb = orc_e4m3_encode(sbf);
        }
        scales[b] = (uint8_t)sb;
        es = (float)orc_e4m3_decode(sb) * gs; /* R3 */
        for (j = 0; j < 16; ++j) {
            float xv = load_elem(x, is_bf16, ld, r, 16 * b + j);
            unsigned mag = 0, code;
            if (es != 0.0f) {
                float q = fabsf(xv) / es;
                mag = orc_e2m1_encode_mag(q);
            }
            code = (signbit(xv) ? 8u : 0u) | mag;
            if ((j & 1) == 0)
                codes[8 * b + j / 2] = (uint8_t)code; /* R4: low nibble first */
            else
                codes[8 * b + j / 2] |= (uint8_t)(code << 4);
        }
    }
}

/* Quantize with a caller-chosen tensor scale (used for calibrated scales
 * and by the tests of the fused repair). */
void orc_quantize_with_scale(const void *x, int is_bf16, int64_t rows, int64_t K, int64_t ld,
                             float gs, uint8_t *codes, uint8_t *scales)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r)
        quantize_row(x, is_bf16, ld, r, K, gs, codes + r * (K / 2), scales + r * (K / 16));
}

/* Full on-the-fly quantization: tensor scale from the whole tensor, then
 * per-block scales and codes.  Returns 0, or -1 if K is not a multiple of
 * 16. */
int orc_quantize(const void *x, int is_bf16, int64_t rows, int64_t K, int64_t ld,
                 uint8_t *codes, uint8_t *scales, float *gs_out)
{
    float gs;
    if (K % 16 != 0)
        return -1;
    gs = orc_tensor_scale(x, is_bf16, rows, K, ld);
    orc_quantize_with_scale(x, is_bf16, rows, K, ld, gs, codes, scales);
    *gs_out = gs;
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Two-level dequant (paper section 5 "fake quantization"; model card      */
/* "Verification" and "Limitations": expansion of NVFP4 to BF16)          */
/* ---------------------------------------------------------------------- */

/* out[r,k] = fp32( E2M1(code) * E4M3(scale) * gs ).  The first product is
 * exact; the whole product is formed exactly in fp64 and rounded once to
 * fp32. */
void orc_dequantize(const uint8_t *codes, const uint8_t *scales, float gs, int64_t rows,
                    int64_t K, float *out)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        int64_t k;
        for (k = 0; k < K; ++k) {
            uint8_t byte = codes[r * (K / 2) + k / 2];
            unsigned code = (k & 1) ? (byte >> 4) : (byte & 15u);
            double v = orc_e2m1_decode(code) * orc_e4m3_decode(scales[r * (K / 16) + k / 16]);
            out[r * K + k] = (float)(v * (double)gs);
        }
    }
}

/* Round an fp32 to bf16 (returned as its 16 bits), nearest, ties to even.
 * Used only to state the bf16 flavour of the dequant output: bf16(fp32(.)). */
static uint16_t f32_to_bf16_bits(float f)
{
    uint32_t u;
    float lo, hi;
    uint32_t ulo, uhi;
    memcpy(&u, &f, sizeof u);
    if (isnan(f))
        return (uint16_t)((u >> 16) | 0x40u);
    /* candidates: truncation toward zero and the next bf16 away from zero */
    ulo = u & 0xFFFF0000u;
    uhi = ulo + 0x10000u;
    memcpy(&lo, &ulo, sizeof lo);
    memcpy(&hi, &uhi, sizeof hi);
    {
        double dl = fabs((double)f - (double)lo), dh = fabs((double)f - (double)hi);
        if (dl < dh)
            return (uint16_t)(ulo >> 16);
        if (dh < dl)
            return (uint16_t)(uhi >> 16);
        return (uint16_t)(((ulo >> 16) & 1u) ? (uhi >> 16) : (ulo >> 16));
    }
}

void orc_dequantize_bf16(const uint8_t *codes, const uint8_t *scales, float gs, int64_t rows,
                         int64_t K, uint16_t *out)
{
    float *tmp = (float *)malloc(sizeof(float) * (size_t)(rows * K));
    int64_t i;
    if (!tmp)
        return;
    orc_dequantize(codes, scales, gs, rows, K, tmp);
    for (i = 0; i < rows * K; ++i)
        out[i] = f32_to_bf16_bits(tmp[i]);
    free(tmp);
}

/* ---------------------------------------------------------------------- */
/* Fused-module repair (paper section 6; reading R6)                      */
/* ---------------------------------------------------------------------- */

/* scales[i] points at member i's [rows[i], kblocks] scale bytes, rewritten
 * in place.  gs[i] is member i's tensor scale.  The shared scale is
 * returned through gs_shared.  Codes are not involved. */
void orc_fuse_rescale(int n, uint8_t **scales, const int64_t *rows, int64_t kblocks,
                      const float *gs, float *gs_shared)
{
    float S = 0.0f;
    int i;
    for (i = 0; i < n; ++i)
        if (gs[i] > S)
            S = gs[i];
    for (i = 0; i < n; ++i) {
        float rho = (S == 0.0f) ? 1.0f : gs[i] / S;
        int64_t j, cnt = rows[i] * kblocks;
        for (j = 0; j < cnt; ++j) {
            unsigned b = scales[i][j];
            if ((b & 0x7Fu) == 0x7Fu)
                continue; /* NaN bytes stay as they are */
            {
                float v = (float)orc_e4m3_decode(b & 0x7Fu) * rho;
                scales[i][j] = (uint8_t)((b & 0x80u) | orc_e4m3_encode(v));
            }
        }
    }
    *gs_shared = S;
}

/* ---------------------------------------------------------------------- */
/* Block-scaled GEMM, exact (paper section 2: both operands NVFP4, FP32    */
/* accumulate on the tensor cores; here the accumulation is exact)        */
/* ---------------------------------------------------------------------- */

/* Integer form of element k of a quantized row: value * 2^10.
 * 2 * E2M1 is an integer in [-12, 12]; 512 * E4M3 is an integer in
 * [0, 229376] for the finite non-negative bytes. */
static int64_t elem_units(const uint8_t *codes_row, const uint8_t *scales_row, int64_t k)
{
    uint8_t byte = codes_row[k / 2];
    unsigned code = (k & 1) ? (byte >> 4) : (byte & 15u);
    double c2 = 2.0 * orc_e2m1_decode(code);
    double s512 = 512.0 * orc_e4m3_decode(scales_row[k / 16]);
    return (int64_t)c2 * (int64_t)s512;
}

/* y[m, n] = sum_k xq[m, k] * wq[n, k] * gs_x * gs_w, exact sum; fp64
 * output.  x*: [M, K] quantized activations, w*: [N, K] quantized weights. */
static double dot_exact(const uint8_t *xc, const uint8_t *xs, const uint8_t *wc,
                        const uint8_t *ws, int64_t K, float gsx, float gsw)
{
    int64_t k, acc = 0;
    for (k = 0; k < K; ++k)
        acc += elem_units(xc, xs, k) * elem_units(wc, ws, k);
    return ldexp((double)acc, -20) * (double)gsx * (double)gsw;
}

void orc_gemm_exact(const uint8_t *xc, const uint8_t *xs, float gsx, const uint8_t *wc,
                    const uint8_t *ws, float gsw, int64_t M, int64_t N, int64_t K, double *y)
{
    int64_t m;
#pragma omp parallel for schedule(dynamic, 1)
    for (m = 0; m < M; ++m) {
        int64_t n;
        for (n = 0; n < N; ++n)
            y[m * N + n] = dot_exact(xc + m * (K / 2), xs + m * (K / 16), wc + n * (K / 2),
                                     ws + n * (K / 16), K, gsx, gsw);
    }
}

/* Only the listed output elements (m_idx[i], n_idx[i]). */
void orc_gemm_exact_sampled(const uint8_t *xc, const uint8_t *xs, float gsx, const uint8_t *wc,
                            const uint8_t *ws, float gsw, int64_t K, int64_t count,
                            const int64_t *m_idx, const int64_t *n_idx, double *y)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < count; ++i) {
        int64_t m = m_idx[i], n = n_idx[i];
        y[i] = dot_exact(xc + m * (K / 2), xs + m * (K / 16), wc + n * (K / 2),
                         ws + n * (K / 16), K, gsx, gsw);
    }
}

/* ---------------------------------------------------------------------- */
/* W4A16: NVFP4 weights against 16-bit activations (model card             */
/* "Gemma-4-31B-IT-NVFP4-FP8attn-text", section "Limitations": without     */
/* native FP4 tensor cores the weights are served as W4A16)                */
/* ---------------------------------------------------------------------- */

/* y[m, n] = gs_w * sum_k x[m, k] * E2M1(code[n, k]) * E4M3(scale[n, k/16]).
 * x is widened exactly to fp32 (bf16 or fp32 input).  Each product
 * x * (E2M1 * E4M3) has at most 24 + 6 significant bits, so it is exact in
 * fp64; the K terms are summed in fp64 in k order, which is within
 * K * 2^-53 * sum|terms| of the exact sum, and the sum is multiplied by
 * gs_w in fp64. */
static double dot_w4a16(const void *x, int is_bf16, int64_t ld, int64_t m, const uint8_t *wc,
                        const uint8_t *ws, int64_t K, float gsw)
{
    int64_t k;
    double acc = 0.0;
    for (k = 0; k < K; ++k) {
        double w = ldexp((double)elem_units(wc, ws, k), -10);
        acc += (double)load_elem(x, is_bf16, ld, m, k) * w;
    }
    return acc * (double)gsw;
}

void orc_gemm_w4a16(const void *x, int is_bf16, int64_t M, int64_t K, int64_t ld, const uint8_t *wc,
                    const uint8_t *ws, float gsw, int64_t N, double *y)
{
    int64_t m;
#pragma omp parallel for schedule(dynamic, 1)
    for (m = 0; m < M; ++m) {
        int64_t n;
        for (n = 0; n < N; ++n)
            y[m * N + n] = dot_w4a16(x, is_bf16, ld, m, wc + n * (K / 2), ws + n * (K / 16), K, gsw);
    }
}

/* Only the listed output elements (m_idx[i], n_idx[i]). */
void orc_gemm_w4a16_sampled(const void *x, int is_bf16, int64_t K, int64_t ld, const uint8_t *wc,
                            const uint8_t *ws, float gsw, int64_t count, const int64_t *m_idx,
                            const int64_t *n_idx, double *y)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < count; ++i)
        y[i] = dot_w4a16(x, is_bf16, ld, m_idx[i], wc + n_idx[i] * (K / 2), ws + n_idx[i] * (K / 16),
                         K, gsw);
}

/* ---------------------------------------------------------------------- */
/* FP8 E4M3 with one per-tensor scale (model card                          */
/* "Gemma-4-31B-IT-NVFP4-FP8attn-text", section "What was quantized,        */
/* exactly": per-tensor scale, float8_e4m3, weights only, served W8A16;    */
/* paper section 7 "KV-cache precision": FP8 KV cache with static           */
/* per-tensor scales).                                                      */
/*                                                                          */
/* Readings where the pages are silent:                                     */
/*   F1 dynamic scale s = RN(amax / 448), the dequant form (largest byte    */
/*      0x7E), as R1 for NVFP4; a static scale is given by the caller.      */
/*   F2 byte = signbit(x) << 7 | E4M3_RNE_sat(RN(|x| / s)) (a divide, as    */
/*      R3); s == 0 gives magnitude 0.                                      */
/*   F3 dequant x = RN(E4M3(byte) * s).                                     */
/* ---------------------------------------------------------------------- */

float orc_fp8_tensor_scale(const void *x, int is_bf16, int64_t rows, int64_t K, int64_t ld)
{
    float amax = 0.0f;
    int64_t r;
#pragma omp parallel for schedule(static) reduction(max : amax)
    for (r = 0; r < rows; ++r) {
        int64_t k;
        for (k = 0; k < K; ++k) {
            float a = fabsf(load_elem(x, is_bf16, ld, r, k));
            if (a > amax)
                amax = a;
        }
    }
    return amax / 448.0f; /* F1 */
}

void orc_fp8_quantize_with_scale(const void *x, int is_bf16, int64_t rows, int64_t K, int64_t ld, float s,
                                 uint8_t *q)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        int64_t k;
        for (k = 0; k < K; ++k) {
            float xv = load_elem(x, is_bf16, ld, r, k);
            unsigned mag = 0;
            if (s != 0.0f)
                mag = orc_e4m3_encode(fabsf(xv) / s); /* F2 */
            q[r * K + k] = (uint8_t)((signbit(xv) ? 0x80u : 0u) | mag);
        }
    }
}

void orc_fp8_dequantize(const uint8_t *q, float s, int64_t rows, int64_t K, float *out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < rows * K; ++i)
        out[i] = (float)(orc_e4m3_decode(q[i]) * (double)s); /* F3: one rounding of the exact product */
}

/* W8A16: y[m, n] = s_w * sum_k x[m, k] * E4M3(wq[n, k]); products exact in
 * fp64 (24 + 4 significant bits), summed in fp64 in k order. */
static double dot_w8a16(const void *x, int is_bf16, int64_t ld, int64_t m, const uint8_t *wq, int64_t K,
                        float sw)
{
    int64_t k;
    double acc = 0.0;
    for (k = 0; k < K; ++k)
        acc += (double)load_elem(x, is_bf16, ld, m, k) * orc_e4m3_decode(wq[k]);
    return acc * (double)sw;
}

void orc_gemm_w8a16(const void *x, int is_bf16, int64_t M, int64_t K, int64_t ld, const uint8_t *wq, float sw,
                    int64_t N, double *y)
{
    int64_t m;
#pragma omp parallel for schedule(dynamic, 1)
    for (m = 0; m < M; ++m) {
        int64_t n;
        for (n = 0; n < N; ++n)
            y[m * N + n] = dot_w8a16(x, is_bf16, ld, m, wq + n * K, K, sw);
    }
}

/* W8A8, exact: every E4M3 value is an integer times 2^-9 below 2^18 in
 * magnitude, so a K-long sum of products is exact in int64 for K < 2^27;
 * y = sum * 2^-18 * s_x * s_w in fp64. */
void orc_gemm_w8a8(const uint8_t *xq, float sx, const uint8_t *wq, float sw, int64_t M, int64_t N, int64_t K,
                   double *y)
{
    int64_t m;
#pragma omp parallel for schedule(dynamic, 1)
    for (m = 0; m < M; ++m) {
        int64_t n, k;
        for (n = 0; n < N; ++n) {
            int64_t acc = 0;
            for (k = 0; k < K; ++k)
                acc += (int64_t)(512.0 * orc_e4m3_decode(xq[m * K + k])) *
                       (int64_t)(512.0 * orc_e4m3_decode(wq[n * K + k]));
            y[m * N + n] = ldexp((double)acc, -18) * (double)sx * (double)sw;
        }
    }
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
