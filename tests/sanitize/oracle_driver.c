/* Address/undefined-behaviour sanitizer driver for the oracle (test
 * infrastructure only).  Runs every oracle entry point on small seeded
 * inputs of ragged shapes -- one row, K = 16, odd row counts, zero tensors,
 * bf16 and fp32 -- so that the sanitizers see every indexing path, and checks
 * a few properties that hold exactly.  Exit status 0 when everything passed;
 * a sanitizer finding aborts the process. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_e2m1_decode(unsigned code);
double orc_e4m3_decode(unsigned byte);
unsigned orc_e4m3_encode(float v);
unsigned orc_e2m1_encode_mag(float r);
float orc_tensor_scale(const void *x, int is_bf16, int64_t rows, int64_t K, int64_t ld);
void orc_quantize_with_scale(const void *x, int is_bf16, int64_t rows, int64_t K, int64_t ld, float gs,
                             uint8_t *codes, uint8_t *scales);
int orc_quantize(const void *x, int is_bf16, int64_t rows, int64_t K, int64_t ld, uint8_t *codes,
                 uint8_t *scales, float *gs_out);
void orc_dequantize(const uint8_t *codes, const uint8_t *scales, float gs, int64_t rows, int64_t K, float *out);
void orc_dequantize_bf16(const uint8_t *codes, const uint8_t *scales, float gs, int64_t rows, int64_t K,
                         uint16_t *out);
void orc_fuse_rescale(int n, uint8_t **scales, const int64_t *rows, int64_t kblocks, const float *gs,
                      float *gs_shared);
void orc_gemm_exact(const uint8_t *xc, const uint8_t *xs, float gsx, const uint8_t *wc, const uint8_t *ws,
                    float gsw, int64_t M, int64_t N, int64_t K, double *y);
void orc_gemm_exact_sampled(const uint8_t *xc, const uint8_t *xs, float gsx, const uint8_t *wc,
                            const uint8_t *ws, float gsw, int64_t K, int64_t count, const int64_t *m_idx,
                            const int64_t *n_idx, double *y);
void orc_gemm_w4a16(const void *x, int is_bf16, int64_t M, int64_t K, int64_t ld, const uint8_t *wc,
                    const uint8_t *ws, float gsw, int64_t N, double *y);
void orc_gemm_w4a16_sampled(const void *x, int is_bf16, int64_t K, int64_t ld, const uint8_t *wc,
                            const uint8_t *ws, float gsw, int64_t count, const int64_t *m_idx,
                            const int64_t *n_idx, double *y);
float orc_fp8_tensor_scale(const void *x, int is_bf16, int64_t rows, int64_t K, int64_t ld);
void orc_fp8_quantize_with_scale(const void *x, int is_bf16, int64_t rows, int64_t K, int64_t ld, float s,
                                 uint8_t *q);
void orc_fp8_dequantize(const uint8_t *q, float s, int64_t rows, int64_t K, float *out);
void orc_gemm_w8a16(const void *x, int is_bf16, int64_t M, int64_t K, int64_t ld, const uint8_t *wq, float sw,
                    int64_t N, double *y);
void orc_gemm_w8a8(const uint8_t *xq, float sx, const uint8_t *wq, float sw, int64_t M, int64_t N, int64_t K,
                   double *y);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform(void) /* xorshift64*, [0, 1) */
{
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) * 0x1p-53;
}

static int failures = 0;
#define CHECK(c, ...)                  \
    do {                               \
        if (!(c)) {                    \
            fprintf(stderr, __VA_ARGS__); \
            fprintf(stderr, "\n");     \
            ++failures;                \
        }                              \
    } while (0)

/* Buffers are allocated at their exact sizes, so any out-of-bounds access
 * by the oracle lands in an ASan redzone. */
static void run_shape(int64_t M, int64_t N, int64_t K, int bf16, int zero)
{
    const int64_t ld = K + (bf16 ? 8 : 4); /* padded rows: ld > K is a path of its own */
    size_t es = bf16 ? 2 : 4;
    void *x = malloc((size_t)(M * ld) * es), *w = malloc((size_t)(N * K) * es);
    int64_t i;
    for (i = 0; i < M * ld; ++i) {
        float v = zero ? 0.0f : (float)((uniform() - 0.5) * 8.0);
        if (bf16) {
            uint32_t b;
            memcpy(&b, &v, 4);
            ((uint16_t *)x)[i] = (uint16_t)(b >> 16);
        } else {
            ((float *)x)[i] = v;
        }
    }
    for (i = 0; i < N * K; ++i) {
        float v = zero ? 0.0f : (float)((uniform() - 0.5) * 0.1);
        if (bf16) {
            uint32_t b;
            memcpy(&b, &v, 4);
            ((uint16_t *)w)[i] = (uint16_t)(b >> 16);
        } else {
            ((float *)w)[i] = v;
        }
    }
    uint8_t *xc = malloc((size_t)(M * K / 2)), *xs = malloc((size_t)(M * K / 16));
    uint8_t *wc = malloc((size_t)(N * K / 2)), *wsc = malloc((size_t)(N * K / 16));
    float gx, gw;
    CHECK(orc_quantize(x, bf16, M, K, ld, xc, xs, &gx) == 0, "quantize X failed");
    CHECK(orc_quantize(w, bf16, N, K, K, wc, wsc, &gw) == 0, "quantize W failed");
    CHECK(orc_tensor_scale(x, bf16, M, K, ld) == gx, "tensor scale differs");
    /* the model card's identity: the largest scale byte is 448 unless zero */
    if (!zero) {
        unsigned mx = 0;
        for (i = 0; i < M * K / 16; ++i)
            if (xs[i] > mx)
                mx = xs[i];
        CHECK(mx == 0x7E, "largest scale byte 0x%02x", mx);
    }
    float *dq = malloc((size_t)(M * K) * 4);
    uint16_t *dqb = malloc((size_t)(M * K) * 2);
    orc_dequantize(xc, xs, gx, M, K, dq);
    orc_dequantize_bf16(xc, xs, gx, M, K, dqb);
    double *y = malloc((size_t)(M * N) * 8);
    orc_gemm_exact(xc, xs, gx, wc, wsc, gw, M, N, K, y);
    int64_t mi[3] = {0, M - 1, M / 2}, ni[3] = {N - 1, 0, N / 2};
    double ys[3];
    orc_gemm_exact_sampled(xc, xs, gx, wc, wsc, gw, K, 3, mi, ni, ys);
    for (i = 0; i < 3; ++i)
        CHECK(ys[i] == y[mi[i] * N + ni[i]], "sampled GEMM differs at %d", (int)i);
    if (bf16) {
        double *y16 = malloc((size_t)(M * N) * 8);
        orc_gemm_w4a16(x, 1, M, K, ld, wc, wsc, gw, N, y16);
        orc_gemm_w4a16_sampled(x, 1, K, ld, wc, wsc, gw, 3, mi, ni, ys);
        for (i = 0; i < 3; ++i)
            CHECK(ys[i] == y16[mi[i] * N + ni[i]], "sampled W4A16 differs at %d", (int)i);
        free(y16);
    }
    /* FP8 per-tensor forms */
    uint8_t *xq = malloc((size_t)(M * K)), *wq = malloc((size_t)(N * K));
    float sx = orc_fp8_tensor_scale(x, bf16, M, K, ld), sw = orc_fp8_tensor_scale(w, bf16, N, K, K);
    orc_fp8_quantize_with_scale(x, bf16, M, K, ld, sx, xq);
    orc_fp8_quantize_with_scale(w, bf16, N, K, K, sw, wq);
    float *fq = malloc((size_t)(M * K) * 4);
    orc_fp8_dequantize(xq, sx, M, K, fq);
    orc_gemm_w8a8(xq, sx, wq, sw, M, N, K, y);
    if (bf16)
        orc_gemm_w8a16(x, 1, M, K, ld, wq, sw, N, y);
    /* fused repair of two members (the W rows split in two) */
    if (N >= 2) {
        int64_t rows[2] = {N / 2, N - N / 2};
        float gss[2] = {gw, gw * 0.5f}, S;
        uint8_t *m0 = malloc((size_t)(rows[0] * K / 16)), *m1 = malloc((size_t)(rows[1] * K / 16));
        memcpy(m0, wsc, (size_t)(rows[0] * K / 16));
        memcpy(m1, wsc + rows[0] * K / 16, (size_t)(rows[1] * K / 16));
        uint8_t *ms[2] = {m0, m1};
        orc_fuse_rescale(2, ms, rows, K / 16, gss, &S);
        CHECK(S == gw, "shared scale");
        CHECK(memcmp(m0, wsc, (size_t)(rows[0] * K / 16)) == 0, "maximal member changed");
        free(m0);
        free(m1);
    }
    free(xq);
    free(wq);
    free(fq);
    free(y);
    free(dq);
    free(dqb);
    free(xc);
    free(xs);
    free(wc);
    free(wsc);
    free(x);
    free(w);
}

int main(void)
{
    static const int64_t shapes[][3] = {{1, 1, 16}, {1, 7, 64}, {3, 5, 48}, {16, 33, 256}, {17, 2, 32}, {5, 9, 512}};
    size_t s;
    int bf16, zero;
    unsigned b, c;
    for (b = 0; b < 256; ++b) {
        double v = orc_e4m3_decode(b);
        if (b < 0x80u && !isnan(v))
            CHECK(orc_e4m3_encode((float)v) == b, "E4M3 round trip of byte 0x%02x", b);
    }
    for (c = 0; c < 8; ++c)
        CHECK(orc_e2m1_encode_mag((float)orc_e2m1_decode(c)) == c, "E2M1 round trip of code %u", c);
    for (s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
        for (bf16 = 0; bf16 < 2; ++bf16)
            for (zero = 0; zero < 2; ++zero)
                run_shape(shapes[s][0], shapes[s][1], shapes[s][2], bf16, zero);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer driver: all checks passed\n");
    return 0;
}
