/* Address/undefined-behaviour sanitizer driver for the C ABI's validation
 * path.  The library's ABI layer is linked against launchers that abort
 * (tests/sanitize/launch_stubs.hip), and every call below must be decided on
 * the host: rejected with the documented status, or accepted as empty with
 * nothing launched.  Fake device addresses are never dereferenced.  The
 * workspace-size functions are called with every extreme shape, where an
 * unchecked product would overflow.  Exit status 0 when everything passed. */
#include <stdint.h>
#include <stdio.h>

#include "../../include/nvfp4.h"

#define A ((void *)(uintptr_t)0x10000) /* 256-byte aligned, never dereferenced */
#define AU8 ((uint8_t *)(uintptr_t)0x10000)
#define AF ((float *)(uintptr_t)0x10000)
#define BIG ((size_t)1 << 40)

static int failures = 0;
#define EXPECT(call, want)                                                              \
    do {                                                                                \
        nvfp4_status_t got_ = (call);                                                   \
        if (got_ != (want)) {                                                           \
            fprintf(stderr, "%s:%d: %s -> %d, expected %d\n", __FILE__, __LINE__, #call, \
                    (int)got_, (int)(want));                                            \
            ++failures;                                                                 \
        }                                                                               \
    } while (0)

int main(void)
{
    static const int64_t extremes[] = {-1, 0, 1, 16, 64, ((int64_t)1 << 31) - 1, (int64_t)1 << 31,
                                       ((int64_t)1 << 40), INT64_MAX};
    const size_t ne = sizeof extremes / sizeof extremes[0];
    size_t i, j, k, total = 0;
    /* sizes: defined (no overflow) for every argument */
    for (i = 0; i < ne; ++i)
        for (j = 0; j < ne; ++j) {
            total += nvfp4_quantize_workspace_size(extremes[i], extremes[j]);
            total += nvfp4_fp8_quantize_workspace_size(extremes[i], extremes[j]);
            for (k = 0; k < ne; ++k) {
                total += nvfp4_gemm_workspace_size(extremes[i], extremes[j], extremes[k]);
                total += nvfp4_gemm_w4a16_workspace_size(extremes[i], extremes[j], extremes[k]);
                total += nvfp4_gemm_w8a16_workspace_size(extremes[i], extremes[j], extremes[k]);
                total += nvfp4_gemm_w8a8_workspace_size(extremes[i], extremes[j], extremes[k]);
            }
        }

    /* quantize */
    EXPECT(nvfp4_quantize(A, (nvfp4_dtype_t)5, 4, 32, 32, AU8, AU8, AF, A, BIG, NULL), NVFP4_ERR_DTYPE);
    EXPECT(nvfp4_quantize(A, NVFP4_BF16, 4, 24, 24, AU8, AU8, AF, A, BIG, NULL), NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_quantize(A, NVFP4_BF16, INT64_MAX, 32, 32, AU8, AU8, AF, A, BIG, NULL), NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_quantize(A, NVFP4_BF16, 4, INT64_MAX - 15, INT64_MAX, AU8, AU8, AF, A, BIG, NULL), NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_quantize(A, NVFP4_BF16, (int64_t)1 << 30, 1 << 16, 1 << 16, AU8, AU8, AF, A, BIG, NULL),
           NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_quantize(NULL, NVFP4_BF16, 4, 32, 32, AU8, AU8, AF, A, BIG, NULL), NVFP4_ERR_NULL);
    EXPECT(nvfp4_quantize(A, NVFP4_BF16, 4, 32, 32, NULL, AU8, AF, A, BIG, NULL), NVFP4_ERR_NULL);
    EXPECT(nvfp4_quantize(A, NVFP4_BF16, 4, 32, 32, AU8, AU8, AF, NULL, BIG, NULL), NVFP4_ERR_WORKSPACE);
    EXPECT(nvfp4_quantize((char *)A + 8, NVFP4_BF16, 4, 32, 32, AU8, AU8, AF, A, BIG, NULL), NVFP4_ERR_ALIGN);
    EXPECT(nvfp4_quantize_static(A, NVFP4_F32, 0, 32, 32, AF, AU8, AU8, NULL), NVFP4_OK);
    EXPECT(nvfp4_quantize_static(A, NVFP4_F32, 4, 32, 32, NULL, AU8, AU8, NULL), NVFP4_ERR_NULL);
    EXPECT(nvfp4_dequantize(AU8, AU8, AF, 0, 32, A, NVFP4_F32, 32, NULL), NVFP4_OK);
    EXPECT(nvfp4_dequantize(AU8, AU8, AF, INT64_MAX, 32, A, NVFP4_F32, 32, NULL), NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_dequantize(AU8, AU8, AF, 4, 32, A, NVFP4_F32, 16, NULL), NVFP4_ERR_SHAPE);

    /* repair */
    {
        uint8_t *sc[2] = {AU8, AU8 + 4096};
        int64_t rows[2] = {1, INT64_MAX};
        const float *gs[2] = {AF + 64, AF + 128};
        EXPECT(nvfp4_fuse_rescale(2, sc, rows, 4, gs, AF, NULL), NVFP4_ERR_SHAPE);
        rows[1] = (int64_t)1 << 30;
        EXPECT(nvfp4_fuse_rescale(2, sc, rows, (int64_t)1 << 30, gs, AF, NULL), NVFP4_ERR_SHAPE);
        EXPECT(nvfp4_fuse_rescale(0, sc, rows, 4, gs, AF, NULL), NVFP4_ERR_INVALID);
        EXPECT(nvfp4_fuse_rescale(17, sc, rows, 4, gs, AF, NULL), NVFP4_ERR_INVALID);
    }

    /* linears: every shape check, then the empty problems that launch nothing */
    EXPECT(nvfp4_gemm(A, NVFP4_BF16, 32, 48, 48, AU8, AU8, AF, 64, A, NVFP4_BF16, 64, A, BIG, NULL),
           NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_gemm(A, NVFP4_BF16, 32, 1 << 23, 1 << 23, AU8, AU8, AF, 64, A, NVFP4_BF16, 64, A, BIG, NULL),
           NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_gemm(A, NVFP4_BF16, 32, 64, 64, AU8, AU8, AF, INT64_MAX, A, NVFP4_BF16, INT64_MAX, A, BIG, NULL),
           NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_gemm(A, NVFP4_BF16, 32, 64, 64, AU8, AU8, AF, 64, A, NVFP4_BF16, 64, A, 10, NULL),
           NVFP4_ERR_WORKSPACE);
    EXPECT(nvfp4_gemm(A, NVFP4_BF16, 0, 64, 64, AU8, AU8, AF, 64, A, NVFP4_BF16, 64, A, BIG, NULL), NVFP4_OK);
    EXPECT(nvfp4_gemm(A, NVFP4_BF16, 32, 64, 64, AU8, AU8, AF, 0, A, NVFP4_BF16, 64, A, BIG, NULL), NVFP4_OK);
    EXPECT(nvfp4_gemm_static(A, NVFP4_BF16, 32, 64, 64, NULL, AU8, AU8, AF, 64, A, NVFP4_BF16, 64, A, BIG, NULL),
           NVFP4_ERR_NULL);
    EXPECT(nvfp4_gemm_run(32, 64, AU8, AU8, AF, 64, A, NVFP4_BF16, 64, A, 10, NULL), NVFP4_ERR_WORKSPACE);
    EXPECT(nvfp4_gemm_run(32, 64, AU8, AU8, AF, 0, A, NVFP4_BF16, 64, A, 10, NULL), NVFP4_OK);
    EXPECT(nvfp4_gemm_prepare(A, NVFP4_BF16, 0, 64, 64, A, BIG, NULL), NVFP4_OK);
    EXPECT(nvfp4_gemm_noalloc(A, NVFP4_BF16, 1 << 16, 5120, 5120, AU8, AU8, AF, 17408, A, NVFP4_BF16, 17408, NULL),
           NVFP4_ERR_WORKSPACE);
    EXPECT(nvfp4_gemm_noalloc(A, NVFP4_BF16, 32, 64, 64, AU8, AU8, AF, 0, A, NVFP4_BF16, 64, NULL), NVFP4_OK);
    EXPECT(nvfp4_gemm_w4a16(A, NVFP4_F32, 32, 64, 64, AU8, AU8, AF, 64, A, NVFP4_BF16, 64, A, BIG, NULL),
           NVFP4_ERR_DTYPE);
    EXPECT(nvfp4_gemm_w4a16(A, NVFP4_BF16, 32, 64, 1 << 23, AU8, AU8, AF, 64, A, NVFP4_BF16, 64, A, BIG, NULL),
           NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_gemm_w8a16(A, NVFP4_BF16, 32, 64, 64, AU8, AF, (int64_t)1 << 30, A, NVFP4_BF16, (int64_t)1 << 30,
                            A, BIG, NULL),
           NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_gemm_w8a8(A, NVFP4_BF16, 32, 1 << 24, 1 << 24, NULL, AU8, AF, 64, A, NVFP4_BF16, 64, A, BIG, NULL),
           NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_fp8_quantize(A, NVFP4_BF16, 4, 32, 32, (uint8_t *)A + 4, AF, A, BIG, NULL), NVFP4_ERR_ALIGN);
    EXPECT(nvfp4_fp8_quantize_static(A, NVFP4_BF16, 0, 32, 32, AF, NULL, NULL), NVFP4_OK);
    EXPECT(nvfp4_fp8_dequantize(AU8, AF, 4, 40, A, NVFP4_F32, 40, NULL), NVFP4_ERR_SHAPE);

    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("ABI sanitizer driver: all checks passed (sizes summed to %zu)\n", total);
    return 0;
}
