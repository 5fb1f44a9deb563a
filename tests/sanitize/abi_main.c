/* Drives the C ABI's host-side logic -- validation, size helpers, status
 * strings -- for an AddressSanitizer + UndefinedBehaviorSanitizer build of
 * the library's host code (test infrastructure). Every call here is
 * rejected before any launch or is an empty call, so no GPU is needed and
 * no kernel runs. Exit status 0 = every check held. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mxq.h"

static int failures;
#define CHECK(c)                                                                   \
    do {                                                                           \
        if (!(c)) {                                                                \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__);        \
            failures++;                                                            \
        }                                                                          \
    } while (0)

int main(void)
{
    void *g = (void *)(uintptr_t)4096; /* aligned, never dereferenced */
    void *odd = (void *)(uintptr_t)4104;
    const int64_t big = (int64_t)1 << 62;

    for (int s = -3; s < 16; s++)
        CHECK(mxq_status_string(s) != NULL && strlen(mxq_status_string(s)) > 0);
    CHECK(mxq_abi_version() == MXQ_ABI_VERSION);

    /* size helpers, including overflowing and negative shapes */
    CHECK(mxq_data_bytes(16, 8, MXQ_OUT_E2M1) == 64 && mxq_data_bytes(16, 8, 7) == 0);
    CHECK(mxq_data_bytes(big, big, MXQ_OUT_E4M3FN) == 0 && mxq_data_bytes(-8, 4, 0) == 0);
    CHECK(mxq_scale_image_bytes(16, 8) == 32 && mxq_scale_image_bytes(big, 8) == 0);
    CHECK(mxq_scale_bytes(16, 8, MXQ_FLAG_DENSE_SCALE) == 4 && mxq_scale_bytes(16, 8, 8u) == 0);
    CHECK(mxq_result_bytes(16, 8, MXQ_RES_F32) == 512 && mxq_result_bytes(big, big, MXQ_RES_BF16) == 0);

    /* quantize: every rejection */
    CHECK(mxq_quantize(g, 16, 8, 2, 0, g, g, NULL) == MXQ_E_IN_DTYPE);
    CHECK(mxq_quantize(g, 16, 8, 0, 3, g, g, NULL) == MXQ_E_OUT_DTYPE);
    CHECK(mxq_quantize(g, 12, 8, 0, 0, g, g, NULL) == MXQ_E_SHAPE_P8);
    CHECK(mxq_quantize(g, 16, 6, 0, 0, g, g, NULL) == MXQ_E_SHAPE_F4);
    CHECK(mxq_quantize(g, big, big, 0, 0, g, g, NULL) == MXQ_E_OVERFLOW);
    CHECK(mxq_quantize(g, (int64_t)1 << 31, 4, 0, 0, g, g, NULL) == MXQ_E_OVERFLOW);
    CHECK(mxq_quantize(NULL, 16, 8, 0, 0, g, g, NULL) == MXQ_E_NULL);
    CHECK(mxq_quantize(odd, 16, 8, 0, 0, g, g, NULL) == MXQ_E_ALIGN);
    CHECK(mxq_quantize(NULL, 0, 8, 0, 0, NULL, NULL, NULL) == MXQ_OK);
    CHECK(mxq_quantize_ex(g, 16, 8, 0, 0, 4u, g, g, NULL) == MXQ_E_FLAGS);

    /* dequantize */
    CHECK(mxq_dequantize(g, g, 16, 8, 0, 2, g, NULL) == MXQ_E_RES_DTYPE);
    CHECK(mxq_dequantize(g, g, 16, 8, 3, 0, g, NULL) == MXQ_E_OUT_DTYPE);
    CHECK(mxq_dequantize(g, g, big, big, 0, 0, g, NULL) == MXQ_E_OVERFLOW);
    CHECK(mxq_dequantize(g, g, (int64_t)1 << 31, 4, 0, 1, g, NULL) == MXQ_E_OVERFLOW);
    CHECK(mxq_dequantize(g, NULL, 16, 8, 0, 0, g, NULL) == MXQ_E_NULL);
    CHECK(mxq_dequantize_ex(g, g, 16, 8, 0, 0, 1u, g, NULL) == MXQ_E_FLAGS);

    /* quantize along an axis */
    CHECK(mxq_quantize_axis(g, 32, 32, 0, 0, 3, 0, g, g, NULL) == MXQ_E_DIM);
    CHECK(mxq_quantize_axis(g, 20, 32, 0, 0, -2, 0, g, g, NULL) == MXQ_E_SHAPE_P8);
    CHECK(mxq_quantize_axis(g, (int64_t)1 << 32, 4, 0, 0, -2, 0, g, g, NULL) == MXQ_E_OVERFLOW);
    CHECK(mxq_quantize_axis(g, 256, (int64_t)1 << 33, 0, 0, -1, 0, g, g, NULL) == MXQ_E_OVERFLOW);
    CHECK(mxq_quantize_axis(g, big, big, 0, 0, -1, 0, g, g, NULL) != MXQ_OK);
    CHECK(mxq_quantize_axis(g, 32, 32, 0, 0, -1, 0, odd, g, NULL) == MXQ_E_ALIGN);

    /* the scaled matmul and its quantized form */
    CHECK(mxq_scaled_matmul(g, g, g, g, 12, 4, 4, 0, 0, 0, g, NULL) == MXQ_E_SHAPE_P8);
    CHECK(mxq_scaled_matmul(g, g, g, g, 8, 6, 4, 0, 0, 0, g, NULL) == MXQ_E_SHAPE_F4);
    CHECK(mxq_scaled_matmul(g, g, g, g, 8, 4, 4, 2, 0, 0, g, NULL) != MXQ_OK);
    CHECK(mxq_scaled_matmul(g, g, g, g, 8, MXQ_MATMUL_MAX_COLS, MXQ_MATMUL_MAX_COLS, 0, 0, 0, g, NULL) ==
          MXQ_E_OVERFLOW);
    CHECK(mxq_scaled_matmul(g, g, g, g, 8, big, 4, 0, 0, 0, g, NULL) == MXQ_E_OVERFLOW);
    CHECK(mxq_scaled_matmul(NULL, g, g, g, 8, 4, 4, 0, 0, 0, g, NULL) == MXQ_E_NULL);
    CHECK(mxq_scaled_matmul_quantize(g, g, g, g, 8, 4, 4, 0, 0, 0, g, g, NULL) == MXQ_E_SHAPE_P8);
    CHECK(mxq_scaled_matmul_quantize(g, g, g, g, 8, 8, 4, 0, 5, 0, g, g, NULL) == MXQ_E_OUT_DTYPE);

    if (failures)
        return 1;
    puts("library host code under sanitizers: ok");
    return 0;
}
