/* Drives every entry point of the CPU oracle on small inputs, for an
 * AddressSanitizer + UndefinedBehaviorSanitizer build (test infrastructure).
 * Inputs sweep every 16-bit pattern (zeros, subnormals, Inf, NaN included)
 * through all type pairs, both scale layouts and both EMAX modes; a few
 * outputs are checked against values the numerics page fixes. Exit status
 * 0 = every check held. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int mxq_oracle_quantize(const uint16_t *in, int64_t P, int64_t F, int in_dtype, int out_dtype, int alt_emax,
                        int scale_layout, uint8_t *data_out, uint8_t *scale_image);
int mxq_oracle_quantize_axis(const uint16_t *in, int64_t R, int64_t C, int in_dtype, int out_dtype, int dim,
                             int alt_emax, int scale_layout, uint8_t *data_out, uint8_t *scale_image);
int mxq_oracle_dequantize(const uint8_t *data, const uint8_t *scale_image, int64_t P, int64_t F, int out_dtype,
                          int res_dtype, int scale_layout, void *out);
int mxq_oracle_scaled_matmul(const uint8_t *lhs, const uint8_t *lhs_scale, const uint8_t *rhs,
                             const uint8_t *rhs_scale, int64_t P, int64_t M, int64_t N, int fmt, int scale_layout,
                             double *out);
int mxq_oracle_scaled_matmul_quantize(const uint8_t *lhs, const uint8_t *lhs_scale, const uint8_t *rhs,
                                      const uint8_t *rhs_scale, int64_t P, int64_t M, int64_t N, int fmt,
                                      int out_dtype, int alt_emax, int scale_layout, uint8_t *data_out,
                                      uint8_t *scale_out);
uint8_t mxq_oracle_e8m0(uint8_t max_exponent, int emax_bias);
int64_t mxq_oracle_lane_remap(int64_t index, int64_t stride);

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
    /* every 16-bit pattern once: P = 64 rows x F = 1024 columns */
    const int64_t P = 64, F = 1024;
    uint16_t *x = malloc((size_t)(P * F) * sizeof(uint16_t));
    uint8_t *data = malloc((size_t)(P * F));
    uint8_t *image = malloc((size_t)(P * F / 4));
    float *res = malloc((size_t)(P * F) * sizeof(float));
    for (int64_t k = 0; k < P * F; k++)
        x[k] = (uint16_t)(k * 40503u);   /* an odd multiplier permutes 0..65535 */
    for (int in = 0; in < 2; in++)
        for (int out = 0; out < 3; out++)
            for (int alt = 0; alt < 2; alt++)
                for (int layout = 0; layout < 2; layout++) {
                    memset(image, 0xA5, (size_t)(P * F / 4));
                    CHECK(mxq_oracle_quantize(x, P, F, in, out, alt, layout, data, image) == 0);
                    CHECK(mxq_oracle_dequantize(data, image, P, F, out, alt, layout, res) == 0);
                    CHECK(mxq_oracle_quantize_axis(x, 32 * 4, F * P / 128, in, out, -2, alt, layout, data,
                                                   image) == 0);
                    CHECK(mxq_oracle_quantize_axis(x, P, F, in, out, -1, alt, layout, data, image) == 0);
                }

    /* the page's fixed points: an all-zero block gets E8M0 1; E8M0 127 maps
     * 1.0 to the e4m3fn code 0x38 */
    uint16_t z[32] = {0};
    uint8_t zd[32], zs[8];
    CHECK(mxq_oracle_quantize(z, 8, 4, 0, 0, 0, 0, zd, zs) == 0 && zs[0] == 1);
    CHECK(mxq_oracle_e8m0(0, 8) == 1 && mxq_oracle_e8m0(135, 8) == 127);
    uint16_t ones[32];
    for (int k = 0; k < 32; k++)
        ones[k] = 0x3F80; /* bf16 1.0 */
    ones[0] = 0x4380;     /* 256: block max exponent 135 -> E8M0 127 */
    CHECK(mxq_oracle_quantize(ones, 8, 4, 0, 0, 0, 0, zd, zs) == 0 && zs[0] == 127 && zd[1] == 0x38);
    CHECK(mxq_oracle_lane_remap(0, 2) == 2 && mxq_oracle_lane_remap(3, 2) == 1 && mxq_oracle_lane_remap(5, 1) == 5);

    /* the matmul and its fused quantize on every code under E8M0 bytes 0..255 */
    const int64_t KP = 16, M = 64, N = 32;
    uint8_t *lhs = malloc((size_t)(KP * 4 * M)), *rhs = malloc((size_t)(KP * 4 * N));
    uint8_t *ls = calloc((size_t)(KP * M), 1), *rs = calloc((size_t)(KP * N), 1);
    double *mm = malloc((size_t)(M * N) * sizeof(double));
    uint8_t *qd = malloc((size_t)(M * N)), *qs = malloc((size_t)(M * N / 4));
    for (int64_t k = 0; k < KP * 4 * M; k++)
        lhs[k] = (uint8_t)(k * 7);
    for (int64_t k = 0; k < KP * 4 * N; k++)
        rhs[k] = (uint8_t)(k * 13 + 5);
    for (int64_t k = 0; k < KP * M; k++)
        ls[k] = (uint8_t)(k * 11);
    for (int64_t k = 0; k < KP * N; k++)
        rs[k] = (uint8_t)(k * 3 + 1);
    for (int fmt = 0; fmt < 2; fmt++)
        for (int layout = 0; layout < 2; layout++) {
            CHECK(mxq_oracle_scaled_matmul(lhs, ls, rhs, rs, KP, M, N, fmt, layout, mm) == 0);
            for (int out = 0; out < 3; out++)
                CHECK(mxq_oracle_scaled_matmul_quantize(lhs, ls, rhs, rs, KP, M, N, fmt, out, 0, layout, qd, qs) ==
                      0);
        }

    /* rejected calls write nothing and return their status */
    CHECK(mxq_oracle_quantize(x, 12, F, 0, 0, 0, 0, data, image) == 3);
    CHECK(mxq_oracle_quantize(x, P, 6, 0, 0, 0, 0, data, image) == 4);
    CHECK(mxq_oracle_quantize(x, P, F, 2, 0, 0, 0, data, image) == 1);
    CHECK(mxq_oracle_quantize(x, P, F, 0, 3, 0, 0, data, image) == 2);
    CHECK(mxq_oracle_quantize(x, 0, F, 0, 0, 0, 0, NULL, NULL) == 0);
    CHECK(mxq_oracle_quantize_axis(x, 20, 32, 0, 0, -2, 0, 0, data, image) == 3);
    CHECK(mxq_oracle_quantize_axis(x, 32, 32, 0, 0, 5, 0, 0, data, image) == 6);

    free(x), free(data), free(image), free(res), free(lhs), free(rhs), free(ls), free(rs), free(mm), free(qd),
        free(qs);
    if (failures)
        return 1;
    puts("oracle under sanitizers: ok");
    return 0;
}
