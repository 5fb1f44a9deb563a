// mxq_api.hip -- the C ABI of the MX quantize library (declared in mxq.h).
//
// Host side only: argument validation, launch geometry, dispatch on
// (input type, output type, strip width) to the kernel templates, and the
// launch itself on the caller's stream. No allocation, no state.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq.h"
#include "mxq_dequantize_kernels.hpp"
#include "mxq_matmul_kernels.hpp"
#include "mxq_quantize_kernels.hpp"

namespace {

// Threads per workgroup: one wave. On MI355X single-wave workgroups stream
// this kernel's 2:1 read/write mix faster than 128- or 256-thread ones (the
// dispatcher spreads the finer tiles more evenly over the CUs).
constexpr uint32_t kThreads = 64;

// The kernel indexes strips, workgroups and per-row offsets with 32-bit
// counts and 64-bit byte offsets; these bounds keep every count in range.
constexpr int64_t kMaxF = (int64_t)1 << 31;
constexpr int64_t kMaxWorkgroups = ((int64_t)1 << 31) - 1;

typedef void (*kernel_fn)(const uint16_t *, uint8_t *, uint8_t *, uint64_t, uint32_t, uint32_t, uint32_t, int,
                          uint32_t);

// Row groups per thread, and non-temporal loads and stores (bit 0 | bit 1):
// every byte is touched exactly once, so nothing is worth keeping in cache.
constexpr int kGroupsPerThread = 1;
constexpr int kNonTemporal = 3;

template <int IN, int OUT> kernel_fn pick_nb(int nb)
{
    return nb == 2 ? (kernel_fn)mxq::quantize_kernel<IN, OUT, 2, kGroupsPerThread, kNonTemporal>
                   : (kernel_fn)mxq::quantize_kernel<IN, OUT, 1, kGroupsPerThread, kNonTemporal>;
}

template <int IN> kernel_fn pick_out(int out_dtype, int nb)
{
    switch (out_dtype) {
    case MXQ_OUT_E4M3FN: return pick_nb<IN, mxq::kOutE4M3FN>(nb);
    case MXQ_OUT_E5M2: return pick_nb<IN, mxq::kOutE5M2>(nb);
    default: return pick_nb<IN, mxq::kOutE2M1>(nb);
    }
}

typedef void (*dq_kernel_fn)(const uint8_t *, const uint8_t *, void *, uint64_t, uint32_t, uint32_t, uint32_t);

template <int FMT, int RES> dq_kernel_fn dq_pick_nb(int nb)
{
    return nb == 2 ? (dq_kernel_fn)mxq::dequantize_kernel<FMT, RES, 2, kNonTemporal>
                   : (dq_kernel_fn)mxq::dequantize_kernel<FMT, RES, 1, kNonTemporal>;
}

template <int RES> dq_kernel_fn dq_pick_fmt(int fmt, int nb)
{
    switch (fmt) {
    case MXQ_OUT_E4M3FN: return dq_pick_nb<mxq::kOutE4M3FN, RES>(nb);
    case MXQ_OUT_E5M2: return dq_pick_nb<mxq::kOutE5M2, RES>(nb);
    default: return dq_pick_nb<mxq::kOutE2M1, RES>(nb);
    }
}

// Largest normal exponent of each output format ("Block-Scale Computation",
// The EMAX Table): the bias subtracted from a block's maximum exponent.
int emax_of(int out_dtype)
{
    switch (out_dtype) {
    case MXQ_OUT_E4M3FN: return 8;
    case MXQ_OUT_E5M2: return 15;
    default: return 2;
    }
}

typedef void (*mm_kernel_fn)(const uint8_t *, const uint8_t *, const uint8_t *, const uint8_t *, uint32_t, uint32_t,
                             uint32_t, uint32_t, uint32_t, void *, uint8_t *, int);

// epi: mxq::kEpiF32, kEpiBF16, or kEpiMx + output format
template <int FMT> mm_kernel_fn mm_pick_epi(int epi)
{
    switch (epi) {
    case mxq::kEpiF32: return (mm_kernel_fn)mxq::scaled_matmul_kernel<FMT, mxq::kEpiF32>;
    case mxq::kEpiBF16: return (mm_kernel_fn)mxq::scaled_matmul_kernel<FMT, mxq::kEpiBF16>;
    case mxq::kEpiMx + mxq::kOutE4M3FN: return (mm_kernel_fn)mxq::scaled_matmul_kernel<FMT, mxq::kEpiMx + mxq::kOutE4M3FN>;
    case mxq::kEpiMx + mxq::kOutE5M2: return (mm_kernel_fn)mxq::scaled_matmul_kernel<FMT, mxq::kEpiMx + mxq::kOutE5M2>;
    default: return (mm_kernel_fn)mxq::scaled_matmul_kernel<FMT, mxq::kEpiMx + mxq::kOutE2M1>;
    }
}

// Operand checks shared by the matmul entry points (everything but the
// result); returns MXQ_OK or the status to report.
int mm_check_operands(const void *lhs, const void *lhs_scale, const void *rhs, const void *rhs_scale, int64_t P,
                      int64_t M, int64_t N, int fmt)
{
    if (fmt != MXQ_OUT_E4M3FN && fmt != MXQ_OUT_E5M2)
        return MXQ_E_OUT_DTYPE;
    if (P < 0 || P % 8 != 0)
        return MXQ_E_SHAPE_P8;
    if (M < 0 || N < 0 || M % 4 != 0 || N % 4 != 0)
        return MXQ_E_SHAPE_F4;
    const int64_t kMax = ((int64_t)1 << 31) - 1;
    if (P > kMax || M > MXQ_MATMUL_MAX_COLS || N > MXQ_MATMUL_MAX_COLS)
        return MXQ_E_OVERFLOW;
    if (M > 0 && N > 0 && P > 0 && (!lhs || !lhs_scale || !rhs || !rhs_scale))
        return MXQ_E_NULL; // with P == 0 the operands are empty and never read
    if (((uintptr_t)lhs | (uintptr_t)lhs_scale | (uintptr_t)rhs | (uintptr_t)rhs_scale) & 15u)
        return MXQ_E_ALIGN;
    return MXQ_OK;
}

int mm_launch(int fmt, int epi, const void *lhs, const void *lhs_scale, const void *rhs, const void *rhs_scale,
              int64_t P, int64_t M, int64_t N, unsigned dense, void *out, void *out_scale, int emax_bias,
              void *stream)
{
    const int64_t tiles_m = (M + mxq::kMmTile - 1) / mxq::kMmTile;
    const int64_t tiles_n = (N + mxq::kMmTile - 1) / mxq::kMmTile;
    if (tiles_m > (((int64_t)1 << 31) - 1) / tiles_n)
        return MXQ_E_OVERFLOW;
    mm_kernel_fn k = fmt == MXQ_OUT_E4M3FN ? mm_pick_epi<mxq::kOutE4M3FN>(epi) : mm_pick_epi<mxq::kOutE5M2>(epi);
    const uint8_t *a0 = (const uint8_t *)lhs;
    const uint8_t *a1 = (const uint8_t *)lhs_scale;
    const uint8_t *a2 = (const uint8_t *)rhs;
    const uint8_t *a3 = (const uint8_t *)rhs_scale;
    uint32_t a4 = (uint32_t)P, a5 = (uint32_t)M, a6 = (uint32_t)N, a7 = (uint32_t)tiles_n;
    uint32_t a8 = dense ? 1u : 0u;
    void *a9 = out;
    uint8_t *a10 = (uint8_t *)out_scale;
    int a11 = emax_bias;
    void *args[] = {&a0, &a1, &a2, &a3, &a4, &a5, &a6, &a7, &a8, &a9, &a10, &a11};
    hipError_t err = hipLaunchKernel((const void *)k, dim3((uint32_t)(tiles_m * tiles_n)), dim3(mxq::kMmThreads), args,
                                     0, (hipStream_t)stream);
    return err == hipSuccess ? MXQ_OK : MXQ_E_HIP;
}

int check_shape(int64_t P, int64_t F)
{
    if (P < 0 || P % 8 != 0)
        return MXQ_E_SHAPE_P8;
    if (F < 0 || F % 4 != 0)
        return MXQ_E_SHAPE_F4;
    if (F > kMaxF)
        return MXQ_E_OVERFLOW;
    if (F > 0 && P > INT64_MAX / 2 / F)
        return MXQ_E_OVERFLOW; // input bytes P*F*2 must fit
    return MXQ_OK;
}

} // namespace

extern "C" {

int mxq_abi_version(void) { return MXQ_ABI_VERSION; }

const char *mxq_status_string(int status)
{
    switch (status) {
    case MXQ_OK: return "ok";
    case MXQ_E_IN_DTYPE: return "input element type must be BF16 or F16";
    case MXQ_E_OUT_DTYPE: return "output element type must be float8_e4m3fn, float8_e5m2 or float4_e2m1";
    case MXQ_E_SHAPE_P8: return "P must be a non-negative multiple of 8 (a block spans 8 partitions)";
    case MXQ_E_SHAPE_F4: return "F must be a non-negative multiple of 4 (x4 packing, 4 columns per block)";
    case MXQ_E_NULL: return "a buffer pointer is NULL";
    case MXQ_E_ALIGN: return "buffer pointers must be 16-byte aligned";
    case MXQ_E_OVERFLOW: return "tensor too large for the library's index range";
    case MXQ_E_HIP: return "the HIP runtime rejected the kernel launch";
    case MXQ_E_FLAGS: return "unknown flag bits";
    case MXQ_E_RES_DTYPE: return "dequantize result type must be F32 or BF16";
    default: return "unknown status";
    }
}

size_t mxq_data_bytes(int64_t P, int64_t F, int out_dtype)
{
    if (check_shape(P, F) != MXQ_OK)
        return 0;
    switch (out_dtype) {
    case MXQ_OUT_E4M3FN:
    case MXQ_OUT_E5M2: return (size_t)(P * F);
    case MXQ_OUT_E2M1: return (size_t)(P * F / 2);
    default: return 0;
    }
}

size_t mxq_scale_image_bytes(int64_t P, int64_t F)
{
    if (check_shape(P, F) != MXQ_OK)
        return 0;
    return (size_t)(P * (F / 4));
}

size_t mxq_scale_bytes(int64_t P, int64_t F, unsigned flags)
{
    if (check_shape(P, F) != MXQ_OK || (flags & ~(unsigned)(MXQ_FLAG_ALT_EMAX | MXQ_FLAG_DENSE_SCALE)))
        return 0;
    return (size_t)((flags & MXQ_FLAG_DENSE_SCALE) ? (P / 8) * (F / 4) : P * (F / 4));
}

size_t mxq_result_bytes(int64_t P, int64_t F, int res_dtype)
{
    if (check_shape(P, F) != MXQ_OK)
        return 0;
    switch (res_dtype) {
    case MXQ_RES_F32: return (size_t)(P * F) * 4;
    case MXQ_RES_BF16: return (size_t)(P * F) * 2;
    default: return 0;
    }
}

int mxq_dequantize(const void *data, const void *scale_in, int64_t P, int64_t F, int fmt, int res_dtype,
                   void *out, void *stream)
{
    return mxq_dequantize_ex(data, scale_in, P, F, fmt, res_dtype, 0u, out, stream);
}

int mxq_dequantize_ex(const void *data, const void *scale_in, int64_t P, int64_t F, int fmt, int res_dtype,
                      unsigned flags, void *out, void *stream)
{
    if (fmt != MXQ_OUT_E4M3FN && fmt != MXQ_OUT_E5M2 && fmt != MXQ_OUT_E2M1)
        return MXQ_E_OUT_DTYPE;
    if (res_dtype != MXQ_RES_F32 && res_dtype != MXQ_RES_BF16)
        return MXQ_E_RES_DTYPE;
    if (flags & ~(unsigned)MXQ_FLAG_DENSE_SCALE)
        return MXQ_E_FLAGS;
    int rc = check_shape(P, F);
    if (rc != MXQ_OK)
        return rc;
    if (F > 0 && P > INT64_MAX / 4 / F)
        return MXQ_E_OVERFLOW; // fp32 result bytes P*F*4 must fit
    if (P == 0 || F == 0)
        return MXQ_OK;
    if (!data || !scale_in || !out)
        return MXQ_E_NULL;
    if (((uintptr_t)data | (uintptr_t)scale_in | (uintptr_t)out) & 15u)
        return MXQ_E_ALIGN;

    const int nb = (F % 8 == 0) ? 2 : 1;
    const int64_t nstrips = F / (4 * nb);
    const int64_t tiles_per_group = (nstrips + kThreads - 1) / kThreads;
    const int64_t groups = P / 8;
    if (groups > kMaxWorkgroups / tiles_per_group)
        return MXQ_E_OVERFLOW;

    dq_kernel_fn k = res_dtype == MXQ_RES_F32 ? dq_pick_fmt<mxq::kResF32>(fmt, nb)
                                              : dq_pick_fmt<mxq::kResBF16>(fmt, nb);
    const uint8_t *a0 = (const uint8_t *)data;
    const uint8_t *a1 = (const uint8_t *)scale_in;
    void *a2 = out;
    uint64_t a3 = (uint64_t)F;
    uint32_t a4 = (uint32_t)nstrips;
    uint32_t a5 = (uint32_t)tiles_per_group;
    uint32_t a6 = (flags & MXQ_FLAG_DENSE_SCALE) ? 1u : 0u;
    void *args[] = {&a0, &a1, &a2, &a3, &a4, &a5, &a6};
    hipError_t err = hipLaunchKernel((const void *)k, dim3((uint32_t)(groups * tiles_per_group)), dim3(kThreads),
                                     args, 0, (hipStream_t)stream);
    return err == hipSuccess ? MXQ_OK : MXQ_E_HIP;
}

int mxq_scaled_matmul(const void *lhs, const void *lhs_scale, const void *rhs, const void *rhs_scale, int64_t P,
                      int64_t M, int64_t N, int fmt, int res_dtype, unsigned flags, void *out, void *stream)
{
    if (fmt != MXQ_OUT_E4M3FN && fmt != MXQ_OUT_E5M2)
        return MXQ_E_OUT_DTYPE;
    if (res_dtype != MXQ_RES_F32 && res_dtype != MXQ_RES_BF16)
        return MXQ_E_RES_DTYPE;
    if (flags & ~(unsigned)MXQ_FLAG_DENSE_SCALE)
        return MXQ_E_FLAGS;
    int rc = mm_check_operands(lhs, lhs_scale, rhs, rhs_scale, P, M, N, fmt);
    if (rc != MXQ_OK)
        return rc;
    if (M == 0 || N == 0)
        return MXQ_OK;
    if (!out)
        return MXQ_E_NULL;
    if ((uintptr_t)out & 15u)
        return MXQ_E_ALIGN;
    return mm_launch(fmt, res_dtype == MXQ_RES_F32 ? mxq::kEpiF32 : mxq::kEpiBF16, lhs, lhs_scale, rhs, rhs_scale,
                     P, M, N, flags & MXQ_FLAG_DENSE_SCALE, out, nullptr, 0, stream);
}

int mxq_scaled_matmul_quantize(const void *lhs, const void *lhs_scale, const void *rhs, const void *rhs_scale,
                               int64_t P, int64_t M, int64_t N, int fmt, int out_dtype, unsigned flags,
                               void *data_out, void *scale_out, void *stream)
{
    if (fmt != MXQ_OUT_E4M3FN && fmt != MXQ_OUT_E5M2)
        return MXQ_E_OUT_DTYPE;
    if (out_dtype != MXQ_OUT_E4M3FN && out_dtype != MXQ_OUT_E5M2 && out_dtype != MXQ_OUT_E2M1)
        return MXQ_E_OUT_DTYPE;
    if (flags & ~(unsigned)(MXQ_FLAG_ALT_EMAX | MXQ_FLAG_DENSE_SCALE))
        return MXQ_E_FLAGS;
    if (M % 8 != 0)
        return MXQ_E_SHAPE_P8; // the result's rows form the quantize's row groups
    int rc = mm_check_operands(lhs, lhs_scale, rhs, rhs_scale, P, M, N, fmt);
    if (rc != MXQ_OK)
        return rc;
    if (M == 0 || N == 0)
        return MXQ_OK;
    if (!data_out || !scale_out)
        return MXQ_E_NULL;
    if (((uintptr_t)data_out | (uintptr_t)scale_out) & 15u)
        return MXQ_E_ALIGN;
    const int bias = emax_of(out_dtype) - ((flags & MXQ_FLAG_ALT_EMAX) ? 1 : 0);
    return mm_launch(fmt, mxq::kEpiMx + out_dtype, lhs, lhs_scale, rhs, rhs_scale, P, M, N,
                     flags & MXQ_FLAG_DENSE_SCALE, data_out, scale_out, bias, stream);
}

int mxq_quantize(const void *in, int64_t P, int64_t F, int in_dtype, int out_dtype, void *data_out,
                 void *scale_out, void *stream)
{
    return mxq_quantize_ex(in, P, F, in_dtype, out_dtype, 0u, data_out, scale_out, stream);
}

int mxq_quantize_ex(const void *in, int64_t P, int64_t F, int in_dtype, int out_dtype, unsigned flags,
                    void *data_out, void *scale_out, void *stream)
{
    if (in_dtype != MXQ_IN_BF16 && in_dtype != MXQ_IN_F16)
        return MXQ_E_IN_DTYPE;
    if (out_dtype != MXQ_OUT_E4M3FN && out_dtype != MXQ_OUT_E5M2 && out_dtype != MXQ_OUT_E2M1)
        return MXQ_E_OUT_DTYPE;
    if (flags & ~(unsigned)(MXQ_FLAG_ALT_EMAX | MXQ_FLAG_DENSE_SCALE))
        return MXQ_E_FLAGS;
    int rc = check_shape(P, F);
    if (rc != MXQ_OK)
        return rc;
    if (P == 0 || F == 0)
        return MXQ_OK;
    if (!in || !data_out || !scale_out)
        return MXQ_E_NULL;
    if (((uintptr_t)in | (uintptr_t)data_out | (uintptr_t)scale_out) & 15u)
        return MXQ_E_ALIGN;

    const int nb = (F % 8 == 0) ? 2 : 1;
    const int64_t nstrips = F / (4 * nb);
    const uint32_t threads = kThreads;
    const int64_t tiles_per_band = (nstrips + threads - 1) / threads;
    const int64_t groups = P / 8;
    const int64_t bands = (groups + kGroupsPerThread - 1) / kGroupsPerThread;
    if (bands > kMaxWorkgroups / tiles_per_band)
        return MXQ_E_OVERFLOW;

    kernel_fn k = in_dtype == MXQ_IN_BF16 ? pick_out<mxq::kInBF16>(out_dtype, nb)
                                          : pick_out<mxq::kInF16>(out_dtype, nb);
    const uint16_t *a0 = (const uint16_t *)in;
    uint8_t *a1 = (uint8_t *)data_out;
    uint8_t *a2 = (uint8_t *)scale_out;
    uint64_t a3 = (uint64_t)F;
    uint32_t a4 = (uint32_t)nstrips;
    uint32_t a5 = (uint32_t)tiles_per_band;
    uint32_t a6 = (uint32_t)groups;
    int a7 = emax_of(out_dtype) - ((flags & MXQ_FLAG_ALT_EMAX) ? 1 : 0);
    uint32_t a8 = (flags & MXQ_FLAG_DENSE_SCALE) ? 1u : 0u;
    void *args[] = {&a0, &a1, &a2, &a3, &a4, &a5, &a6, &a7, &a8};
    hipError_t err = hipLaunchKernel((const void *)k, dim3((uint32_t)(bands * tiles_per_band)), dim3(threads),
                                     args, 0, (hipStream_t)stream);
    return err == hipSuccess ? MXQ_OK : MXQ_E_HIP;
}

} // extern "C"
