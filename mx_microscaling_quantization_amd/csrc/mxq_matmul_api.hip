// mxq_matmul_api.hip -- mxq_scaled_matmul and mxq_scaled_matmul_quantize:
// operand validation and the launch of scaled_matmul_kernel (one
// 512-thread workgroup per 256 x 256 output tile) on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq.h"
#include "mxq_host.hpp"
#include "mxq_matmul_kernels.hpp"

namespace {

using mxq_host::check_shape;
using mxq_host::emax_of;
using mxq_host::kMaxF;
using mxq_host::grid_fits;

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
    if (!grid_fits(tiles_m, tiles_n, mxq::kMmThreads))
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

} // namespace

extern "C" {

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

} // extern "C"
