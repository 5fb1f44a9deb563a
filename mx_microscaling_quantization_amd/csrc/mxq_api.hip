// mxq_api.hip -- the C ABI's helpers (declared in mxq.h): ABI version,
// status messages and output sizes. The entry points that launch kernels
// live in one file per operation (mxq_*_api.hip).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq.h"
#include "mxq_host.hpp"

using mxq_host::check_shape;

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
    case MXQ_E_DIM: return "quantize axis must be the last (-1) or second-to-last (-2) dimension";
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

} // extern "C"
