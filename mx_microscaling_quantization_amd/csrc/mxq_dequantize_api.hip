// mxq_dequantize_api.hip -- mxq_dequantize / mxq_dequantize_ex: validation,
// launch geometry and dispatch to dequantize_kernel on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq.h"
#include "mxq_host.hpp"
#include "mxq_dequantize_kernels.hpp"

namespace {

using mxq_host::check_shape;
using mxq_host::emax_of;
using mxq_host::kMaxF;
using mxq_host::grid_fits;

// One 64-lane wave per workgroup, non-temporal loads and stores (the data
// streams through once), as for the quantize. When the result rows do not
// start on 128-byte lines, workgroups are renumbered so that each XCD walks
// one contiguous range of tiles and the lines neighbours share stay in one
// L2, as for the quantize (F = 8200: 666 -> 565 us; F = 8188: 889 -> 581
// us; aligned pitches are faster without it).
//
// On such a pitch workgroups own their lines: with 16 result bytes per
// thread and row (bf16 with two-block strips, f32) each decodes 56 strips of
// its own and the next 8, with 8 bytes (bf16 with one-block strips, F % 8 ==
// 4) 48 and the next 16, and writes exactly the 128-byte lines that start
// inside its own strips, the stores of rows it does not own dropped by the
// buffer's range check. No line is then written in part by two workgroups
// (but the one a row boundary splits). 131072 rows, same box, against the
// shared-line launch (all bit-identical):
//   F = 8200: e4m3fn -> bf16 542 -> 525 us (cap 8), -> f32 894 -> 837 us
//             (cap 10); e2m1 -> bf16 546 -> 452 us (cap 14), -> f32
//             866 -> 776 us (cap 10)
//   F = 8208: 530 -> 524, 883 -> 834, 519 -> 453, 795 -> 780 us
//   F = 8188 (one-block bf16): e4m3fn 590 -> 564 us (cap 16; 586 at 14,
//             580 at 20), e2m1 530 -> 495 us (cap 24; 528 at 20, 503 at 32)
constexpr uint32_t kThreads = 64;
constexpr int kNonTemporal = 3;
constexpr int kXcds = 8;

typedef void (*dq_kernel_fn)(const uint8_t *, const uint8_t *, void *, uint64_t, uint32_t, uint32_t, uint32_t);

template <int FMT, int RES, int XCD> dq_kernel_fn dq_pick_nb(int nb, bool own)
{
    if constexpr (XCD != 0) {
        if (own) {
            if constexpr (RES == mxq::kResF32) // f32 takes one-block strips only
                return (dq_kernel_fn)mxq::dequantize_kernel<FMT, RES, 1, kNonTemporal, XCD, 1>;
            else
                return nb == 2 ? (dq_kernel_fn)mxq::dequantize_kernel<FMT, RES, 2, kNonTemporal, XCD, 1>
                               : (dq_kernel_fn)mxq::dequantize_kernel<FMT, RES, 1, kNonTemporal, XCD, 1>;
        }
    }
    return nb == 2 ? (dq_kernel_fn)mxq::dequantize_kernel<FMT, RES, 2, kNonTemporal, XCD>
                   : (dq_kernel_fn)mxq::dequantize_kernel<FMT, RES, 1, kNonTemporal, XCD>;
}

template <int RES, int XCD> dq_kernel_fn dq_pick_fmt(int fmt, int nb, bool own)
{
    switch (fmt) {
    case MXQ_OUT_E4M3FN: return dq_pick_nb<mxq::kOutE4M3FN, RES, XCD>(nb, own);
    case MXQ_OUT_E5M2: return dq_pick_nb<mxq::kOutE5M2, RES, XCD>(nb, own);
    default: return dq_pick_nb<mxq::kOutE2M1, RES, XCD>(nb, own);
    }
}

} // namespace

extern "C" {

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

    // Two blocks per thread where the stores stay whole: 8 bf16 results are
    // one 16-byte store per row. With f32 results a thread would write 32
    // bytes as two 16-byte stores 32 bytes apart, each store instruction
    // covering every other 16 bytes of its lines; one block per thread keeps
    // each store lane-contiguous (1.07 G elements, e4m3fn -> f32: 1792 us
    // with two blocks, 851 us with one).
    const int nb = (F % 8 == 0 && res_dtype != MXQ_RES_F32) ? 2 : 1;
    const int64_t rowbytes = F * (res_dtype == MXQ_RES_F32 ? 4 : 2);
    const uint32_t lane_bytes = 4u * nb * (res_dtype == MXQ_RES_F32 ? 4u : 2u); // 8 or 16
    const bool aligned = rowbytes % 128 == 0; // result row pitch
    // line ownership on misaligned pitches, for rows that one 32-bit buffer
    // range covers with room for the dropped offset
    const bool own = !aligned && rowbytes < (int64_t)mxq::kDropOffset;
    const int64_t nstrips = F / (4 * nb);
    const int64_t per_tile = own ? kThreads - mxq::dq_own_extra(lane_bytes) : kThreads;
    const int64_t tiles_per_group = (nstrips + per_tile - 1) / per_tile;
    const int64_t groups = P / 8;
    if (!grid_fits(groups, tiles_per_group, kThreads))
        return MXQ_E_OVERFLOW;

    dq_kernel_fn k = res_dtype == MXQ_RES_F32
                         ? (aligned ? dq_pick_fmt<mxq::kResF32, 0>(fmt, nb, false)
                                    : dq_pick_fmt<mxq::kResF32, kXcds>(fmt, nb, own))
                         : (aligned ? dq_pick_fmt<mxq::kResBF16, 0>(fmt, nb, false)
                                    : dq_pick_fmt<mxq::kResBF16, kXcds>(fmt, nb, own));
    const uint8_t *a0 = (const uint8_t *)data;
    const uint8_t *a1 = (const uint8_t *)scale_in;
    void *a2 = out;
    uint64_t a3 = (uint64_t)F;
    uint32_t a4 = (uint32_t)nstrips;
    uint32_t a5 = (uint32_t)tiles_per_group;
    uint32_t a6 = (flags & MXQ_FLAG_DENSE_SCALE) ? 1u : 0u;
    void *args[] = {&a0, &a1, &a2, &a3, &a4, &a5, &a6};
    // A residency cap once the tensor outgrows the cache, set per path by a
    // sweep at 131072 x 8192 (waves per CU 6, 8, 10, 12, 16, uncapped):
    //   e4m3fn -> f32   6: 824-832 us, 8: 844-855 us, uncapped 904 us
    //   e2m1 -> f32     8: 708 us, 10: 741 us, 6: 853 us
    //   e4m3fn -> bf16  6: 472-474 us, 8: 478-479 us, uncapped 513 us
    //   e2m1 -> bf16    16: 417 us, 12: 435 us, 8: 470 us
    // One-block strips (F % 8 == 4) keep their earlier sweep: 8 waves, 12
    // for FP4 -> bf16, which moves the fewest bytes per thread (131072 x
    // 8188: 581 us at 8, 521 us at 12).
    // Line-owning launches: caps from the sweep above (f32 10; bf16 with
    // two-block strips FP8 8, FP4 14; with one-block strips FP8 16, FP4 24).
    uint32_t waves;
    if (own && res_dtype == MXQ_RES_F32)
        waves = 10u;
    else if (own)
        waves = nb == 2 ? (fmt == MXQ_OUT_E2M1 ? 14u : 8u) : (fmt == MXQ_OUT_E2M1 ? 24u : 16u);
    else if (res_dtype == MXQ_RES_F32)
        waves = fmt == MXQ_OUT_E2M1 ? 8u : 6u;
    else if (nb == 2)
        waves = fmt == MXQ_OUT_E2M1 ? 16u : 6u;
    else
        waves = fmt == MXQ_OUT_E2M1 ? 12u : 8u;
    const uint32_t lds = mxq_host::occupancy_cap_lds(P * F, res_dtype == MXQ_RES_F32 ? 5 : 3, kThreads, waves);
    hipError_t err = hipLaunchKernel((const void *)k, dim3((uint32_t)(groups * tiles_per_group)), dim3(kThreads),
                                     args, lds, (hipStream_t)stream);
    return err == hipSuccess ? MXQ_OK : MXQ_E_HIP;
}

} // extern "C"
