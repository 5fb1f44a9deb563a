// mxq_axis_api.hip -- mxq_quantize_axis: validation, the [K/4, 4*O] view's
// geometry, and dispatch to quantize_down_kernel (dim -2) or
// quantize_along_kernel (dim -1) on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq.h"
#include "mxq_host.hpp"
#include "mxq_axis_kernels.hpp"

namespace {

using mxq_host::check_shape;
using mxq_host::emax_of;
using mxq_host::kMaxF;
using mxq_host::grid_fits;

typedef void (*down_kernel_fn)(const uint16_t *, uint8_t *, uint8_t *, uint64_t, uint32_t, uint32_t, int, uint32_t);
typedef void (*along_kernel_fn)(const uint16_t *, uint8_t *, uint8_t *, uint64_t, uint64_t, uint32_t, int, uint32_t,
                                uint32_t);

// The down kernel's workgroups are renumbered so that each XCD walks one
// contiguous range of tiles when the view rows do not start on 128-byte
// lines, as for the plain quantize (N = 8200: 630 -> 566 us). The along
// kernel slows down under that renumbering at every pitch; instead, when
// the row count is not a multiple of its 256-row tile (so its view-row runs
// do not start on run-size boundaries), each XCD takes four adjacent row
// tiles of every window of 32 workgroups. 8192 columns, bf16 -> e4m3fn:
// 131080 rows 621 -> 593 us, 131074 672 -> 631 us, 131040 593 -> 565 us;
// multiples of 256 rows are as fast or faster without it (131072: 545 us).
//
// The down kernel with four-column strips on such a pitch owns its lines, as
// the plain quantize does: each workgroup quantizes 128 bytes' worth of
// strips beyond its own and writes exactly the 128-byte lines that start
// inside its own (W [131072, 8200], bit-identical; two boxes):
//   -> e4m3fn 568 -> 546 us at 8 waves per CU, 551 -> 524 us at 7 (537 at 6)
//   -> e2m1   489 -> 477 us at 8, 469 -> 459 us at 8 (482 at 7)
constexpr int kXcds = 8;

template <int IN, int OUT, int XCD> down_kernel_fn down_pick_nb(int nb, bool own)
{
    if constexpr (XCD != 0) {
        if (own && nb == 4)
            return (down_kernel_fn)mxq::quantize_down_kernel<IN, OUT, 4, XCD, 1>;
    }
    switch (nb) {
    case 4: return (down_kernel_fn)mxq::quantize_down_kernel<IN, OUT, 4, XCD>;
    case 2: return (down_kernel_fn)mxq::quantize_down_kernel<IN, OUT, 2, XCD>;
    default: return (down_kernel_fn)mxq::quantize_down_kernel<IN, OUT, 1, XCD>;
    }
}

template <int IN, int OUT> down_kernel_fn down_pick(int nb, bool aligned, bool own)
{
    return aligned ? down_pick_nb<IN, OUT, 0>(nb, false) : down_pick_nb<IN, OUT, kXcds>(nb, own);
}

template <int IN, int OUT> along_kernel_fn along_pick(int narrow)
{
    return narrow ? (along_kernel_fn)mxq::quantize_along_kernel<IN, OUT, 1>
                  : (along_kernel_fn)mxq::quantize_along_kernel<IN, OUT, 0>;
}

template <int IN>
void axis_pick(int out_dtype, int down, int width, bool aligned, bool own, down_kernel_fn *d,
               along_kernel_fn *a)
{
    switch (out_dtype) {
    case MXQ_OUT_E4M3FN:
        *d = down ? down_pick<IN, mxq::kOutE4M3FN>(width, aligned, own) : nullptr;
        *a = down ? nullptr : along_pick<IN, mxq::kOutE4M3FN>(width);
        break;
    case MXQ_OUT_E5M2:
        *d = down ? down_pick<IN, mxq::kOutE5M2>(width, aligned, own) : nullptr;
        *a = down ? nullptr : along_pick<IN, mxq::kOutE5M2>(width);
        break;
    default:
        *d = down ? down_pick<IN, mxq::kOutE2M1>(width, aligned, own) : nullptr;
        *a = down ? nullptr : along_pick<IN, mxq::kOutE2M1>(width);
        break;
    }
}

} // namespace

extern "C" {

int mxq_quantize_axis(const void *in, int64_t R, int64_t C, int in_dtype, int out_dtype, int dim, unsigned flags,
                      void *data_out, void *scale_out, void *stream)
{
    if (in_dtype != MXQ_IN_BF16 && in_dtype != MXQ_IN_F16)
        return MXQ_E_IN_DTYPE;
    if (out_dtype != MXQ_OUT_E4M3FN && out_dtype != MXQ_OUT_E5M2 && out_dtype != MXQ_OUT_E2M1)
        return MXQ_E_OUT_DTYPE;
    if (flags & ~(unsigned)(MXQ_FLAG_ALT_EMAX | MXQ_FLAG_DENSE_SCALE))
        return MXQ_E_FLAGS;
    if (dim < 0)
        dim += 2; // rank 2: -1 -> 1 (last), -2 -> 0 (second-to-last)
    if (dim != 0 && dim != 1)
        return MXQ_E_DIM;
    if (R < 0 || C < 0)
        return MXQ_E_SHAPE_F4;
    const int down = dim == 0;
    const int64_t K = down ? R : C, O = down ? C : R;
    if (K % 32 != 0)
        return MXQ_E_SHAPE_P8;
    if (O > kMaxF / 4)
        return MXQ_E_OVERFLOW;
    int rc = check_shape(K / 4, 4 * O); // the [K/4, 4*O] view's limits
    if (rc != MXQ_OK)
        return rc;
    if (R == 0 || C == 0)
        return MXQ_OK;
    if (!in || !data_out || !scale_out)
        return MXQ_E_NULL;
    if (((uintptr_t)in | (uintptr_t)data_out | (uintptr_t)scale_out) & 15u)
        return MXQ_E_ALIGN;

    const int bias = emax_of(out_dtype) - ((flags & MXQ_FLAG_ALT_EMAX) ? 1 : 0);
    const uint32_t dense = (flags & MXQ_FLAG_DENSE_SCALE) ? 1u : 0u;
    const int64_t threads = 64;
    int width;
    int64_t grid, tiles;
    const bool aligned = (out_dtype == MXQ_OUT_E2M1 ? 2 * O : 4 * O) % 128 == 0; // view row pitch
    // line ownership (down kernel, four-column strips, misaligned view rows
    // that one 32-bit buffer range covers with room for the dropped offset)
    const bool own = down && !aligned && O % 4 == 0 && 4 * O < (int64_t)mxq::kDropOffset;
    if (down) {
        width = (O % 4 == 0) ? 4 : (O % 2 == 0) ? 2 : 1; // columns per thread
        const int64_t per_tile = own ? threads - 128 / (out_dtype == MXQ_OUT_E2M1 ? 8 : 16) : threads;
        tiles = (O / width + per_tile - 1) / per_tile;   // per 32-row band
        if (!grid_fits(K / 32, tiles, threads))
            return MXQ_E_OVERFLOW;
        grid = (K / 32) * tiles;
    } else {
        width = O % 4 != 0;                                   // rows of the view not 16-byte aligned
        tiles = (O + mxq::kAlongRows - 1) / mxq::kAlongRows; // row tiles
        const int64_t ktiles = (K / 32 + 1) / 2;              // two blocks per tile
        if (!grid_fits(ktiles, tiles, 64 * mxq::kAlongWaves))
            return MXQ_E_OVERFLOW;
        grid = ktiles * tiles;
    }
    down_kernel_fn dk = nullptr;
    along_kernel_fn ak = nullptr;
    if (in_dtype == MXQ_IN_BF16)
        axis_pick<mxq::kInBF16>(out_dtype, down, width, aligned, own, &dk, &ak);
    else
        axis_pick<mxq::kInF16>(out_dtype, down, width, aligned, own, &dk, &ak);

    const uint16_t *a0 = (const uint16_t *)in;
    uint8_t *a1 = (uint8_t *)data_out;
    uint8_t *a2 = (uint8_t *)scale_out;
    int a6 = bias;
    uint32_t a7 = dense;
    hipError_t err;
    if (down) {
        uint64_t a3 = (uint64_t)O;
        uint32_t a4 = (uint32_t)(O / width), a5 = (uint32_t)tiles;
        void *args[] = {&a0, &a1, &a2, &a3, &a4, &a5, &a6, &a7};
        // at most 8 waves per CU once the tensor outgrows the cache (1.07 G
        // elements: 514 us uncapped, 487 us capped), 12 for one-column
        // strips, whose threads move a quarter of the bytes (32768 x 32769:
        // 746 us at 8, 665 us at 12; two- and four-column strips are fastest
        // at 8); the along kernel's own LDS tile already sets its residency,
        // and more reserve slows it
        // (owned lines: 7 for FP8, 8 for FP4, from the sweep above)
        const uint32_t waves = own ? (out_dtype == MXQ_OUT_E2M1 ? 8u : 7u) : width == 1 ? 12u : 8u;
        const uint32_t lds = mxq_host::occupancy_cap_lds(K * O, 3, (uint32_t)threads, waves);
        err = hipLaunchKernel((const void *)dk, dim3((uint32_t)grid), dim3((uint32_t)threads), args, lds,
                              (hipStream_t)stream);
    } else {
        uint64_t a3 = (uint64_t)O, a4 = (uint64_t)K;
        uint32_t a5 = (uint32_t)tiles;
        uint32_t a8 = O % mxq::kAlongRows != 0 ? 1u : 0u;
        void *args[] = {&a0, &a1, &a2, &a3, &a4, &a5, &a6, &a7, &a8};
        err = hipLaunchKernel((const void *)ak, dim3((uint32_t)grid), dim3(64 * mxq::kAlongWaves), args, 0,
                              (hipStream_t)stream);
    }
    return err == hipSuccess ? MXQ_OK : MXQ_E_HIP;
}

} // extern "C"
