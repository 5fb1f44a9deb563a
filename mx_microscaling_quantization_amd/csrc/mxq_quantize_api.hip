// mxq_quantize_api.hip -- mxq_quantize / mxq_quantize_ex: validation, launch
// geometry and dispatch on (input type, output type, strip width) to
// quantize_kernel, launched on the caller's stream. No allocation, no state.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq.h"
#include "mxq_host.hpp"
#include "mxq_quantize_kernels.hpp"

namespace {

using mxq_host::check_shape;
using mxq_host::emax_of;
using mxq_host::kMaxF;
using mxq_host::grid_fits;

// Workgroups of one wave stream this kernel fastest, with a residency cap
// once the tensor outgrows the cache: at most 10 waves per CU for FP8 output
// (2:1 read/write; 1.07 G-element bf16 -> e4m3fn: 488 us uncapped, 473 us
// capped) and 8 for FP4 output (4:1; -> e2m1: 434 us uncapped, 414 us at 10,
// 391 us at 8). A thread of one-block strips (F % 8 == 4) moves half the
// bytes, so 12 waves keep as much in flight (131072 x 8188: -> e4m3fn 549 us
// at 10, 535 us at 12; -> e2m1 529 us at 8, 437 us at 12).
constexpr uint32_t kThreads = 64;
inline uint32_t waves_per_cu(int out_dtype, int nb)
{
    if (nb == 1)
        return 12u;
    return out_dtype == MXQ_OUT_E2M1 ? 8u : 10u;
}

// When the data rows do not start on 128-byte lines (row pitch F bytes for
// FP8, F/2 for FP4, not a multiple of 128), neighbouring workgroups share
// the first and last line of each row segment. Workgroups go to the 8 XCDs
// round-robin, so neighbours sit behind different L2 caches and both write
// partial lines. Renumbering the workgroups so that each XCD walks one
// contiguous range of tiles keeps both halves of almost every shared line
// in one L2 (F = 8200: 729 -> 538 us; F = 8188: 944 -> 582 us; aligned
// pitches measured faster without it).
//
// FP8 output with two-block strips on such a pitch goes further: each
// one-wave workgroup owns 48 strips, also quantizes the next 16, and writes
// exactly the 128-byte lines that start inside its own strips, so that every
// line but the one a row boundary splits is written whole by one wave. The
// extra strips cost a third more loads (L2 hits: the neighbour reads them
// too). 131072 rows -> e4m3fn, same box, caps 10 / 11 / 12 / 14 waves per
// CU: F = 8200 525 / 527 / 531 / 545 us (547 us with shared lines); F =
// 8208 518 / 518 / 522 / 534 us (537 us); the aligned F = 8192 takes 476 us.
// Narrower strips (one block, or FP4's 4 bytes a row) would need as many
// extra strips as owned ones; they keep the shared lines.
constexpr int kXcds = 8;
inline bool pitch_aligned(int64_t F, int out_dtype)
{
    return (out_dtype == MXQ_OUT_E2M1 ? F / 2 : F) % 128 == 0;
}
inline bool owns_lines(bool aligned, int out_dtype, int nb, int64_t F)
{
    // rows that one 32-bit buffer range covers with room for the dropped offset
    return !aligned && out_dtype != MXQ_OUT_E2M1 && nb == 2 && F < (int64_t)mxq::kDropOffset;
}

typedef void (*kernel_fn)(const uint16_t *, uint8_t *, uint8_t *, uint64_t, uint32_t, uint32_t, uint32_t, int,
                          uint32_t);

// Row groups per thread, and non-temporal loads and stores (bit 0 | bit 1):
// every byte is touched exactly once, so nothing is worth keeping in cache.
constexpr int kGroupsPerThread = 1;
constexpr int kNonTemporal = 3;

template <int IN, int OUT, int XCD> kernel_fn pick_nb(int nb, bool own)
{
    if constexpr (OUT != mxq::kOutE2M1 && XCD != 0) {
        if (own)
            return (kernel_fn)mxq::quantize_kernel<IN, OUT, 2, kGroupsPerThread, kNonTemporal, XCD, 1>;
    }
    return nb == 2 ? (kernel_fn)mxq::quantize_kernel<IN, OUT, 2, kGroupsPerThread, kNonTemporal, XCD>
                   : (kernel_fn)mxq::quantize_kernel<IN, OUT, 1, kGroupsPerThread, kNonTemporal, XCD>;
}

template <int IN, int XCD> kernel_fn pick_out(int out_dtype, int nb, bool own)
{
    switch (out_dtype) {
    case MXQ_OUT_E4M3FN: return pick_nb<IN, mxq::kOutE4M3FN, XCD>(nb, own);
    case MXQ_OUT_E5M2: return pick_nb<IN, mxq::kOutE5M2, XCD>(nb, own);
    default: return pick_nb<IN, mxq::kOutE2M1, XCD>(nb, own);
    }
}

} // namespace

extern "C" {

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
    const bool aligned = pitch_aligned(F, out_dtype);
    const bool own = owns_lines(aligned, out_dtype, nb, F);
    const uint32_t lds = mxq_host::occupancy_cap_lds(P * F, 3, threads, waves_per_cu(out_dtype, nb));
    const int64_t per_tile = own ? threads - mxq::kOwnExtra : threads;
    const int64_t tiles_per_band = (nstrips + per_tile - 1) / per_tile;
    const int64_t groups = P / 8;
    const int64_t bands = (groups + kGroupsPerThread - 1) / kGroupsPerThread;
    if (!grid_fits(bands, tiles_per_band, threads))
        return MXQ_E_OVERFLOW;

    kernel_fn k = in_dtype == MXQ_IN_BF16
                      ? (aligned ? pick_out<mxq::kInBF16, 0>(out_dtype, nb, false)
                                 : pick_out<mxq::kInBF16, kXcds>(out_dtype, nb, own))
                      : (aligned ? pick_out<mxq::kInF16, 0>(out_dtype, nb, false)
                                 : pick_out<mxq::kInF16, kXcds>(out_dtype, nb, own));
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
                                     args, lds, (hipStream_t)stream);
    return err == hipSuccess ? MXQ_OK : MXQ_E_HIP;
}

} // extern "C"
