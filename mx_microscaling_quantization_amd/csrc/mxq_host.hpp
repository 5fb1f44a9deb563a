// mxq_host.hpp -- host-side helpers shared by the library's entry points:
// the EMAX table, the index-range limits of the quantize geometry and the
// occupancy cap of the streaming kernels.
#pragma once

#include <stdint.h>

#include "mxq.h"

namespace mxq_host {

// The kernel indexes strips, workgroups and per-row offsets with 32-bit
// counts and 64-bit byte offsets; these bounds keep every count in range.
constexpr int64_t kMaxF = (int64_t)1 << 31;

// A launch's grid: `a` x `b` workgroups of `threads` threads. The dispatch
// packet counts work-items (workgroups x threads) in 32 bits, so a grid
// fits only when that product is at most 2^32 - 1 (which also keeps the
// workgroup count, a 32-bit kernel argument, in range).
constexpr int64_t kMaxWorkItems = ((int64_t)1 << 32) - 1;
inline bool grid_fits(int64_t a, int64_t b, int64_t threads)
{
    return a >= 0 && b > 0 && a <= kMaxWorkItems / threads / b;
}

// EMAX of an output format ("MX Microscaling: Quantize, Block-Scaling and
// E8M0", The EMAX Table).
inline int emax_of(int out_dtype)
{
    switch (out_dtype) {
    case MXQ_OUT_E4M3FN: return 8;
    case MXQ_OUT_E5M2: return 15;
    default: return 2;
    }
}

// LDS to reserve per workgroup of `wg_threads` threads so that a CU holds at
// most `waves_per_cu` waves of a streaming kernel, or 0 (no cap). The
// kernels never touch the reserve; it only limits residency. Once a call's
// traffic (elements x about `bytes_per_element`) exceeds the 256 MiB
// Infinity Cache, the stream runs from HBM, and there fewer waves in flight
// measured faster (the workgroups in flight keep fewer DRAM pages open);
// within the cache full occupancy is faster, so nothing is reserved.
constexpr int64_t kInfinityCacheBytes = (int64_t)256 << 20;
constexpr uint32_t kLdsBytesPerCU = 160u * 1024u;
inline uint32_t occupancy_cap_lds(int64_t elements, int64_t bytes_per_element, uint32_t wg_threads,
                                  uint32_t waves_per_cu)
{
    const uint32_t wgs = waves_per_cu / (wg_threads / 64);
    if (wgs == 0 || elements <= kInfinityCacheBytes / bytes_per_element)
        return 0;
    return kLdsBytesPerCU / wgs;
}

// P % 8, F % 4 and the byte-count limits of a [P, F] quantize.
inline int check_shape(int64_t P, int64_t F)
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

} // namespace mxq_host
