// mxq_axis_kernels.hpp -- gfx950 kernels of the MX quantize along either axis
// of a plain row-major tensor.
//
// QuantizeMX's dim ("MX-FP8 Microscaling Legalization", The MX
// backend_config schemas; Normalize dim) picks the axis of the 32-element
// blocks: the last (-1) or the second-to-last (-2). With the crosswalk's
// block of 8 partitions x 4 elements and x4 containers along the block axis,
// an R x C tensor whose block axis has K elements (the other axis O) is
// quantized into the partition-major [K/4, 4*O] layout the plain quantize
// produces -- element (p, 4o + j) is block-axis element 4p + j at
// other-axis index o -- which is the layout the scaled matmul reads.
//
// Both kernels do the plain quantize's arithmetic with its own helpers
// (packed 16-bit block max, E8M0 clamp, scaled conversions, saturation,
// special-code pass); they differ only in how the 32 elements of a block
// reach the lanes that quantize them and where its codes go. One HBM pass,
// non-temporal hints.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "mxq_quantize_kernels.hpp"

namespace mxq {

// 16-bit element h (0/1) of a dword.
__device__ __forceinline__ uint32_t half16(uint32_t w, uint32_t h) { return (w >> (16u * h)) & 0xFFFFu; }

// Blocks down the columns (dim -2) of W [K][N] (row pitch N).
//
// A thread owns NB adjacent columns n0 .. n0 + NB - 1 of one band of 32 rows
// (row group g of the [K/4, 4N] view): it loads the 32 rows (2*NB bytes
// each; a wave's row load is 128*NB contiguous bytes), takes the NB block
// maxima with one packed max per loaded word, and for view row p = 8g + pr
// builds column b's x4 container from rows 4pr .. 4pr + 3. A view row of
// the strip is NB containers: 4*NB bytes (FP8) or 2*NB (FP4) at
// p * 4N + 4*n0 (FP8) / p * 2N + 2*n0 (FP4); the NB E8M0 bytes go to the
// placed (or dense) scale row at column n0.
//   nstrips   N / NB;  tiles_per_band  ceil(nstrips / strips per tile);
//   XCD != 0 renumbers workgroups as the plain quantize does (each XCD walks
//   one contiguous range of tiles)
// OWN != 0 (8 or 16 code bytes per thread and view row; for view rows that
// are not a multiple of 128 bytes): as in the plain quantize, a workgroup
// owns 64 - 128 / (bytes per thread) strips, also quantizes the next ones,
// and writes exactly the 128-byte lines that start inside its own strips.
template <int IN, int OUT, int NB, int XCD = 0, int OWN = 0>
__global__ __launch_bounds__(64) void quantize_down_kernel(const uint16_t *__restrict__ in,
                                                           uint8_t *__restrict__ data,
                                                           uint8_t *__restrict__ scale, uint64_t N,
                                                           uint32_t nstrips, uint32_t tiles_per_band,
                                                           int emax_bias, uint32_t dense)
{
    static_assert(NB == 1 || NB == 2 || NB == 4, "1, 2 or 4 columns per thread");
    constexpr int NW = (NB + 1) / 2;   // loaded dwords per row
    constexpr uint32_t LANE_BYTES = OUT == kOutE2M1 ? 2 * NB : 4 * NB; // code bytes per view row
    static_assert(!OWN || LANE_BYTES >= 8, "line ownership: 8 or 16 code bytes per view row");
    const uint32_t tile = tile_index<XCD>();
    const uint32_t band = tile / tiles_per_band;
    const uint32_t run = tile - band * tiles_per_band;
    const uint32_t owned = OWN ? 64u - 128u / LANE_BYTES : 64u;
    const uint32_t strip = run * owned + threadIdx.x;
    if (strip >= nstrips)
        return;
    const uint64_t n0 = (uint64_t)strip * NB;

    // With OWN: the view rows' buffers and this thread's store offsets (an
    // offset past the row's range for a row it does not own, which the
    // hardware drops), fixed before the loads in registers of their own, as
    // in the plain quantize. View row pitch < 2^31 bytes (checked on the host).
    __amdgpu_buffer_rsrc_t own_rs[8];
    uint32_t own_off[8];
    if constexpr (OWN) {
        const uint32_t rowbytes = (uint32_t)(OUT == kOutE2M1 ? 2 * N : 4 * N);
        const uint32_t c0 = LANE_BYTES * owned * run, c1 = c0 + LANE_BYTES * owned, c = LANE_BYTES * strip;
#pragma unroll
        for (int pr = 0; pr < 8; pr++) {
            uint8_t *rowp = data + ((uint64_t)band * 8u + pr) * rowbytes;
            const uint32_t mis = (uint32_t)(uintptr_t)rowp & 127u; // row start within its line
            const uint32_t lo = run == 0 ? 0u : ((mis + c0 + 127u) & ~127u) - mis;
            const uint32_t hi = run + 1 == tiles_per_band ? rowbytes : ((mis + c1 + 127u) & ~127u) - mis;
            own_rs[pr] = __builtin_amdgcn_make_buffer_rsrc(rowp, (short)0, (int)rowbytes, kBufferFlags);
            own_off[pr] = (c >= lo && c < hi) ? c : kDropOffset;
            asm volatile("" : "+v"(own_off[pr]));
        }
    }

    uint32_t v[32][NW];
    const uint16_t *rows = in + (uint64_t)band * 32u * N + n0;
#pragma unroll
    for (int r = 0; r < 32; r++) {
        const uint16_t *p = rows + (uint64_t)r * N;
        if constexpr (NB == 4) {
            const u32x2_t t = load<1>(reinterpret_cast<const u32x2_t *>(p));
            v[r][0] = t.x;
            v[r][1] = t.y;
        } else if constexpr (NB == 2) {
            v[r][0] = load<1>(reinterpret_cast<const uint32_t *>(p));
        } else {
            v[r][0] = load<1>(p);
        }
    }

    uint32_t e[NB];
    float s[NB];
    bool special = false;
#pragma unroll
    for (int h = 0; h < NW; h++) {
        uint32_t m = 0;
#pragma unroll
        for (int r = 0; r < 32; r++)
            m = pk_max_u16(m, v[r][h] & 0x7FFF7FFFu);
#pragma unroll
        for (int q = 0; q < 2 && 2 * h + q < NB; q++) {
            const uint32_t mag = half16(m, q);
            e[2 * h + q] = block_e8m0<IN>(mag, emax_bias);
            s[2 * h + q] = e8m0_to_scale(e[2 * h + q]);
            special |= mag > InfBits<IN>::value || e[2 * h + q] == 254u;
        }
    }

    // All 8 view rows' codes, then the rare special-code pass (which lays the
    // view rows out again from the loaded rows), then the 8 stores, each
    // with its own data and address registers: a store waiting on write
    // backpressure then holds up nothing after it.
    const uint64_t F = 4 * N;
    constexpr int OW = OUT == kOutE2M1 ? NW : NB;   // output words per view row
    // view row pr's input dwords, laid out as the plain quantize holds a
    // strip row: block b's elements j = 0..3 in w[2b] (j = 0, 1), w[2b+1]
    auto view_row = [&](int pr, uint32_t *w) {
#pragma unroll
        for (int b = 0; b < NB; b++) {
            const int h = b / 2, q = b & 1;
            w[2 * b] = half16(v[4 * pr][h], q) | half16(v[4 * pr + 1][h], q) << 16;
            w[2 * b + 1] = half16(v[4 * pr + 2][h], q) | half16(v[4 * pr + 3][h], q) << 16;
        }
    };
    uint32_t out[8][OW];
#pragma unroll
    for (int pr = 0; pr < 8; pr++) {
        uint32_t w[2 * NB];
        view_row(pr, w);
        if constexpr (OUT == kOutE2M1) {
#pragma unroll
            for (int h = 0; h < NW; h++) {
                out[pr][h] = fp4_container<IN, 0>(0u, w[4 * h], w[4 * h + 1], s[2 * h]);
                if constexpr (NB > 1)
                    out[pr][h] = fp4_container<IN, 1>(out[pr][h], w[4 * h + 2], w[4 * h + 3], s[2 * h + 1]);
            }
        } else {
#pragma unroll
            for (int b = 0; b < NB; b++)
                out[pr][b] = fp8x4<IN, OUT>(w[2 * b], w[2 * b + 1], s[b]);
        }
    }
    if (special) {
#pragma unroll
        for (int pr = 0; pr < 8; pr++) {
            uint32_t w[2 * NB];
            view_row(pr, w);
            fix_special_codes<IN, OUT, NB>(w, e, out[pr]);
        }
    }
    if constexpr (OWN) {
#pragma unroll
        for (int pr = 0; pr < 8; pr++) {
            if constexpr (LANE_BYTES == 16) {
                u32x4_t w = {out[pr][0], out[pr][1], out[pr][2], out[pr][3]};
                __builtin_amdgcn_raw_buffer_store_b128(w, own_rs[pr], (int)own_off[pr], 0, kBufferNT);
            } else {
                u32x2_t w = {out[pr][0], out[pr][1]};
                __builtin_amdgcn_raw_buffer_store_b64(w, own_rs[pr], (int)own_off[pr], 0, kBufferNT);
            }
        }
        if (threadIdx.x >= owned)
            return; // the next run's strips: their scales are that run's
    } else {
        uint8_t *dst[8];
#pragma unroll
        for (int pr = 0; pr < 8; pr++) {
            const uint64_t p = (uint64_t)band * 8u + pr;
            dst[pr] = OUT == kOutE2M1 ? data + (p * F) / 2 + 2 * n0 : data + p * F + 4 * n0;
        }
#pragma unroll
        for (int pr = 0; pr < 8; pr++)
            store_bytes<LANE_BYTES, 1>(dst[pr], out[pr]);
    }

    const uint64_t slot = dense ? (uint64_t)band : (uint64_t)(band & 3u) + 32u * (uint64_t)(band >> 2);
    uint32_t packed[1] = {0};
#pragma unroll
    for (int b = 0; b < NB; b++)
        packed[0] |= e[b] << (8 * b);
    store_bytes<NB, 1>(scale + slot * N + n0, packed);
}

// Max of x over the four lanes of each lane quad (DPP quad permutations; every
// lane of the wave must be active).
__device__ __forceinline__ uint32_t quad_max(uint32_t x)
{
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false)); // lane ^ 1
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false)); // lane ^ 2
    return x;
}

// Blocks along the rows (dim -1) of X [M][K] (row pitch K).
//
// A block is 32 contiguous elements of one row, and its codes go to 8 view
// rows at column m: 4 bytes (FP8) or 2 bytes (FP4) per view row. A lane per
// block would read one cache line per lane and write 4-byte pieces, so the
// codes go through LDS. A workgroup of kAlongWaves waves owns kAlongRows
// consecutive rows x 2 blocks (128 bytes of each row); wave w owns rows
// 128w .. 128w + 127 of the tile.
//  * Load: lane l reads 16-byte chunk c = l mod 8 (quarter q = c mod 4 of
//    block c/4: elements 8q .. 8q + 7, the containers of view rows 2q and
//    2q + 1) of wave row 4i + (k mod 4) + 32*(k/4), i = l/8, for its loads
//    k = 0..15. One load instruction reads 8 rows x 128 contiguous bytes.
//  * Block max: a lane-local packed max of its 8 elements, then two DPP steps
//    across the lane quad that holds the block's four quarters.
//  * Codes: after each four loads a lane holds four consecutive rows' codes
//    for each of its two view rows (16 or 8 bytes) and writes them into
//    that view row's LDS strip of kAlongRows codes; the quad's first lane
//    writes the four E8M0 bytes into the block's strip.
//  * Store: after one barrier each of the tile's 16 view rows leaves as one
//    contiguous run of kAlongRows codes (1 KiB for FP8), 16 (FP8) or 8 (FP4)
//    bytes per lane, and each scale strip as 4 bytes per lane. With NARROW
//    (M % 4 != 0: view rows are not 16-byte aligned) every lane stores one
//    row: 4 or 2 code bytes and 1 scale byte.
// Row tiles vary fastest over the grid (ceil(M / kAlongRows) x ceil(K / 64)),
// so the workgroups in flight write few view rows, each in long runs. With
// `chunked` each full window of 32 workgroups is renumbered so that the XCD
// receiving workgroups x, x + 8, x + 16 and x + 24 of it (they are dealt out
// round-robin) handles row tiles 4x .. 4x + 3 of the window: adjacent runs,
// and most lines at run boundaries, then stay behind one L2.
constexpr uint32_t kAlongWaves = 2;
constexpr uint32_t kAlongWaveRows = 128;
constexpr uint32_t kAlongRows = kAlongWaves * kAlongWaveRows;

template <int IN, int OUT, int NARROW>
__global__ __launch_bounds__(64 * kAlongWaves) void quantize_along_kernel(const uint16_t *__restrict__ in,
                                                                          uint8_t *__restrict__ data,
                                                                          uint8_t *__restrict__ scale, uint64_t M,
                                                                          uint64_t K, uint32_t tiles_m, int emax_bias,
                                                                          uint32_t dense, uint32_t chunked)
{
    constexpr uint32_t RT = kAlongRows, KG = kAlongWaveRows / 32; // four-load groups per lane
    constexpr uint32_t CB = OUT == kOutE2M1 ? 2 : 4;              // code bytes per row and view row
    constexpr uint32_t PITCH = RT * CB + 16;                      // LDS bytes per view-row strip
    static_assert(RT % 256 == 0 && 16 % kAlongWaves == 0, "whole 4-row lanes per store, whole view rows per wave");
    __shared__ __attribute__((aligned(16))) uint8_t codes[16 * PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t e8m0[2 * RT];

    const uint32_t t = threadIdx.x, w = t >> 6, l = t & 63u;
    const uint32_t c = l & 7u, i = l >> 3, q = c & 3u, bl = c >> 2;
    uint32_t tile = blockIdx.x;
    if (chunked && tile < gridDim.x / 32u * 32u)
        tile = (tile & ~31u) | (tile & 7u) << 2 | (tile >> 3 & 3u);
    const uint32_t tk = tile / tiles_m;
    const uint64_t m0 = (uint64_t)(tile - tk * tiles_m) * RT;
    const uint64_t G = K / 32;
    const uint64_t g = (uint64_t)tk * 2u + bl;

    // Every load is issued, back to back: a lane past the tensor reads the
    // first row of block column 0 (in bounds) and zeroes what it got. (With
    // the loads behind per-row branches, the compiler waited for the second
    // load to land before issuing the other fourteen.)
    u32x4_t v[4 * KG];
#pragma unroll
    for (uint32_t k = 0; k < 4 * KG; k++) {
        const uint64_t m = m0 + kAlongWaveRows * w + 4u * i + (k & 3u) + 32u * (k >> 2);
        const bool ok = g < G && m < M;
        v[k] = load<1>(reinterpret_cast<const u32x4_t *>(in + (ok ? m * K + g * 32u : 0u) + 8u * q));
        v[k] = ok ? v[k] : u32x4_t{0u, 0u, 0u, 0u};
    }

#pragma unroll
    for (uint32_t kg = 0; kg < KG; kg++) {
        uint32_t lo[4], hi[4], eb[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const u32x4_t x = v[4 * kg + j];
            uint32_t mm = pk_max_u16(x.x & 0x7FFF7FFFu, x.y & 0x7FFF7FFFu);
            mm = pk_max_u16(mm, x.z & 0x7FFF7FFFu);
            mm = pk_max_u16(mm, x.w & 0x7FFF7FFFu);
            const uint32_t mag = quad_max(max(mm & 0xFFFFu, mm >> 16));
            uint32_t e[1] = {block_e8m0<IN>(mag, emax_bias)};
            const float s = e8m0_to_scale(e[0]);
            uint32_t w0[2] = {x.x, x.y}, w1[2] = {x.z, x.w};
            uint32_t o0[1], o1[1];
            if constexpr (OUT == kOutE2M1) {
                o0[0] = fp4_container<IN, 0>(0u, w0[0], w0[1], s);
                o1[0] = fp4_container<IN, 0>(0u, w1[0], w1[1], s);
            } else {
                o0[0] = fp8x4<IN, OUT>(w0[0], w0[1], s);
                o1[0] = fp8x4<IN, OUT>(w1[0], w1[1], s);
            }
            if (mag > InfBits<IN>::value || e[0] == 254u) {
                fix_special_codes<IN, OUT, 1>(w0, e, o0);
                fix_special_codes<IN, OUT, 1>(w1, e, o1);
            }
            lo[j] = o0[0];
            hi[j] = o1[0];
            eb[j] = e[0];
        }
        const uint32_t r = kAlongWaveRows * w + 4u * i + 32u * kg; // first of the lane's four tile rows
        uint8_t *s0 = codes + (8u * bl + 2u * q) * PITCH + CB * r;
        if constexpr (OUT == kOutE2M1) {
            *reinterpret_cast<u32x2_t *>(s0) = u32x2_t{lo[0] | lo[1] << 16, lo[2] | lo[3] << 16};
            *reinterpret_cast<u32x2_t *>(s0 + PITCH) = u32x2_t{hi[0] | hi[1] << 16, hi[2] | hi[3] << 16};
        } else {
            *reinterpret_cast<u32x4_t *>(s0) = u32x4_t{lo[0], lo[1], lo[2], lo[3]};
            *reinterpret_cast<u32x4_t *>(s0 + PITCH) = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
        }
        if (q == 0)
            *reinterpret_cast<uint32_t *>(e8m0 + bl * RT + r) = eb[0] | eb[1] << 8 | eb[2] << 16 | eb[3] << 24;
    }
    __syncthreads();

    const uint64_t F = 4 * M;
    constexpr uint32_t RPL = NARROW ? 1 : 4;     // rows per lane and store
    constexpr uint32_t VPW = 16 / kAlongWaves;   // view rows per wave
    constexpr uint32_t SPR = RT / (64 * RPL);    // stores per view row and lane
    // the store's type: RPL rows of CB code bytes
    using T = typename std::conditional<NARROW, typename std::conditional<OUT == kOutE2M1, uint16_t, uint32_t>::type,
                                        typename std::conditional<OUT == kOutE2M1, u32x2_t, u32x4_t>::type>::type;
    // All of the wave's LDS reads first, then its stores, each with its own
    // data and address registers: a store waiting on write backpressure then
    // holds up nothing after it.
    T val[VPW][SPR];
    uint8_t *dst[VPW][SPR];
    bool ok[VPW][SPR];
#pragma unroll
    for (uint32_t j = 0; j < VPW; j++) {
        const uint32_t vr = VPW * w + j;
        const uint64_t gg = (uint64_t)tk * 2u + (vr >> 3);
        const uint64_t p = gg * 8u + (vr & 7u);
#pragma unroll
        for (uint32_t s = 0; s < SPR; s++) {
            const uint32_t r = 64u * RPL * s + RPL * l;
            ok[j][s] = gg < G && m0 + r < M;
            val[j][s] = *reinterpret_cast<const T *>(codes + vr * PITCH + CB * r);
            dst[j][s] = OUT == kOutE2M1 ? data + (p * F) / 2 + 2u * (m0 + r) : data + p * F + 4u * (m0 + r);
        }
    }
#pragma unroll
    for (uint32_t j = 0; j < VPW; j++)
#pragma unroll
        for (uint32_t s = 0; s < SPR; s++)
            if (ok[j][s])
                store<1>(reinterpret_cast<T *>(dst[j][s]), val[j][s]);
    // the two scale strips: the E8M0 of block gg for rows m0 .. m0 + RT - 1
    // goes to the placed (or dense) row of gg at column m
#pragma unroll
    for (uint32_t idx = t; idx < 2 * RT / RPL; idx += 64 * kAlongWaves) {
        const uint32_t strip = idx / (RT / RPL), r = RPL * (idx - strip * (RT / RPL));
        const uint64_t gg = (uint64_t)tk * 2u + strip;
        if (gg < G && m0 + r < M) {
            const uint64_t slot = dense ? gg : (gg & 3u) + 32u * (gg >> 2);
            if constexpr (NARROW)
                store<1>(scale + slot * M + m0 + r, e8m0[strip * RT + r]);
            else
                store<1>(reinterpret_cast<uint32_t *>(scale + slot * M + m0 + r),
                         *reinterpret_cast<const uint32_t *>(e8m0 + strip * RT + r));
        }
    }
}

} // namespace mxq
