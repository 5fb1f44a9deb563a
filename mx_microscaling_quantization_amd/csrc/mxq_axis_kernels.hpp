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
// reach a thread and where its codes go. One HBM pass, non-temporal hints.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
//   nstrips   N / NB;  tiles_per_band  ceil(nstrips / 64)
template <int IN, int OUT, int NB>
__global__ __launch_bounds__(64) void quantize_down_kernel(const uint16_t *__restrict__ in,
                                                           uint8_t *__restrict__ data,
                                                           uint8_t *__restrict__ scale, uint64_t N,
                                                           uint32_t nstrips, uint32_t tiles_per_band,
                                                           int emax_bias, uint32_t dense)
{
    static_assert(NB == 1 || NB == 2 || NB == 4, "1, 2 or 4 columns per thread");
    constexpr int NW = (NB + 1) / 2;   // loaded dwords per row
    const uint32_t band = blockIdx.x / tiles_per_band;
    const uint32_t strip = (blockIdx.x - band * tiles_per_band) * 64u + threadIdx.x;
    if (strip >= nstrips)
        return;
    const uint64_t n0 = (uint64_t)strip * NB;

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

    const uint64_t F = 4 * N;
#pragma unroll
    for (int pr = 0; pr < 8; pr++) {
        const uint64_t p = (uint64_t)band * 8u + pr;
        // the view row's input dwords, laid out as the plain quantize holds a
        // strip row: block b's elements j = 0..3 in w[2b] (j = 0, 1), w[2b+1]
        uint32_t w[2 * NB];
#pragma unroll
        for (int b = 0; b < NB; b++) {
            const int h = b / 2, q = b & 1;
            w[2 * b] = half16(v[4 * pr][h], q) | half16(v[4 * pr + 1][h], q) << 16;
            w[2 * b + 1] = half16(v[4 * pr + 2][h], q) | half16(v[4 * pr + 3][h], q) << 16;
        }
        if constexpr (OUT == kOutE2M1) {
            uint32_t out[NW];
#pragma unroll
            for (int h = 0; h < NW; h++) {
                out[h] = fp4_container<IN, 0>(0u, w[4 * h], w[4 * h + 1], s[2 * h]);
                if constexpr (NB > 1)
                    out[h] = fp4_container<IN, 1>(out[h], w[4 * h + 2], w[4 * h + 3], s[2 * h + 1]);
            }
            if (special)
                fix_special_codes<IN, OUT, NB>(w, e, out);
            store_bytes<2 * NB, 1>(data + (p * F) / 2 + 2 * n0, out);
        } else {
            uint32_t out[NB];
#pragma unroll
            for (int b = 0; b < NB; b++)
                out[b] = fp8x4<IN, OUT>(w[2 * b], w[2 * b + 1], s[b]);
            if (special)
                fix_special_codes<IN, OUT, NB>(w, e, out);
            store_bytes<4 * NB, 1>(data + p * F + 4 * n0, out);
        }
    }

    const uint64_t slot = dense ? (uint64_t)band : (uint64_t)(band & 3u) + 32u * (uint64_t)(band >> 2);
    uint32_t packed[1] = {0};
#pragma unroll
    for (int b = 0; b < NB; b++)
        packed[0] |= e[b] << (8 * b);
    store_bytes<NB, 1>(scale + slot * N + n0, packed);
}

// Blocks along the rows (dim -1) of X [M][K] (row pitch K).
//
// A block is 32 contiguous elements of one row, but its codes go to 8 view
// rows at column m, so a wave must cover 64 consecutive rows to store
// contiguously -- and 64 rows read one block each would touch 64 cache lines
// per load. So a 256-thread workgroup stages a tile of 64 rows x 256
// elements (8 blocks) in LDS with coalesced loads (a wave's load is two
// 512-byte row segments), then thread (row r = t mod 64, blocks 2w and
// 2w + 1 for wave w) quantizes from LDS. The LDS row pitch is 528 bytes: the
// 16-byte skew per row puts the 16 rows that 16 lanes read in distinct
// banks. Block g's view rows are p = 8g + pr, and row m's container in view
// row p is elements 4p .. 4p + 3 of the block, i.e. dwords 2pr, 2pr + 1 of
// its 16; it goes to p * 4M + 4m (FP8) / p * 2M + 2m (FP4), so a wave
// writes 256 (128) contiguous bytes per view row. The E8M0 byte goes to
// the placed (or dense) scale row of g at column m.
//   tiles_m   ceil(M / 64); the grid is tiles_m x ceil(K / 256)
constexpr uint32_t kAlongRows = 64;
constexpr uint32_t kAlongTileK = 256;
constexpr uint32_t kAlongPitch = 2 * kAlongTileK + 16;

template <int IN, int OUT>
__global__ __launch_bounds__(256) void quantize_along_kernel(const uint16_t *__restrict__ in,
                                                             uint8_t *__restrict__ data,
                                                             uint8_t *__restrict__ scale, uint64_t M,
                                                             uint64_t K, uint32_t tiles_m, int emax_bias,
                                                             uint32_t dense)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[kAlongRows * kAlongPitch];
    const uint32_t tk = blockIdx.x / tiles_m;
    const uint64_t m0 = (uint64_t)(blockIdx.x - tk * tiles_m) * kAlongRows;
    const uint64_t k0 = (uint64_t)tk * kAlongTileK;
    const uint32_t nblk = (uint32_t)min((uint64_t)(kAlongTileK / 32), (K - k0) / 32);
    const uint32_t t = threadIdx.x;

    // 64 rows x 32 pieces of 16 bytes; piece q: row q / 32, piece q mod 32
#pragma unroll
    for (uint32_t i = 0; i < 8; i++) {
        const uint32_t q = t + 256u * i;
        const uint32_t r = q >> 5, c = q & 31u;
        if (m0 + r < M && c < 4u * nblk) {
            const u32x4_t v = load<1>(reinterpret_cast<const u32x4_t *>(in + (m0 + r) * K + k0 + 8u * c));
            *reinterpret_cast<u32x4_t *>(tile + r * kAlongPitch + 16u * c) = v;
        }
    }
    __syncthreads();

    const uint32_t r = t & (kAlongRows - 1);
    const uint64_t m = m0 + r;
    if (m >= M)
        return;
    const uint64_t F = 4 * M;
#pragma unroll
    for (uint32_t bb = 0; bb < 2; bb++) {
        const uint32_t b = 2u * (t >> 6) + bb;
        if (b >= nblk)
            break;
        uint32_t d[16];
#pragma unroll
        for (uint32_t q = 0; q < 4; q++) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t *>(tile + r * kAlongPitch + 64u * b + 16u * q);
            d[4 * q + 0] = v.x;
            d[4 * q + 1] = v.y;
            d[4 * q + 2] = v.z;
            d[4 * q + 3] = v.w;
        }
        uint32_t mm = 0;
#pragma unroll
        for (int k = 0; k < 16; k++)
            mm = pk_max_u16(mm, d[k] & 0x7FFF7FFFu);
        const uint32_t mag = max(mm & 0xFFFFu, mm >> 16);
        uint32_t e[1] = {block_e8m0<IN>(mag, emax_bias)};
        const float s = e8m0_to_scale(e[0]);
        const bool special = mag > InfBits<IN>::value || e[0] == 254u;
        const uint64_t g = k0 / 32 + b;
#pragma unroll
        for (int pr = 0; pr < 8; pr++) {
            const uint64_t p = g * 8u + pr;
            uint32_t w[2] = {d[2 * pr], d[2 * pr + 1]};
            uint32_t out[1];
            if constexpr (OUT == kOutE2M1)
                out[0] = fp4_container<IN, 0>(0u, w[0], w[1], s);
            else
                out[0] = fp8x4<IN, OUT>(w[0], w[1], s);
            if (special)
                fix_special_codes<IN, OUT, 1>(w, e, out);
            if constexpr (OUT == kOutE2M1)
                store_bytes<2, 1>(data + (p * F) / 2 + 2 * m, out);
            else
                store_bytes<4, 1>(data + p * F + 4 * m, out);
        }
        const uint64_t slot = dense ? g : (g & 3u) + 32u * (g >> 2);
        store_bytes<1, 1>(scale + slot * M + m, e);
    }
}

} // namespace mxq
