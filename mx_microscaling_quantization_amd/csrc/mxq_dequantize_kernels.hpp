// mxq_dequantize_kernels.hpp -- gfx950 kernels of the MX dequantize.
//
// The inverse the consumer applies ("MX Microscaling: Quantize,
// Block-Scaling and E8M0", quantizeDataApplyingMxScales: the dequant side
// multiplies each decoded element by 2^(E8M0 - 127) with an fp32 ldexpf; the
// E8M0 byte is read back from the placed scale row and FP4 nibbles through
// the same container lane order).
//
// Same work split as the quantize: a thread owns an 8-row strip of NB
// blocks; it reads the strip's NB scale bytes once from the placed image row
// and 4*NB codes (FP8) or 2*NB bytes (FP4) per row, and writes 4*NB results
// per row. gfx950's v_cvt_scalef32_pk_{f32,bf16}_{fp8,bf8,fp4} compute
// decode(q) * scale for two codes at once and round once to the result type,
// which is exactly ldexpf (then nearest-even to bf16); the scale operand is
// the fp32 2^(E8M0 - 127): a normal number for E8M0 1..254 and the denormal
// 2^-127 for E8M0 0. E8M0 255 (2^128) is not an fp32 number, so such a block
// takes a rarely used branch that applies 2^127 and then doubles (exact:
// the scaled value has at most four significant bits).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq_quantize_kernels.hpp"

namespace mxq {

enum { kResF32 = 0, kResBF16 = 1 };

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 scale operand for an E8M0 byte in 0..254 (255 handled by the caller).
__device__ __forceinline__ float e8m0_scale_operand(uint32_t e)
{
    return __uint_as_float(e == 0 ? 0x00400000u : (e << 23));
}

// Nearest-even fp32 -> bf16 of a value (used only on the E8M0-255 branch).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t b = __float_as_uint(f);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u)
        return (b >> 16) | 0x40u;
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Two results from two codes. FP8: the codes are bytes 2*HI, 2*HI+1 of `w`.
// FP4: the codes are the low and high nibble of byte SEL of `w`.
// RES f32: r[0], r[1] are the two fp32 bit patterns; bf16: r[0] holds both.
template <int FMT, int RES, int SEL>
__device__ __forceinline__ void decode2(uint32_t w, float s, uint32_t *r)
{
    if constexpr (RES == kResF32) {
        f32x2_t v;
        if constexpr (FMT == kOutE4M3FN)
            v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, s, SEL != 0);
        else if constexpr (FMT == kOutE5M2)
            v = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(w, s, SEL != 0);
        else
            v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, SEL);
        r[0] = __float_as_uint(v.x);
        r[1] = __float_as_uint(v.y);
    } else {
        bf16x2_t v;
        if constexpr (FMT == kOutE4M3FN)
            v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, s, SEL != 0);
        else if constexpr (FMT == kOutE5M2)
            v = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, s, SEL != 0);
        else
            v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, SEL);
        r[0] = __builtin_bit_cast(uint32_t, v);
    }
}

// Decode the four codes of one block into four results (element order
// e0..e3). `w` holds the block's codes: FP8 -- the whole u32 lane (e_k in
// byte k); FP4 -- the dword holding the block's 16-bit container at byte
// offset 2*HALF (byte 2*HALF+1 = e0 | e1 << 4, byte 2*HALF = e2 | e3 << 4).
// out: f32 -> 4 words; bf16 -> 2 words.
template <int FMT, int RES, int HALF>
__device__ __forceinline__ void decode_block(uint32_t w, float s, uint32_t *out)
{
    constexpr int step = RES == kResF32 ? 2 : 1;
    if constexpr (FMT == kOutE2M1) {
        decode2<FMT, RES, 2 * HALF + 1>(w, s, out);      // e0, e1
        decode2<FMT, RES, 2 * HALF>(w, s, out + step);   // e2, e3
    } else {
        decode2<FMT, RES, 0>(w, s, out);                 // bytes 0, 1
        decode2<FMT, RES, 1>(w, s, out + step);          // bytes 2, 3
    }
}

// The E8M0 = 255 block: decode with 2^127, then double, then round.
template <int FMT, int RES, int HALF>
__device__ __forceinline__ void decode_block_e255(uint32_t w, uint32_t *out)
{
    uint32_t f[4];
    decode_block<FMT, kResF32, HALF>(w, __uint_as_float(254u << 23), f);
#pragma unroll
    for (int k = 0; k < 4; k++)
        f[k] = __float_as_uint(__uint_as_float(f[k]) * 2.0f);
    if constexpr (RES == kResF32) {
#pragma unroll
        for (int k = 0; k < 4; k++)
            out[k] = f[k];
    } else {
        out[0] = f32_to_bf16_bits(__uint_as_float(f[0])) | (f32_to_bf16_bits(__uint_as_float(f[1])) << 16);
        out[1] = f32_to_bf16_bits(__uint_as_float(f[2])) | (f32_to_bf16_bits(__uint_as_float(f[3])) << 16);
    }
}

// The dequantize kernel. Grid as the quantize (GPT = 1): one workgroup per
// (row group, run of strips); XCD != 0 renumbers workgroups as the quantize
// does, so each XCD walks one contiguous range of tiles.
//   data    FP8: P*F bytes; FP4: P*F/2 bytes
//   scale   the P x F/4 scale image (only the placed rows are read), or with
//           dense = 1 the [P/8, F/4] scale array
//   out     P x F results, fp32 or bf16
//
// OWN != 0 (for result rows that are not a multiple of 128 bytes): a
// workgroup owns blockDim.x - dq_own_extra(lane bytes) strips and also
// decodes the next ones, and in every row it writes exactly the 128-byte
// lines that start inside its own strips, so that no line is written in part
// by two workgroups (except the one a row boundary splits). 128 bytes of
// extra strips reach past any line boundary.
constexpr uint32_t dq_own_extra(uint32_t lane_bytes) { return 128u / lane_bytes; }

template <int FMT, int RES, int NB, int NT, int XCD = 0, int OWN = 0>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t *__restrict__ data,
                                                         const uint8_t *__restrict__ scale,
                                                         void *__restrict__ out, uint64_t F,
                                                         uint32_t nstrips, uint32_t tiles_per_band,
                                                         uint32_t dense)
{
    static_assert(NB == 1 || NB == 2, "a strip is 1 or 2 blocks");
    constexpr int LD = NT & 1, ST = (NT >> 1) & 1;
    constexpr int RES_BYTES = RES == kResF32 ? 4 : 2;
    constexpr uint32_t LANE_BYTES = 4 * NB * RES_BYTES;
    static_assert(!OWN || LANE_BYTES == 16 || LANE_BYTES == 8, "line ownership: 8 or 16 result bytes per row");
    const uint32_t tile = tile_index<XCD>();
    const uint32_t group = tile / tiles_per_band;
    const uint32_t run = tile - group * tiles_per_band;
    const uint32_t owned = OWN ? blockDim.x - dq_own_extra(LANE_BYTES) : blockDim.x;
    const uint32_t strip = run * owned + threadIdx.x;
    if (strip >= nstrips)
        return;

    // the strip's E8M0 bytes, from logical row `group`'s placed image row
    // (or its row of the dense array)
    const uint64_t slot = dense ? (uint64_t)group : (uint64_t)(group & 3u) + 32u * (uint64_t)(group >> 2);
    const uint8_t *srow = scale + slot * (F / 4) + (uint64_t)strip * NB;
    uint32_t e[NB];
    if constexpr (NB == 2) {
        const uint32_t two = load<LD>(reinterpret_cast<const uint16_t *>(srow));
        e[0] = two & 0xFFu;
        e[1] = two >> 8;
    } else {
        e[0] = load<LD>(srow);
    }
    float s[NB];
    bool any255 = false;
#pragma unroll
    for (int b = 0; b < NB; b++) {
        any255 |= e[b] == 255u;
        s[b] = e8m0_scale_operand(e[b] & 0xFFu);
    }

    // codes of all 8 rows first, then convert and store row by row
    uint32_t c[8][NB];
    const uint64_t row0 = (uint64_t)group * 8u;

    // With OWN, this thread stores the rows whose 16 bytes lie in the lines
    // from the first one starting at or after the run's first byte to the
    // first one starting at or after the next run's (the row's own ends at
    // either side); both neighbours place each boundary at the same address.
    // Each row is a buffer over that row (row pitch < 2^31 bytes, checked on
    // the host), and a row this thread does not own gets an offset past the
    // buffer's end, which the hardware drops: no branch. The offsets are
    // fixed here, before the loads, in registers of their own: computed
    // between the stores, they took the registers of the previous store's
    // data and made each store wait for the one before.
    __amdgpu_buffer_rsrc_t own_rs[8];
    uint32_t own_off[8];
    if constexpr (OWN) {
        const uint32_t rowbytes = (uint32_t)(F * RES_BYTES);
        const uint32_t c0 = LANE_BYTES * owned * run, c1 = c0 + LANE_BYTES * owned;
        const uint32_t c = LANE_BYTES * strip;
#pragma unroll
        for (int r = 0; r < 8; r++) {
            uint8_t *rowp = reinterpret_cast<uint8_t *>(out) + (row0 + r) * (uint64_t)rowbytes;
            const uint32_t mis = (uint32_t)(uintptr_t)rowp & 127u; // row start within its line
            const uint32_t lo = run == 0 ? 0u : ((mis + c0 + 127u) & ~127u) - mis;
            const uint32_t hi = run + 1 == tiles_per_band ? rowbytes : ((mis + c1 + 127u) & ~127u) - mis;
            own_rs[r] = __builtin_amdgcn_make_buffer_rsrc(rowp, (short)0, (int)rowbytes, kBufferFlags);
            own_off[r] = (c >= lo && c < hi) ? c : kDropOffset;
            asm volatile("" : "+v"(own_off[r]));
        }
    }
    // The 8 destinations, each its own address: a single pointer stepped
    // between the stores shared registers with the first store's data, and
    // a store blocked on write backpressure then held up the rest of the
    // wave (1.07 G elements e2m1 -> f32: 790 us against 719 us).
    uint8_t *dst[8];
#pragma unroll
    for (int r = 0; r < 8; r++)
        dst[r] = reinterpret_cast<uint8_t *>(out) + ((row0 + r) * F + (uint64_t)strip * (4 * NB)) * RES_BYTES;
#pragma unroll
    for (int r = 0; r < 8; r++) {
        const uint64_t row = row0 + r;
        if constexpr (FMT == kOutE2M1) {
            const uint8_t *p = data + (row * F) / 2 + (uint64_t)strip * (2 * NB);
            if constexpr (NB == 2)
                c[r][0] = load<LD>(reinterpret_cast<const uint32_t *>(p));
            else
                c[r][0] = load<LD>(reinterpret_cast<const uint16_t *>(p));
        } else {
            const uint8_t *p = data + row * F + (uint64_t)strip * (4 * NB);
            if constexpr (NB == 2) {
                u32x2_t v = load<LD>(reinterpret_cast<const u32x2_t *>(p));
                c[r][0] = v.x;
                c[r][1] = v.y;
            } else {
                c[r][0] = load<LD>(reinterpret_cast<const uint32_t *>(p));
            }
        }
    }

    // Decode all 8 rows, then patch E8M0-255 blocks, then store: with the
    // rare branch outside the row loop the 8 stores issue back to back once
    // the loads have landed (decoding and storing row by row, each store
    // waited on the next row's load: 1.07 G elements e2m1 -> f32 at a cap of
    // 10 waves, 881 us against 743 us).
    uint32_t res[8][NB * RES_BYTES]; // per row: 4*NB results of RES_BYTES each, in words
#pragma unroll
    for (int r = 0; r < 8; r++)
#pragma unroll
        for (int b = 0; b < NB; b++) {
            const uint32_t w = FMT == kOutE2M1 ? c[r][0] : c[r][b];
            if (b == 0)
                decode_block<FMT, RES, 0>(w, s[b], res[r] + b * RES_BYTES);
            else
                decode_block<FMT, RES, 1>(w, s[b], res[r] + b * RES_BYTES);
        }
    if (any255) {
#pragma unroll
        for (int r = 0; r < 8; r++)
#pragma unroll
            for (int b = 0; b < NB; b++) {
                if (e[b] != 255u)
                    continue;
                const uint32_t w = FMT == kOutE2M1 ? c[r][0] : c[r][b];
                if (b == 0)
                    decode_block_e255<FMT, RES, 0>(w, res[r] + b * RES_BYTES);
                else
                    decode_block_e255<FMT, RES, 1>(w, res[r] + b * RES_BYTES);
            }
    }
    if constexpr (OWN) {
#pragma unroll
        for (int r = 0; r < 8; r++) {
            if constexpr (LANE_BYTES == 16) {
                u32x4_t v = {res[r][0], res[r][1], res[r][2], res[r][3]};
                __builtin_amdgcn_raw_buffer_store_b128(v, own_rs[r], (int)own_off[r], 0, ST ? kBufferNT : 0);
            } else {
                u32x2_t v = {res[r][0], res[r][1]};
                __builtin_amdgcn_raw_buffer_store_b64(v, own_rs[r], (int)own_off[r], 0, ST ? kBufferNT : 0);
            }
        }
        return;
    }
#pragma unroll
    for (int r = 0; r < 8; r++) {
        if constexpr (NB * RES_BYTES == 8) { // 32 bytes: fp32, two blocks
            u32x4_t lo = {res[r][0], res[r][1], res[r][2], res[r][3]};
            u32x4_t hi = {res[r][4], res[r][5], res[r][6], res[r][7]};
            store<ST>(reinterpret_cast<u32x4_t *>(dst[r]), lo);
            store<ST>(reinterpret_cast<u32x4_t *>(dst[r]) + 1, hi);
        } else {
            store_bytes<4 * NB * RES_BYTES, ST>(dst[r], res[r]);
        }
    }
}

} // namespace mxq
