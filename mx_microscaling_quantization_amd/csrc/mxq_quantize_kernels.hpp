// mxq_quantize_kernels.hpp -- gfx950 kernels of the MX quantize.
//
// One kernel pass per call: every byte of the input is read once from HBM,
// every output byte is written once, nothing intermediate goes to memory.
//
// Work split. A thread owns a column strip of one row group: 8 rows x 4*NB
// columns, i.e. NB whole 8x4 blocks (NB = 2 when F % 8 == 0, else 1). It
// issues one 16-byte (NB = 2) or 8-byte (NB = 1) load per row, so a wave's
// load of one row is 1 KiB (or 512 B) of contiguous memory. The block
// maximum is then a reduction inside the thread's own registers -- no
// cross-lane traffic, no LDS. A workgroup (one wave) covers 64 consecutive
// strips of one row group. Loads and stores carry the non-temporal hint:
// the data streams through once.
//
// Arithmetic ("MX Microscaling: Quantize, Block-Scaling and E8M0"):
//  * the largest biased exponent of the fp32-widened block equals the
//    exponent of the widened largest magnitude, because widening is
//    monotone in |x|; so the kernel takes a packed 16-bit max over the
//    magnitude bits (v_pk_max_u16) and widens only that one value
//    (findMaxExponentPerInputBlock);
//  * E8M0 = max(1, m - bias) (generateMxScales, both clamps at once), with
//    bias = EMAX, or EMAX - 1 in the alternative mode;
//  * prescale + round + pack run on gfx950's scaled conversions
//    (v_cvt_scalef32_pk_{fp8,bf8,fp4}_{bf16,f16}), which compute
//    RNE(x / scale) from the 16-bit inputs directly. With scale =
//    2^(E8M0 - 127) that is exactly RNE(x * 2^(127 - E8M0))
//    (quantizeDataApplyingMxScales followed by the narrow): the division by
//    a power of two is exact and the product is rounded once, as in the
//    page's fp32 multiply (whose own rounding only touches values far below
//    every format's smallest subnormal);
//  * these conversions do not saturate FP8/BF8: an overflow gives the NaN
//    code (e4m3fn, 0x7F) or the Inf code (e5m2, 0x7C). A SWAR pass moves
//    those bytes one code down, to the largest finite code;
//  * NaN inputs: the conversions give a NaN code (FP8) or +-6 (FP4), while
//    the quantizer's rule is a zero with the NaN's sign. A NaN can only sit
//    in a block whose maximum magnitude pattern is above the Inf pattern, so
//    a rarely taken per-thread branch rewrites exactly those codes;
//  * E8M0 254 (only FP4 in the alternative mode, for a block holding Inf or
//    NaN) makes the page's multiplier +0: every element of such a block is a
//    zero of its own sign. The same branch writes those codes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

enum { kInBF16 = 0, kInF16 = 1 };
enum { kOutE4M3FN = 0, kOutE5M2 = 1, kOutE2M1 = 2 };

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// Magnitude pattern of +Inf in the input type; anything above it is a NaN.
template <int IN> struct InfBits;
template <> struct InfBits<kInBF16> { static constexpr uint32_t value = 0x7F80u; };
template <> struct InfBits<kInF16> { static constexpr uint32_t value = 0x7C00u; };

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b)
{
    u16x2_t x = __builtin_bit_cast(u16x2_t, a);
    u16x2_t y = __builtin_bit_cast(u16x2_t, b);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}

// Biased fp32 exponent field of the widened value whose 16-bit magnitude
// pattern is `mag` (sign already cleared).
template <int IN> __device__ __forceinline__ uint32_t widened_exponent(uint32_t mag)
{
    if constexpr (IN == kInBF16) {
        return mag >> 7; // bf16 keeps the fp32 exponent field in bits 14..7
    } else {
        // exact f16 -> f32 (f16 subnormals become fp32 normals)
        float f = (float)__builtin_bit_cast(_Float16, (uint16_t)mag);
        return (__float_as_uint(f) >> 23) & 0xFFu;
    }
}

// E8M0 of one block given the magnitude max over its 32 elements and the
// EMAX bias (the format's EMAX, or EMAX - 1 in the alternative mode).
template <int IN> __device__ __forceinline__ uint32_t block_e8m0(uint32_t mag, int emax_bias)
{
    int v = (int)widened_exponent<IN>(mag) - emax_bias;
    return (uint32_t)(v < 1 ? 1 : v);
}

// The conversion's scale operand for an E8M0 byte: the fp32 2^(e - 127).
__device__ __forceinline__ float e8m0_to_scale(uint32_t e) { return __uint_as_float(e << 23); }

// Four FP8 codes (one u32 lane) from two input dwords holding elements
// (0,1) and (2,3), saturated.
template <int IN, int OUT> __device__ __forceinline__ uint32_t fp8x4(uint32_t p01, uint32_t p23, float s)
{
    i16x2_t r = {0, 0};
    if constexpr (IN == kInBF16) {
        bf16x2_t a = __builtin_bit_cast(bf16x2_t, p01), b = __builtin_bit_cast(bf16x2_t, p23);
        if constexpr (OUT == kOutE4M3FN) {
            r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, a, s, false);
            r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, b, s, true);
        } else {
            r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(r, a, s, false);
            r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(r, b, s, true);
        }
    } else {
        f16x2_t a = __builtin_bit_cast(f16x2_t, p01), b = __builtin_bit_cast(f16x2_t, p23);
        if constexpr (OUT == kOutE4M3FN) {
            r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(r, a, s, false);
            r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(r, b, s, true);
        } else {
            r = __builtin_amdgcn_cvt_scalef32_pk_bf8_f16(r, a, s, false);
            r = __builtin_amdgcn_cvt_scalef32_pk_bf8_f16(r, b, s, true);
        }
    }
    uint32_t w = __builtin_bit_cast(uint32_t, r);
    // Overflow codes: e4m3fn 0x7F (NaN) and e5m2 0x7C (Inf), either sign.
    // Adding 1 (resp. 4) to the low 7 bits of a byte carries into bit 7 for
    // exactly those codes (and e5m2's NaN codes, which only a NaN input makes
    // and the NaN pass rewrites); subtracting that carry gives 0x7E / 0x7B.
    constexpr uint32_t bump = OUT == kOutE4M3FN ? 0x01010101u : 0x04040404u;
    uint32_t t = ((w & 0x7F7F7F7Fu) + bump) & 0x80808080u;
    return w - (t >> 7);
}

// One FP4 container (16 bits) from elements (0,1) in p01 and (2,3) in p23,
// placed as byte 0 = e2 | e3 << 4, byte 1 = e0 | e1 << 4, and written into
// bytes 2*HALF, 2*HALF+1 of `acc`.
template <int IN, int HALF>
__device__ __forceinline__ uint32_t fp4_container(uint32_t acc, uint32_t p01, uint32_t p23, float s)
{
    if constexpr (IN == kInBF16) {
        bf16x2_t a = __builtin_bit_cast(bf16x2_t, p01), b = __builtin_bit_cast(bf16x2_t, p23);
        acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(acc, b, s, 2 * HALF);
        acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(acc, a, s, 2 * HALF + 1);
    } else {
        f16x2_t a = __builtin_bit_cast(f16x2_t, p01), b = __builtin_bit_cast(f16x2_t, p23);
        acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(acc, b, s, 2 * HALF);
        acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(acc, a, s, 2 * HALF + 1);
    }
    return acc;
}

// Bit offset, inside the u32 holding a row's FP4 output for one strip, of
// element k (0..7) of the strip: container k/4, then {8, 12, 0, 4}.
__device__ __forceinline__ uint32_t fp4_bit_offset(uint32_t k)
{
    return 16u * (k >> 2) + ((0x40C8u >> (4u * (k & 3u))) & 0xFu);
}

// Rewrite the codes that the conversions cannot give: a NaN element, and
// every element of a block with E8M0 254, becomes a zero of its own sign.
// `w` holds the input dwords of one row of a strip (2*NB of them, element k
// in the 16-bit half k&1 of w[k/2]); `e` the strip's E8M0 bytes; `out` the
// row's output codes: FP8 byte k of the strip is byte k&3 of out[k/4]; FP4
// element k is in out[k/8] at fp4_bit_offset(k mod 8).
template <int IN, int OUT, int NB>
__device__ __forceinline__ void fix_special_codes(const uint32_t *w, const uint32_t *e, uint32_t *out)
{
#pragma unroll
    for (uint32_t k = 0; k < 4 * NB; k++) {
        uint32_t h = (w[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
        if ((h & 0x7FFFu) <= InfBits<IN>::value && e[k >> 2] != 254u)
            continue;
        uint32_t sign = h >> 15;
        if constexpr (OUT == kOutE2M1) {
            uint32_t sh = fp4_bit_offset(k & 7);
            out[k >> 3] = (out[k >> 3] & ~(0xFu << sh)) | ((sign << 3) << sh);
        } else {
            uint32_t sh = 8 * (k & 3);
            out[k >> 2] = (out[k >> 2] & ~(0xFFu << sh)) | ((sign << 7) << sh);
        }
    }
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Loads and stores with an optional non-temporal hint (streaming data that
// no later access of this kernel touches again).
template <int NT, typename T> __device__ __forceinline__ T load(const T *p)
{
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}
template <int NT, typename T> __device__ __forceinline__ void store(T *p, T v)
{
    if constexpr (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// One row of a strip: 4*NB input elements = 2*NB dwords, fetched as one
// 8-byte (NB = 1) or NB/2 16-byte loads.
template <int NB, int NT> __device__ __forceinline__ void load_row(const uint16_t *row, uint32_t strip, uint32_t *w)
{
    if constexpr (NB == 1) {
        u32x2_t v = load<NT>(reinterpret_cast<const u32x2_t *>(row) + strip);
        w[0] = v.x;
        w[1] = v.y;
    } else {
        const u32x4_t *p = reinterpret_cast<const u32x4_t *>(row) + (uint64_t)strip * (NB / 2);
#pragma unroll
        for (int i = 0; i < NB / 2; i++) {
            u32x4_t v = load<NT>(p + i);
            w[4 * i + 0] = v.x;
            w[4 * i + 1] = v.y;
            w[4 * i + 2] = v.z;
            w[4 * i + 3] = v.w;
        }
    }
}

// Store NBYTES (2, 4, 8 or 16) bytes held in out[] to dst (NBYTES-aligned).
template <int NBYTES, int NT> __device__ __forceinline__ void store_bytes(uint8_t *dst, const uint32_t *out)
{
    if constexpr (NBYTES == 1) {
        store<NT>(dst, (uint8_t)out[0]);
    } else if constexpr (NBYTES == 2) {
        store<NT>(reinterpret_cast<uint16_t *>(dst), (uint16_t)out[0]);
    } else if constexpr (NBYTES == 4) {
        store<NT>(reinterpret_cast<uint32_t *>(dst), out[0]);
    } else if constexpr (NBYTES == 8) {
        u32x2_t v = {out[0], out[1]};
        store<NT>(reinterpret_cast<u32x2_t *>(dst), v);
    } else {
        u32x4_t v = {out[0], out[1], out[2], out[3]};
        store<NT>(reinterpret_cast<u32x4_t *>(dst), v);
    }
}

template <int XCD> __device__ __forceinline__ uint32_t tile_index()
{
    if constexpr (XCD == 0) {
        return blockIdx.x;
    } else {
        // workgroup i runs on chiplet i mod XCD; give chiplet c the tiles
        // [c*q, (c+1)*q) of the first XCD*q, and leave the tail in place
        const uint32_t q = gridDim.x / XCD;
        const uint32_t i = blockIdx.x;
        return i < q * XCD ? (i % XCD) * q + i / XCD : i;
    }
}

// The quantize kernel.
//
// Grid: one workgroup per (band, run of up to blockDim.x strips), where a
// band is GPT consecutive row groups and `tiles_per_band` runs cover a band.
// A strip is NB blocks side by side (4*NB columns, F % (4*NB) == 0). Each
// thread quantizes the same strip in every row group of its band; all 8*GPT
// rows are loaded before any arithmetic. NT bit 0 marks the loads
// non-temporal, bit 1 the stores. XCD != 0 renumbers workgroups so that each
// of the XCD chiplets (which receive workgroups round-robin) walks one
// contiguous range of tiles.
//   F          columns (pitch of the input and of FP8 data)
//   nstrips    F / (4*NB)
//   ngroups    P / 8
//   emax_bias  EMAX of the output format, or EMAX - 1 (alternative mode)
//   dense      0: scale row of group i is (i mod 4) + 32*floor(i/4) of the
//              P-row image; 1: row i of a dense [P/8, F/4] array
//
// OWN != 0 (FP8 codes, NB = 2; for row pitches that are not a multiple of
// 128 bytes): each workgroup owns blockDim.x - kOwnExtra strips and also
// computes the next kOwnExtra (the next workgroup's first ones), and in
// every row it writes exactly the 128-byte lines that start inside its own
// strips -- so no line is written in part by two workgroups (except the one
// a row boundary splits). 16 strips of 8 bytes reach past any line boundary
// within 128 bytes.
constexpr uint32_t kOwnExtra = 16;
// Raw untyped buffer (32-bit data format); the non-temporal cache-policy
// bit of buffer stores; an offset past any buffer used with it (stores at
// such an offset are dropped by the buffer's range check).
constexpr uint32_t kBufferFlags = 0x00020000u;
constexpr int kBufferNT = 2;
constexpr uint32_t kDropOffset = 0x80000000u;

template <int IN, int OUT, int NB, int GPT, int NT, int XCD = 0, int OWN = 0>
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t *__restrict__ in,
                                                       uint8_t *__restrict__ data,
                                                       uint8_t *__restrict__ scale,
                                                       uint64_t F, uint32_t nstrips,
                                                       uint32_t tiles_per_band, uint32_t ngroups,
                                                       int emax_bias, uint32_t dense)
{
    static_assert(NB == 1 || NB == 2 || NB == 4, "a strip is 1, 2 or 4 blocks");
    static_assert(!OWN || (NB == 2 && GPT == 1 && OUT != kOutE2M1), "line ownership: FP8, two-block strips");
    constexpr int LD = NT & 1, ST = (NT >> 1) & 1;
    const uint32_t tile = tile_index<XCD>();
    const uint32_t band = tile / tiles_per_band;
    const uint32_t run = tile - band * tiles_per_band;
    const uint32_t owned = OWN ? blockDim.x - kOwnExtra : blockDim.x;
    const uint32_t strip = run * owned + threadIdx.x;
    if (strip >= nstrips)
        return;

    const uint32_t g0 = band * GPT;

    // With OWN, this thread stores the rows whose 8 bytes lie in the lines
    // from the first one starting at or after the run's first byte to the
    // first one starting at or after the next run's (the row's own ends at
    // either side); both neighbours place each boundary at the same address.
    // Each row is a buffer over that row (row pitch < 2^31 bytes, checked on
    // the host), and a row this thread does not own gets an offset past the
    // buffer's end, which the hardware drops: no branch around the stores.
    // The offsets are fixed here, before the loads, in registers of their
    // own: computed between the stores, they took the registers of the
    // previous store's data and made each store wait for the one before.
    __amdgpu_buffer_rsrc_t own_rs[8];
    uint32_t own_off[8];
    if constexpr (OWN) {
        const uint32_t c0 = 8u * owned * run, c1 = c0 + 8u * owned, c = 8u * strip;
#pragma unroll
        for (int r = 0; r < 8; r++) {
            uint8_t *rowp = data + ((uint64_t)g0 * 8u + r) * F;
            const uint32_t mis = (uint32_t)(uintptr_t)rowp & 127u; // row start within its line
            const uint32_t lo = run == 0 ? 0u : ((mis + c0 + 127u) & ~127u) - mis;
            const uint32_t hi = run + 1 == tiles_per_band ? (uint32_t)F : ((mis + c1 + 127u) & ~127u) - mis;
            own_rs[r] = __builtin_amdgcn_make_buffer_rsrc(rowp, (short)0, (int)F, kBufferFlags);
            own_off[r] = (c >= lo && c < hi) ? c : kDropOffset;
            asm volatile("" : "+v"(own_off[r]));
        }
    }

    uint32_t w[GPT][8][2 * NB];
#pragma unroll
    for (int j = 0; j < GPT; j++) {
        if (GPT > 1 && g0 + j >= ngroups)
            break;
        const uint16_t *rows = in + (uint64_t)(g0 + j) * 8u * F;
#pragma unroll
        for (int r = 0; r < 8; r++)
            load_row<NB, LD>(rows + r * F, strip, w[j][r]);
    }

#pragma unroll
    for (int j = 0; j < GPT; j++) {
        const uint32_t group = g0 + j;
        if (GPT > 1 && group >= ngroups)
            break;
        const uint64_t row0 = (uint64_t)group * 8u;

        // Block maxima of the magnitude patterns, two 16-bit lanes at a time.
        uint32_t e[NB];
        float s[NB];
        bool special = false;
#pragma unroll
        for (int b = 0; b < NB; b++) {
            uint32_t m = 0;
#pragma unroll
            for (int r = 0; r < 8; r++) {
                m = pk_max_u16(m, w[j][r][2 * b] & 0x7FFF7FFFu);
                m = pk_max_u16(m, w[j][r][2 * b + 1] & 0x7FFF7FFFu);
            }
            const uint32_t mag = max(m & 0xFFFFu, m >> 16);
            e[b] = block_e8m0<IN>(mag, emax_bias);
            s[b] = e8m0_to_scale(e[b]);
            special |= mag > InfBits<IN>::value || e[b] == 254u;
        }

        uint32_t own_codes[8][NB]; // with OWN: every row's codes, stored after the loop
#pragma unroll
        for (int r = 0; r < 8; r++) {
            const uint64_t row = row0 + r;
            if constexpr (OUT == kOutE2M1) {
                // two blocks (two containers) per output dword
                uint32_t out[(NB + 1) / 2];
#pragma unroll
                for (int h = 0; h < (NB + 1) / 2; h++) {
                    out[h] = fp4_container<IN, 0>(0u, w[j][r][4 * h], w[j][r][4 * h + 1], s[2 * h]);
                    if constexpr (NB > 1)
                        out[h] = fp4_container<IN, 1>(out[h], w[j][r][4 * h + 2], w[j][r][4 * h + 3], s[2 * h + 1]);
                }
                if (special)
                    fix_special_codes<IN, OUT, NB>(w[j][r], e, out);
                store_bytes<2 * NB, ST>(data + (row * F) / 2 + (uint64_t)strip * (2 * NB), out);
            } else {
                uint32_t out[NB];
#pragma unroll
                for (int b = 0; b < NB; b++)
                    out[b] = fp8x4<IN, OUT>(w[j][r][2 * b], w[j][r][2 * b + 1], s[b]);
                if (special)
                    fix_special_codes<IN, OUT, NB>(w[j][r], e, out);
                if constexpr (OWN) {
#pragma unroll
                    for (int b = 0; b < NB; b++)
                        own_codes[r][b] = out[b];
                } else {
                    store_bytes<4 * NB, ST>(data + row * F + (uint64_t)strip * (4 * NB), out);
                }
            }
        }
        if constexpr (OWN) {
#pragma unroll
            for (int r = 0; r < 8; r++) {
                u32x2_t v = {own_codes[r][0], own_codes[r][1]};
                __builtin_amdgcn_raw_buffer_store_b64(v, own_rs[r], (int)own_off[r], 0, ST ? kBufferNT : 0);
            }
        }

        // Scale placement: logical row `group` goes to image row
        // (group mod 4) + 32 * floor(group / 4), or to row `group` of the
        // dense array.
        if (OWN && threadIdx.x >= owned)
            continue; // the next run's strips: their scales are that run's
        const uint64_t slot = dense ? (uint64_t)group : (uint64_t)(group & 3u) + 32u * (uint64_t)(group >> 2);
        uint32_t packed[1] = {0};
#pragma unroll
        for (int b = 0; b < NB; b++)
            packed[0] |= e[b] << (8 * b);
        store_bytes<NB, ST>(scale + slot * (F / 4) + (uint64_t)strip * NB, packed);
    }
}

} // namespace mxq
