// mxq_matmul_kernels.hpp -- gfx950 block-scaled matmul of two MX operands.
//
// The consumer of the quantize ("MX-FP8 Microscaling Legalization",
// LegalizeScaledMatmul and the crosswalk: a 32-element group is 8
// partitions x 4 elements with one E8M0, and the engine unpacks each x4
// container into the contraction dimension). An operand quantized as
// [P, 4C] is the matrix X[k][c] with k = 4p + j (p the row, j the position
// in the x4 container) and c the container index; element value
// decode(q) * 2^(E8M0 - 127) with the E8M0 of row group k / 32. The kernel
// computes out[m][n] = sum_k L[k][m] * R[k][n] (K = 4P), fp32 accumulation.
//
// Tiling: a 512-thread workgroup computes a 256 x 256 tile of out; each of
// its 8 waves a 64 (M) x 128 (N) part as 2 x 4 MFMAs of 32 x 32. Two waves
// share each SIMD and run half a K step apart ("ping-pong"): while one
// issues its MFMAs, the other reads its next operands from LDS and issues
// its copies. Workgroups are renumbered so that the 32 CUs of one XCD (which
// receive every eighth workgroup) work on a compact block of tiles and share
// operand panels in their L2. Tails in M, N and K read as zeros, so every
// MFMA runs with all 64 lanes active.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq_quantize_kernels.hpp"

namespace mxq {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kMmTile = 256;        // output tile edge (M and N)
constexpr int kMmThreads = 512;
constexpr int kMmXcds = 8;
constexpr int kMmGroupRows = 4;     // tile rows walked together (L2 reuse)
constexpr uint32_t kMmBufferFlags = 0x00020000u;   // raw untyped buffer, 32-bit data format

// MFMA operand-format code of an element format (cbsz / blgp field).
template <int FMT> struct MfmaFmt;
template <> struct MfmaFmt<kOutE4M3FN> { static constexpr int value = 0; };
template <> struct MfmaFmt<kOutE5M2> { static constexpr int value = 1; };

// What the kernel does with its fp32 sums: store them, store them rounded
// to bf16, or quantize them (rounded to bf16) into MX data + E8M0 scales of
// format EPI - kEpiMx.
enum { kEpiF32 = 0, kEpiBF16 = 1, kEpiMx = 2 };

// fp32 -> bf16 bits, round to nearest even; a NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t mm_bf16_bits(float v)
{
    const uint32_t bits = __float_as_uint(v);
    const uint32_t nearest = (bits + 0x7FFFu + ((bits >> 16) & 1u)) >> 16;
    const uint32_t quiet = (bits >> 16) | 0x40u;
    return (bits & 0x7FFFFFFFu) > 0x7F800000u ? quiet : nearest;   // a select, no branch
}

// ----------------------------------------------------------------------------
// The kernel: v_mfma_scale_f32_32x32x64_f8f6f4, operands copied global ->
// LDS by the buffer unit itself (buffer_load_dwordx4 ... lds), no registers.
//
// MFMA mapping (measured on gfx950): lane l = i + 32 h supplies row i of A
// (column i of B); byte b of its 32 pairs with byte b of the same lane half
// of the other operand; scale block j (one E8M0) is bytes 16 j .. 16 j + 15 of
// both halves, and half h's scale byte covers block h (op_sel picks the byte
// of the scale register); result register r of lane l is
// D[8 (r >> 2) + 4 h + (r & 3)][i].
// One K step is 64 = 16 operand rows = 4 row quads = 2 row groups (MX
// blocks). LDS holds each operand row-major, as the copy lands it: row quad
// q at q * kMmQuadPitch, row 4 q + v of it at + 1024 v, container c at + 4 c.
// Lane (i, h) supplies rows 4 h .. 4 h + 3 (block 0) and 8 + 4 h .. 11 + 4 h
// (block 1) of its container. The containers are interleaved across
// sub-tiles so that one LDS read serves several: in A sub-tile a (of 2) lane
// i takes container wm + 2 i + a (one 8-byte read per row feeds both), in B
// sub-tile u (of 4) container wn + 4 i + u (one 16-byte read per row feeds
// all four); register moves then gather each sub-tile's 8 dwords. Hence
// result register r of lane (i, h) in sub-tile (a, u) is
// out[m0 + wm + 2 (8 (r >> 2) + 4 h + (r & 3)) + a][n0 + wn + 4 i + u]: a lane
// holds 4 adjacent columns of each row it has, and for each r >> 2 all 8 rows
// of one 8-row group.
//
// In a 64-lane buffer_load_dwordx4 ... lds, lane L's 16 bytes go to LDS base +
// 16 L: lane L fetches containers 4 L .. 4 L + 3 of one row, and one load
// copies a 256-container row. Wave (g, q) (group g = wave / 4) copies row
// quad q of operand g (A for g = 0, B for g = 1) per step, 4 loads, and
// waves with q < 2 one E8M0 row (K block q of the step) of that operand; the
// other waves issue the same load with an empty range into a spare LDS row,
// so that every wave has 5 loads per step and one wait count.
// kMmStages stages: the copies of step s + kMmStages - 1 are issued in a
// wave's memory phase of step s, into the stage of step s - 1, which every
// wave has finished reading by then.
// ----------------------------------------------------------------------------
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr uint32_t kMmStepRows = 16;                      // operand rows per K step (K = 64)
constexpr int kMmStages = 3;                               // (4 measured no faster)
constexpr uint32_t kMmQuadPitch = kMmTile * 16 + 128;    // one row quad of a tile, padded
constexpr uint32_t kMmTileBytes = 4 * kMmQuadPitch;
constexpr uint32_t kMmScaleBytes = 2 * kMmTile;           // 2 K blocks x 256 containers
constexpr uint32_t kMmStageBytes = 2 * kMmTileBytes + 2 * kMmScaleBytes;
constexpr uint32_t kMmSpareBytes = 256;                   // target of the empty scale loads
constexpr int kMmCopies = 5;                              // loads per wave per step

struct MmSource {
    const uint8_t *data;    // column c0 of operand row 0
    const uint8_t *scale;   // column c0 of scale row 0
    uint32_t pitch;         // 4 C bytes
    uint32_t C;             // containers
    uint32_t scale_cols;    // scale bytes left in a row from c0
    uint32_t col_bytes;     // 4 c0
};

__device__ __forceinline__ void mm_source(MmSource &s, const uint8_t *data, const uint8_t *scale, uint32_t C,
                                           uint32_t c0)
{
    s.pitch = 4u * C;
    s.data = data + 4ull * c0;
    s.scale = scale + c0;
    s.C = C;
    s.scale_cols = C - c0;
    s.col_bytes = 4u * c0;
}

// Row quad `quad` of K step `step` of one operand -> `tile` (LDS). The
// range of the buffer starts at column c0 of the step's first row and ends
// at the operand's last byte when the step reaches row P: rows past P read
// as zero; a step at or past row P gets an empty range and touches no
// memory. Columns past C read bytes of the next row (or zeros); they only
// reach results outside the output.
__device__ __forceinline__ void mm_copy_quad(const MmSource &s, uint8_t *tile, uint32_t P, uint32_t step,
                                              uint32_t quad, uint32_t lane)
{
    const bool in_range = step * kMmStepRows < P;
    const uint32_t rows_left = in_range ? min(P - step * kMmStepRows, kMmStepRows) : 0u;
    const uint32_t bytes = in_range ? rows_left * s.pitch - s.col_bytes : 0u;
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(s.data + (in_range ? (uint64_t)step * kMmStepRows * s.pitch : 0ull)), (short)0, (int)bytes,
        kMmBufferFlags);
    const uint32_t q0 = 4u * quad * s.pitch;
#pragma unroll
    for (uint32_t v = 0; v < 4; v++)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void_t *)(tile + kMmQuadPitch * quad + 1024u * v), 16,
                                                 16u * lane, q0 + v * s.pitch, 0, 0);
}

// E8M0 row of K block kb (256 containers from c0) -> `stile` (LDS); blocks
// past P / 8 read as zero (their data is zero too). A wave without a scale
// row (has == false) loads from an empty range into `spare` instead.
__device__ __forceinline__ void mm_copy_scale(const MmSource &s, uint8_t *stile, uint8_t *spare, bool has,
                                               uint32_t P, uint32_t kb, uint32_t dense, uint32_t lane)
{
    const bool ok = has && kb < P / 8;
    // uniform; said so, or the compiler builds the address in vector
    // registers and loops over its (single) value
    const uint32_t srow = __builtin_amdgcn_readfirstlane(!ok ? 0u : dense ? kb : (kb & 3u) + 32u * (kb >> 2));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(s.scale + (uint64_t)srow * s.C), (short)0, ok ? (int)s.scale_cols : 0, kMmBufferFlags);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)(has ? stile : spare), 4, 4u * lane, 0, 0, 0);
}

// One step's operand bytes of a lane as read from LDS: a[v] = row v's two A
// containers (v = 0..3: rows 4 h + v; 4..7: rows 8 + 4 h + v - 4), b[v] the
// four B containers of the same row, and the E8M0 bytes of its K block.
struct MmRaw {
    uint32_t a[8][2];
    uint32_t b[8][4];
    uint32_t as[2];
    uint32_t bs;        // byte u: B sub-tile u
};

// Dword reads, which the compiler combines into 8- and 16-byte reads. Read
// through a 16-byte vector type instead, they got a wait for every copy in
// flight (vmcnt(0)) in front of them; read as 32-bit integers they do not.
// No such wait is needed: the reads' stage was completed by the wait and
// barrier that closed the previous phase, and the copies in flight write
// other stages.
__device__ __forceinline__ void mm_read(const uint8_t *st, uint32_t a_off, uint32_t b_off, uint32_t a_sc,
                                        uint32_t b_sc, MmRaw &r)
{
#pragma unroll
    for (int v = 0; v < 8; v++) {
        const uint32_t roff = (v < 4 ? 0u : 2u * kMmQuadPitch) + 1024u * (v & 3);
        const uint32_t *pa = reinterpret_cast<const uint32_t *>(st + a_off + roff);
        const uint32_t *pb = reinterpret_cast<const uint32_t *>(st + b_off + roff);
        r.a[v][0] = pa[0];
        r.a[v][1] = pa[1];
#pragma unroll
        for (int u = 0; u < 4; u++)
            r.b[v][u] = pb[u];
    }
    r.as[0] = st[a_sc];
    r.as[1] = st[a_sc + 1];
    r.bs = *reinterpret_cast<const uint32_t *>(st + b_sc);
}

// s_waitcnt encodings (gfx9: vmcnt bits 3..0 and 15..14, expcnt 6..4,
// lgkmcnt 11..8).
constexpr int mm_wait_vm_lgkm(int vm) { return ((vm >> 4) << 14) | (0x7 << 4) | (vm & 15); }
constexpr int mm_wait_vm(int vm) { return mm_wait_vm_lgkm(vm) | (0xF << 8); }
constexpr int kMmAhead = (kMmStages - 2) * kMmCopies;     // loads that may stay in flight
static_assert(kMmAhead <= 63, "vmcnt counts to 63");
constexpr int kWaitAllCopies = mm_wait_vm(0);

// Quantize-on-produce: lane (i, h) holds, for each row group k = r >> 2 of
// its two A sub-tiles, the whole 8 x 4 block at rows m0 + wm + 16 k + 8 h
// + (2 j + a), j = r & 3, columns n0 + wn + 4 i .. + 3 (B sub-tiles u): the
// block maximum needs no lane exchange, and each row's 4 values are one x4
// container.
template <int OUT>
__device__ __forceinline__ void mm_quantize_epilogue(const f32x16_t (&acc)[2][4], uint32_t row0, uint32_t col,
                                                      uint32_t M, uint32_t N, uint8_t *__restrict__ data,
                                                      uint8_t *__restrict__ scale, int emax_bias, uint32_t dense)
{
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint32_t row = row0 + 16u * k;   // first row of the block
        uint32_t w[8][2];
        uint32_t m2 = 0;
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int a = 0; a < 2; a++) {
                const int r = 4 * k + j;
                uint32_t *x = w[2 * j + a];
                x[0] = mm_bf16_bits(acc[a][0][r]) | mm_bf16_bits(acc[a][1][r]) << 16;
                x[1] = mm_bf16_bits(acc[a][2][r]) | mm_bf16_bits(acc[a][3][r]) << 16;
                m2 = pk_max_u16(m2, pk_max_u16(x[0] & 0x7FFF7FFFu, x[1] & 0x7FFF7FFFu));
            }
        const uint32_t mag = max(m2 & 0xFFFFu, m2 >> 16);
        uint32_t e[1] = {block_e8m0<kInBF16>(mag, emax_bias)};
        const float sc = e8m0_to_scale(e[0]);
        const bool special = mag > InfBits<kInBF16>::value || e[0] == 254u;
        if (row >= M || col >= N)
            continue;
#pragma unroll
        for (int t = 0; t < 8; t++) {
            uint32_t out[1];
            if constexpr (OUT == kOutE2M1)
                out[0] = fp4_container<kInBF16, 0>(0u, w[t][0], w[t][1], sc);
            else
                out[0] = fp8x4<kInBF16, OUT>(w[t][0], w[t][1], sc);
            if (special)
                fix_special_codes<kInBF16, OUT, 1>(w[t], e, out);
            const uint64_t o = (uint64_t)(row + t) * N + col;
            if constexpr (OUT == kOutE2M1)
                *reinterpret_cast<uint16_t *>(data + o / 2) = (uint16_t)out[0];
            else
                *reinterpret_cast<uint32_t *>(data + o) = out[0];
        }
        const uint32_t grp = row / 8;
        const uint64_t slot = dense ? grp : (grp & 3u) + 32ull * (grp >> 2);
        scale[slot * (N / 4) + col / 4] = (uint8_t)e[0];
    }
}

// The lane's 8 operand dwords with the blocks whose flag is clear zeroed:
// dwords 0..3 belong to K block 0 of the step, 4..7 to block 1.
__device__ __forceinline__ i32x8_t mm_keep_blocks(const i32x8_t &v, bool block0, bool block1)
{
    i32x8_t o;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        o[k] = block0 ? v[k] : 0;
        o[k + 4] = block1 ? v[k + 4] : 0;
    }
    return o;
}

// The K step of one A sub-tile against the wave's 4 B sub-tiles where scale
// bytes may be 255. An E8M0 byte e stands for 2^(e - 127) for every e, 255
// (2^128) included -- the consumer's dequant is ldexpf(x, E8M0 - 127) --
// but the matrix cores read a scale byte of 0xFF as NaN. So every 255 is fed
// as 254 (2^127), which leaves each flagged block's products at half their
// value per flagged side. Lane (i, h) carries the scale of K block h of its
// row (column) i, so the flag of block 1 - h comes from lane (i, 1 - h).
// With A' and B' the operands keeping only their flagged blocks (dwords
// 0..3 are block 0, 4..7 block 1), the step adds (A, B) + (A', B) +
// (A', B') + (A, B'): a block flagged on one side counts twice, on both
// sides four times, an unflagged one once.
template <int F>
__device__ __forceinline__ void mm_step_255(f32x16_t (&acc)[4], const i32x8_t &aop, const i32x8_t (&bop)[4],
                                            uint32_t as, uint32_t bs, uint32_t h)
{
    // flag bits: 2 u + j for block j of B sub-tile u, 8 + j for block j of A
    uint32_t own = as == 255u ? 1u << 8 : 0u, bclamp = 0;
#pragma unroll
    for (int u = 0; u < 4; u++) {
        const uint32_t byte = (bs >> (8 * u)) & 0xFFu;
        own |= (byte == 255u ? 1u : 0u) << (2 * u);
        bclamp |= (byte == 255u ? 254u : byte) << (8 * u);
    }
    const uint32_t other = (uint32_t)__shfl_xor((int)own, 32);
    const uint32_t flags = h ? (own << 1) | other : own | (other << 1);
    const int sa = (int)min(as, 254u);
    const i32x8_t ta = mm_keep_blocks(aop, (flags >> 8) & 1u, (flags >> 9) & 1u);
#pragma unroll
    for (int u = 0; u < 4; u++) {
        const int sb = (int)(bclamp >> (8 * u));   // byte u in byte 0, op_sel 0
        const i32x8_t tb = mm_keep_blocks(bop[u], (flags >> (2 * u)) & 1u, (flags >> (2 * u + 1)) & 1u);
        acc[u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop[u], acc[u], F, F, 0, sa, 0, sb);
        acc[u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ta, bop[u], acc[u], F, F, 0, sa, 0, sb);
        acc[u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ta, tb, acc[u], F, F, 0, sa, 0, sb);
        acc[u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, tb, acc[u], F, F, 0, sa, 0, sb);
    }
}

// A buffer over the K step `step` of an operand from column c0 (as the
// copies use): rows past P and bytes past the operand read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mm_step_rsrc(const MmSource &s, uint32_t P, uint32_t step)
{
    const uint32_t rows_left = min(P - step * kMmStepRows, kMmStepRows);
    return __builtin_amdgcn_make_buffer_rsrc((void *)(s.data + (uint64_t)step * kMmStepRows * s.pitch), (short)0,
                                             (int)(rows_left * s.pitch - s.col_bytes), kMmBufferFlags);
}

// The rare path: a wave's whole 64 x 128 part of the tile computed again,
// one A sub-tile at a time, with mm_step_255, the operands read straight
// from global memory in the main loop's lane mapping (lane (i, h): A
// container c0a + 2 i + a, B containers c0b + 4 i + u, rows 4 h .. 4 h + 3 and
// 8 + 4 h .. 11 + 4 h of each K step). No LDS and no barrier: the other
// waves go on undisturbed.
template <int F>
__device__ __forceinline__ void mm_tile_255(f32x16_t (&acc)[2][4], const uint8_t *lhs, const uint8_t *lhs_scale,
                                            const uint8_t *rhs, const uint8_t *rhs_scale, uint32_t P, uint32_t M,
                                            uint32_t N, uint32_t c0a, uint32_t c0b, uint32_t dense, uint32_t i,
                                            uint32_t h)
{
    MmSource sa, sb;
    mm_source(sa, lhs, lhs_scale, M, c0a);
    mm_source(sb, rhs, rhs_scale, N, c0b);
    const uint32_t groups = P / 8;
    const uint32_t nsteps = (P + kMmStepRows - 1) / kMmStepRows;
    const uint32_t lane_a = 4u * h * sa.pitch + 8u * i, lane_b = 4u * h * sb.pitch + 16u * i;
    // every sum restarts from zero at once, so no earlier value stays live
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int u = 0; u < 4; u++)
            acc[a][u] = f32x16_t{};
#pragma unroll
    for (int a = 0; a < 2; a++) {
        for (uint32_t s = 0; s < nsteps; s++) {
            const __amdgpu_buffer_rsrc_t ra = mm_step_rsrc(sa, P, s), rb = mm_step_rsrc(sb, P, s);
            // row 4 h + (v & 3) (+ 8 for v >= 4): the lane's part of the
            // offset in a vector register, the row's in a scalar one
            i32x8_t aop, bop[4];
#pragma unroll
            for (int v = 0; v < 8; v++) {
                const uint32_t vrow = (v < 4 ? 0u : 8u) + (v & 3);
                aop[v] = (int)__builtin_amdgcn_raw_buffer_load_b32(ra, lane_a + 4u * a, vrow * sa.pitch, 0);
#pragma unroll
                for (int u = 0; u < 4; u++)
                    bop[u][v] = (int)__builtin_amdgcn_raw_buffer_load_b32(rb, lane_b + 4u * u, vrow * sb.pitch, 0);
            }
            // this lane's scales: K block 2 s + h of its A container and B
            // containers; a block past P / 8 has zero data and gets 127
            const uint32_t g = 2u * s + h;
            uint32_t as = 0x7Fu, bs = 0x7F7F7F7Fu;
            if (g < groups) {
                // the scale row from column c0 on, as the copies read it:
                // containers past the operand's last read as zero
                const uint64_t srow = dense ? g : (g & 3u) + 32u * (g >> 2);
                const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)(sa.scale + srow * M), (short)0, (int)sa.scale_cols, kMmBufferFlags);
                const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)(sb.scale + srow * N), (short)0, (int)sb.scale_cols, kMmBufferFlags);
                as = __builtin_amdgcn_raw_buffer_load_b8(rsa, 2u * i + a, 0, 0);
                bs = __builtin_amdgcn_raw_buffer_load_b32(rsb, 4u * i, 0, 0);
            }
            mm_step_255<F>(acc[a], aop, bop, as, bs, h);
        }
    }
}

// Store a wave's sums (64 x 128 from row wm0, column wn0): f32, bf16 or MX
// quantized. M and N are multiples of 4 (checked on the host), so a row's 4
// adjacent results are one aligned 16-byte (f32) or 8-byte (bf16) store.
template <int EPI>
__device__ __forceinline__ void mm_epilogue(const f32x16_t (&acc)[2][4], uint32_t wm0, uint32_t wn0, uint32_t M,
                                            uint32_t N, void *__restrict__ out, uint8_t *__restrict__ out_scale,
                                            int emax_bias, uint32_t dense, uint32_t i, uint32_t h)
{
    const uint32_t col = wn0 + 4u * i;
    const uint32_t row0 = wm0 + 8u * h;   // + 16 (r >> 2) + 2 (r & 3) + a
    if constexpr (EPI >= kEpiMx) {
        mm_quantize_epilogue<EPI - kEpiMx>(acc, row0, col, M, N, reinterpret_cast<uint8_t *>(out), out_scale,
                                            emax_bias, dense);
        return;
    }
    if (col >= N)
        return;
#pragma unroll
    for (int r = 0; r < 16; r++)
#pragma unroll
        for (int a = 0; a < 2; a++) {
            const uint32_t m = row0 + 16u * (r >> 2) + 2u * (r & 3) + a;
            if (m >= M)
                continue;
            const uint64_t o = (uint64_t)m * N + col;
            if constexpr (EPI == kEpiF32)
                *reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + o) =
                    float4{acc[a][0][r], acc[a][1][r], acc[a][2][r], acc[a][3][r]};
            else
                *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(out) + o) =
                    uint2{mm_bf16_bits(acc[a][0][r]) | mm_bf16_bits(acc[a][1][r]) << 16,
                          mm_bf16_bits(acc[a][2][r]) | mm_bf16_bits(acc[a][3][r]) << 16};
        }
}

// The rare path as a function of its own (not inlined): its registers are
// allocated apart from the main loop's, and nothing of the caller but a few
// scalars is live across the call. It computes the wave's part with
// mm_tile_255 and stores it.
template <int F, int EPI>
__device__ __attribute__((noinline)) void mm_rare_part(const uint8_t *lhs, const uint8_t *lhs_scale,
                                                       const uint8_t *rhs, const uint8_t *rhs_scale, uint32_t P,
                                                       uint32_t M, uint32_t N, uint32_t wm0, uint32_t wn0,
                                                       uint32_t dense, void *out, uint8_t *out_scale, int emax_bias)
{
    const uint32_t lane = __lane_id();
    const uint32_t i = lane & 31u, h = lane >> 5;
    f32x16_t acc[2][4];
    mm_tile_255<F>(acc, lhs, lhs_scale, rhs, rhs_scale, P, M, N, wm0, wn0, dense, i, h);
    mm_epilogue<EPI>(acc, wm0, wn0, M, N, out, out_scale, emax_bias, dense, i, h);
}

// The kernel: one 256 x 256 result tile per workgroup, the main loop in
// ping-pong, then the finiteness check, then the epilogue.
template <int FMT, int EPI>
__global__ __launch_bounds__(kMmThreads) void scaled_matmul_kernel(
    const uint8_t *__restrict__ lhs, const uint8_t *__restrict__ lhs_scale, const uint8_t *__restrict__ rhs,
    const uint8_t *__restrict__ rhs_scale, uint32_t P, uint32_t M, uint32_t N, uint32_t tiles_n, uint32_t dense,
    void *__restrict__ out, uint8_t *__restrict__ out_scale, int emax_bias)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[kMmStages * kMmStageBytes + kMmSpareBytes];
    constexpr int F = MfmaFmt<FMT>::value;

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t grp = wave >> 2, wq = wave & 3u;
    const uint32_t i = lane & 31u, h = lane >> 5;

    // Tile order. Workgroup w runs on XCD w % 8, so XCD x is given the
    // consecutive tile numbers [x * q, (x + 1) * q) (a tail stays in place).
    // Tile numbers walk the output in groups of kMmGroupRows tile rows,
    // column by column: the workgroups one XCD runs at a time cover a compact
    // block (4 tile rows x 8 tile columns for 32 CUs) and share its operand
    // panels in that XCD's L2.
    const uint32_t ntiles = gridDim.x;
    const uint32_t tiles_m = ntiles / tiles_n;
    const uint32_t q = ntiles / kMmXcds;
    const uint32_t w = blockIdx.x;
    const uint32_t t = w < q * kMmXcds ? (w % kMmXcds) * q + w / kMmXcds : w;
    const uint32_t group = t / (kMmGroupRows * tiles_n);
    const uint32_t first_row = group * kMmGroupRows;
    const uint32_t rows_in_group = min((uint32_t)kMmGroupRows, tiles_m - first_row);
    const uint32_t in_group = t - group * kMmGroupRows * tiles_n;
    const uint32_t m0 = (first_row + in_group % rows_in_group) * kMmTile;
    const uint32_t n0 = (in_group / rows_in_group) * kMmTile;
    const uint32_t wm = 64u * wq, wn = 128u * grp;
    const uint32_t nsteps = (P + kMmStepRows - 1) / kMmStepRows;

    MmSource src;                                          // the operand this wave copies
    mm_source(src, grp ? rhs : lhs, grp ? rhs_scale : lhs_scale, grp ? N : M, grp ? n0 : m0);
    const uint32_t t_off = grp ? kMmTileBytes : 0u;
    const bool has_scale = wq < 2u;
    const uint32_t s_off = 2u * kMmTileBytes + (grp ? kMmScaleBytes : 0u) + kMmTile * (wq & 1u);
    uint8_t *spare = lds + kMmStages * kMmStageBytes;

    // lane-constant LDS offsets of the operand reads
    const uint32_t a_off = kMmQuadPitch * h + 4u * (wm + 2u * i);
    const uint32_t b_off = kMmTileBytes + kMmQuadPitch * h + 4u * (wn + 4u * i);
    const uint32_t a_sc = 2u * kMmTileBytes + kMmTile * h + wm + 2u * i;
    const uint32_t b_sc = 2u * kMmTileBytes + kMmScaleBytes + kMmTile * h + wn + 4u * i;

    f32x16_t acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int u = 0; u < 4; u++)
            acc[a][u] = f32x16_t{};

    // prologue: steps 0 .. kMmStages - 2 into stages 0 .. kMmStages - 2
#pragma unroll
    for (uint32_t st = 0; st < kMmStages - 1; st++) {
        uint8_t *stage = lds + st * kMmStageBytes;
        mm_copy_quad(src, stage + t_off, P, st, wq, lane);
        mm_copy_scale(src, stage + s_off, spare, has_scale, P, 2 * st + (wq & 1u), dense, lane);
    }
    __builtin_amdgcn_s_waitcnt(mm_wait_vm(kMmAhead));     // step 0 has landed
    __builtin_amdgcn_s_barrier();
    // Group 1 runs half a step behind: barrier j closes group 0's memory
    // phase and group 1's compute phase (j even), or the other way round.
    // Every wave passes 2 nsteps + 2 barriers.
    if (grp)
        __builtin_amdgcn_s_barrier();

    uint32_t cur_i = 0;
    for (uint32_t s = 0; s < nsteps; s++) {
        const uint32_t fre_i = cur_i == 0 ? kMmStages - 1 : cur_i - 1u;   // step s - 1's stage
        const uint8_t *cur = lds + cur_i * kMmStageBytes;
        uint8_t *fre = lds + fre_i * kMmStageBytes;

        // memory phase: read step s's operands, copy step s + kMmStages - 1;
        // then wait for my reads and for my copies of step s + 1 (the barrier
        // then makes everyone's copies of step s + 1 visible)
        __builtin_amdgcn_sched_barrier(0);
        MmRaw r;
        mm_read(cur, a_off, b_off, a_sc, b_sc, r);
        const uint32_t ahead = s + kMmStages - 1;
        mm_copy_quad(src, fre + t_off, P, ahead, wq, lane);
        mm_copy_scale(src, fre + s_off, spare, has_scale, P, 2 * ahead + (wq & 1u), dense, lane);
        __builtin_amdgcn_s_waitcnt(mm_wait_vm_lgkm(kMmAhead));
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);

        // compute phase: gather the sub-tile operands, 8 MFMAs
        i32x8_t aop[2], bop[4];
#pragma unroll
        for (int a = 0; a < 2; a++)
            aop[a] = i32x8_t{(int)r.a[0][a], (int)r.a[1][a], (int)r.a[2][a], (int)r.a[3][a],
                             (int)r.a[4][a], (int)r.a[5][a], (int)r.a[6][a], (int)r.a[7][a]};
#pragma unroll
        for (int u = 0; u < 4; u++)
            bop[u] = i32x8_t{(int)r.b[0][u], (int)r.b[1][u], (int)r.b[2][u], (int)r.b[3][u],
                             (int)r.b[4][u], (int)r.b[5][u], (int)r.b[6][u], (int)r.b[7][u]};
#pragma unroll
        for (int a = 0; a < 2; a++) {
            acc[a][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop[a], bop[0], acc[a][0], F, F, 0,
                                                                        (int)r.as[a], 0, (int)r.bs);
            acc[a][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop[a], bop[1], acc[a][1], F, F, 0,
                                                                        (int)r.as[a], 1, (int)r.bs);
            acc[a][2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop[a], bop[2], acc[a][2], F, F, 0,
                                                                        (int)r.as[a], 2, (int)r.bs);
            acc[a][3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop[a], bop[3], acc[a][3], F, F, 0,
                                                                        (int)r.as[a], 3, (int)r.bs);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        cur_i = cur_i == kMmStages - 1 ? 0u : cur_i + 1u;
    }
    if (!grp)
        __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_waitcnt(kWaitAllCopies);

    // The matrix cores read a scale byte of 255 as NaN, where it stands for
    // 2^128. A sum that is not finite may come from one, so the wave then
    // computes its part again on the rare path, which gives every byte its
    // value (and any other non-finite sum the same value again), and stores
    // that.
    bool finite = true;
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int u = 0; u < 4; u++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                finite = finite && __builtin_isfinite(acc[a][u][r]);

    if (__builtin_amdgcn_ballot_w64(!finite) != 0) {
        mm_rare_part<F, EPI>(lhs, lhs_scale, rhs, rhs_scale, P, M, N, m0 + wm, n0 + wn, dense, out, out_scale,
                             emax_bias);
        // the wave ends here (no path back to the epilogue below, whose
        // sums would otherwise have to stay live across this branch)
        __builtin_amdgcn_endpgm();
    }
    mm_epilogue<EPI>(acc, m0 + wm, n0 + wn, M, N, out, out_scale, emax_bias, dense, i, h);
}

} // namespace mxq
