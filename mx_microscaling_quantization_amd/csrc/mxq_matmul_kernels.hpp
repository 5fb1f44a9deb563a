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
// Tiling: a 256-thread workgroup computes a 256 x 256 tile of out; each of
// its 4 waves a 128 x 128 quarter as 4 x 4 MFMAs of 32 x 32 (accumulators in
// AGPRs). Workgroups are renumbered so that the 32 CUs of one XCD (which
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
constexpr int kMmWaveTile = 128;    // per-wave output edge
constexpr int kMmThreads = 256;
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
    if ((bits & 0x7FFFFFFFu) > 0x7F800000u)
        return (bits >> 16) | 0x40u;
    return (bits + 0x7FFFu + ((bits >> 16) & 1u)) >> 16;
}

// ----------------------------------------------------------------------------
// The kernel: v_mfma_scale_f32_32x32x64_f8f6f4, operands copied global ->
// LDS by the buffer unit itself (buffer_load_dwordx4 ... lds), no registers.
//
// MFMA mapping (measured on gfx950): lane l = i + 32 h supplies row i of A
// (column i of B); byte b of its 32 pairs with byte b of the same lane half
// of the other operand; scale block j (one E8M0) is bytes 16 j .. 16 j + 15 of
// both halves, and half h's scale byte covers block h; result register r of
// lane l is D[8 (r >> 2) + 4 h + (r & 3)][i].
// One K step is 64 = 16 operand rows = 4 row quads = 2 row groups (MX
// blocks). LDS holds each operand row-major, as the copy lands it: row quad
// q at q * kMmQuadPitch, row 4 q + v of it at + 1024 v, container c at + 4 c.
// Lane (i, h) supplies rows 4 h .. 4 h + 3 (block 0) and 8 + 4 h .. 11 + 4 h
// (block 1) of its container: 8 dword reads, VGPR v = row v, on a 256-byte
// grid so they pair into ds_read2st64_b32. The 128-byte pad of a row quad
// puts the two lane halves (row quads h and h + 1) in opposite halves of the
// LDS banks.
//
// In a 64-lane buffer_load_dwordx4 ... lds, lane L's 16 bytes go to LDS base +
// 16 L: lane L fetches containers 4 L .. 4 L + 3 of one row, and one load
// copies a 256-container row. Wave w copies row quad w of each operand (8
// loads) and one scale row (K block w mod 2 of operand w / 2) per step: 9
// loads. (Dword loads straight into a container-major layout cost four
// times as many instructions and measured slower than register staging.)
// kMmStages stages: the copy of step s + kMmStages - 1 is issued during
// row tiles 0 and 1 of step s into the stage step s - 1 used, and each wave
// waits for its copy of step s + 1 (the later copies may stay in flight)
// before the one barrier per step.
// ----------------------------------------------------------------------------
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kMmSub = kMmWaveTile / 32;                 // 4 x 4 MFMA tiles of 32 x 32 per wave
constexpr uint32_t kMmStepRows = 16;                      // operand rows per K step (K = 64)
constexpr int kMmStages = 3;                               // (4 measured no faster)
constexpr uint32_t kMmQuadPitch = kMmTile * 16 + 128;    // one row quad of a tile, padded
constexpr uint32_t kMmTileBytes = 4 * kMmQuadPitch;
constexpr uint32_t kMmScaleBytes = 2 * kMmTile;           // 2 K blocks x 256 containers
constexpr uint32_t kMmStageBytes = 2 * kMmTileBytes + 2 * kMmScaleBytes;
constexpr int kMmCopies = 9;                              // loads per wave per step

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
// past P / 8 read as zero (their data is zero too).
__device__ __forceinline__ void mm_copy_scale(const MmSource &s, uint8_t *stile, uint32_t P, uint32_t kb,
                                               uint32_t dense, uint32_t lane)
{
    const bool ok = kb < P / 8;
    const uint32_t srow = !ok ? 0u : dense ? kb : (kb & 3u) + 32u * (kb >> 2);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(s.scale + (uint64_t)srow * s.C), (short)0, ok ? (int)s.scale_cols : 0, kMmBufferFlags);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)stile, 4, 4u * lane, 0, 0, 0);
}

// A lane's operand for sub-tile t: its container in rows 4 h + v and
// 8 + 4 h + v (v = 0..3); `off` = row quad h, container of sub-tile 0.
__device__ __forceinline__ i32x8_t mm_operand(const uint8_t *tile, uint32_t off, int t)
{
    const uint32_t *p = reinterpret_cast<const uint32_t *>(tile + off + 128u * t);
    constexpr uint32_t Q2 = 2 * kMmQuadPitch / 4; // two row quads on, in dwords
    return i32x8_t{(int)p[0], (int)p[256], (int)p[512], (int)p[768],
                   (int)p[Q2], (int)p[Q2 + 256], (int)p[Q2 + 512], (int)p[Q2 + 768]};
}

// s_waitcnt encodings (gfx9: vmcnt bits 3..0 and 15..14, expcnt 6..4,
// lgkmcnt 11..8): the copies of all but the next step may be outstanding,
// with lgkmcnt(0); and vmcnt(0).
constexpr int kMmAhead = (kMmStages - 2) * kMmCopies;
static_assert(kMmAhead <= 63, "vmcnt counts to 63");
constexpr int kWaitNextCopyAndLds = ((kMmAhead >> 4) << 14) | (0x7 << 4) | (kMmAhead & 15);
constexpr int kWaitAllCopies = (0x7 << 4) | (0xF << 8);

// Quantize-on-produce for the 32 x 32 layout: lane (i, h) holds column
// 32 b + i, rows 8 k + 4 h .. 8 k + 4 h + 3 (registers 4 k .. 4 k + 3) of sub-tile
// (a, b). Within each quad of lanes (4 consecutive columns) the bf16 values
// are transposed so that lane j of the quad holds row 8 k + 4 h + j, columns
// 4 q .. 4 q + 3: one x4 container. A block (rows 8 k .. 8 k + 7, the quad's
// columns) is the quad's lanes in both halves; its maximum is a reduction
// over lanes xor 1, xor 2 and xor 32. Every lane runs the shuffles (full
// EXEC); only the stores are predicated.
template <int OUT>
__device__ __forceinline__ void mm_quantize_epilogue(const f32x16_t (&acc)[kMmSub][kMmSub], uint32_t row0,
                                                      uint32_t col0, uint32_t M, uint32_t N, uint32_t lane,
                                                      uint8_t *__restrict__ data, uint8_t *__restrict__ scale,
                                                      int emax_bias, uint32_t dense)
{
    const uint32_t i = lane & 31u, h = lane >> 5, j = lane & 3u, quad = lane & ~3u;
#pragma unroll
    for (int a = 0; a < kMmSub; a++)
#pragma unroll
        for (int b = 0; b < kMmSub; b++)
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const uint32_t c01 = mm_bf16_bits(acc[a][b][4 * k]) | mm_bf16_bits(acc[a][b][4 * k + 1]) << 16;
                const uint32_t c23 = mm_bf16_bits(acc[a][b][4 * k + 2]) | mm_bf16_bits(acc[a][b][4 * k + 3]) << 16;
                uint32_t hv[4];
#pragma unroll
                for (int jj = 0; jj < 4; jj++) {
                    const uint32_t d01 = (uint32_t)__shfl((int)c01, (int)(quad | jj));
                    const uint32_t d23 = (uint32_t)__shfl((int)c23, (int)(quad | jj));
                    hv[jj] = ((j & 2u) ? d23 : d01) >> (16u * (j & 1u)) & 0xFFFFu;
                }
                uint32_t w[2] = {hv[0] | hv[1] << 16, hv[2] | hv[3] << 16};

                const uint32_t m2 = pk_max_u16(w[0] & 0x7FFF7FFFu, w[1] & 0x7FFF7FFFu);
                uint32_t mag = max(m2 & 0xFFFFu, m2 >> 16);
                mag = max(mag, (uint32_t)__shfl_xor((int)mag, 1));
                mag = max(mag, (uint32_t)__shfl_xor((int)mag, 2));
                mag = max(mag, (uint32_t)__shfl_xor((int)mag, 32));
                uint32_t e[1] = {block_e8m0<kInBF16>(mag, emax_bias)};
                const float sc = e8m0_to_scale(e[0]);
                const bool special = mag > InfBits<kInBF16>::value || e[0] == 254u;

                const uint32_t row = row0 + 32u * a + 8u * k + 4u * h + j;
                const uint32_t col = col0 + 32u * b + 4u * (i >> 2);
                uint32_t out[1];
                if constexpr (OUT == kOutE2M1)
                    out[0] = fp4_container<kInBF16, 0>(0u, w[0], w[1], sc);
                else
                    out[0] = fp8x4<kInBF16, OUT>(w[0], w[1], sc);
                if (special)
                    fix_special_codes<kInBF16, OUT, 1>(w, e, out);
                if (row < M && col < N) {
                    if constexpr (OUT == kOutE2M1)
                        *reinterpret_cast<uint16_t *>(data + ((uint64_t)row * N + col) / 2) = (uint16_t)out[0];
                    else
                        *reinterpret_cast<uint32_t *>(data + (uint64_t)row * N + col) = out[0];
                    if (j == 0 && h == 0) { // the block's first row writes its E8M0
                        const uint32_t grp = row / 8;
                        const uint64_t slot = dense ? grp : (grp & 3u) + 32ull * (grp >> 2);
                        scale[slot * (N / 4) + col / 4] = (uint8_t)e[0];
                    }
                }
            }
}

template <int FMT, int EPI>
__global__ __launch_bounds__(kMmThreads) void scaled_matmul_kernel(
    const uint8_t *__restrict__ lhs, const uint8_t *__restrict__ lhs_scale, const uint8_t *__restrict__ rhs,
    const uint8_t *__restrict__ rhs_scale, uint32_t P, uint32_t M, uint32_t N, uint32_t tiles_n, uint32_t dense,
    void *__restrict__ out, uint8_t *__restrict__ out_scale, int emax_bias)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[kMmStages * kMmStageBytes];
    constexpr int F = MfmaFmt<FMT>::value;

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    const uint32_t wm = (wave >> 1) * kMmWaveTile, wn = (wave & 1u) * kMmWaveTile;
    const uint32_t nsteps = (P + kMmStepRows - 1) / kMmStepRows;

    MmSource src_a, src_b;
    mm_source(src_a, lhs, lhs_scale, M, m0);
    mm_source(src_b, rhs, rhs_scale, N, n0);
    MmSource src_s;                                        // this wave's scale rows
    mm_source(src_s, wave < 2 ? lhs : rhs, wave < 2 ? lhs_scale : rhs_scale, wave < 2 ? M : N, wave < 2 ? m0 : n0);
    const uint32_t s_kb = wave & 1u, s_off = (wave < 2 ? 0u : kMmScaleBytes) + kMmTile * s_kb;

    // lane-constant LDS offsets of the operand reads (sub-tile 0)
    const uint32_t a_off = kMmQuadPitch * h + 4u * (wm + i);
    const uint32_t b_off = kMmTileBytes + kMmQuadPitch * h + 4u * (wn + i);
    const uint32_t a_sc = 2 * kMmTileBytes + kMmTile * h + wm + i;
    const uint32_t b_sc = 2 * kMmTileBytes + kMmScaleBytes + kMmTile * h + wn + i;

    f32x16_t acc[kMmSub][kMmSub];
#pragma unroll
    for (int a = 0; a < kMmSub; a++)
#pragma unroll
        for (int b = 0; b < kMmSub; b++)
            acc[a][b] = f32x16_t{};

    // prologue: steps 0 .. kMmStages - 2 into stages 0 .. kMmStages - 2
#pragma unroll
    for (uint32_t st = 0; st < kMmStages - 1; st++) {
        uint8_t *stage = lds + st * kMmStageBytes;
        mm_copy_quad(src_a, stage, P, st, wave, lane);
        mm_copy_quad(src_b, stage + kMmTileBytes, P, st, wave, lane);
        mm_copy_scale(src_s, stage + 2 * kMmTileBytes + s_off, P, 2 * st + s_kb, dense, lane);
    }
    __builtin_amdgcn_s_waitcnt(kWaitNextCopyAndLds);
    __builtin_amdgcn_s_barrier();

    i32x8_t bop[kMmSub];
    int bsc[kMmSub];
    i32x8_t aop = mm_operand(lds, a_off, 0);
    int asc = lds[a_sc];
#pragma unroll
    for (int b = 0; b < kMmSub; b++) {
        bop[b] = mm_operand(lds, b_off, b);
        bsc[b] = lds[b_sc + 32u * b];
    }

    // Per step s (stage s mod kMmStages): row tile a issues its 4 MFMAs and
    // reads the next row tile's A operand; row tiles 0 and 1 also issue the
    // copy of step s + kMmStages - 1 into step s - 1's stage, free since the
    // previous barrier; before row tile 3 every wave waits for its copy of
    // step s + 1 and for its LDS reads, then one barrier; row tile 3 reads
    // step s + 1's B operands and first A operand between its MFMAs.
    uint32_t cur_i = 0;
    for (uint32_t s = 0; s < nsteps; s++) {
        const uint32_t nxt_i = cur_i == kMmStages - 1 ? 0u : cur_i + 1u;
        const uint32_t fre_i = cur_i == 0 ? kMmStages - 1 : cur_i - 1u; // step s - 1's stage
        const uint8_t *cur = lds + cur_i * kMmStageBytes;
        const uint8_t *nxt = lds + nxt_i * kMmStageBytes;
        uint8_t *fre = lds + fre_i * kMmStageBytes;
#pragma unroll
        for (int a = 0; a < kMmSub; a++) {
            __builtin_amdgcn_sched_barrier(0);
            if (a == kMmSub - 1) {
                __builtin_amdgcn_s_waitcnt(kWaitNextCopyAndLds);
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
            }
            i32x8_t an;
            int ans;
            if (a + 1 < kMmSub) {
                an = mm_operand(cur, a_off, a + 1);
                ans = cur[a_sc + 32u * (a + 1)];
            } else {
                an = mm_operand(nxt, a_off, 0);
                ans = nxt[a_sc];
            }
            const uint32_t ahead = s + kMmStages - 1;
            if (a == 0) {
                mm_copy_quad(src_a, fre, P, ahead, wave, lane);
                mm_copy_scale(src_s, fre + 2 * kMmTileBytes + s_off, P, 2 * ahead + s_kb, dense, lane);
            }
            if (a == 1)
                mm_copy_quad(src_b, fre + kMmTileBytes, P, ahead, wave, lane);
#pragma unroll
            for (int b = 0; b < kMmSub; b++) {
                acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop[b], acc[a][b], F, F, 0, asc, 0,
                                                                            bsc[b]);
                if (a == kMmSub - 1) {
                    bop[b] = mm_operand(nxt, b_off, b);
                    bsc[b] = nxt[b_sc + 32u * b];
                }
            }
            // instruction order inside the row tile (masks: 0x008 MFMA,
            // 0x100 LDS read, 0x020 global load)
            __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);          // next A operand first
#pragma unroll
            for (int b = 0; b < kMmSub; b++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (a == kMmSub - 1)
                    __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);  // next step's B operand b
                else if (a == 0 && b == 0)
                    __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
                else if (a <= 1)
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
            aop = an;
            asc = ans;
        }
        cur_i = nxt_i;
    }
    __builtin_amdgcn_s_waitcnt(kWaitAllCopies);

    if constexpr (EPI >= kEpiMx) {
        mm_quantize_epilogue<EPI - kEpiMx>(acc, m0 + wm, n0 + wn, M, N, lane, reinterpret_cast<uint8_t *>(out),
                                            out_scale, emax_bias, dense);
        return;
    }
    // result register r of lane (i, h) in sub-tile (a, b) is
    // out[m0 + wm + 32a + 8(r >> 2) + 4h + (r & 3)][n0 + wn + 32b + i]
#pragma unroll
    for (int a = 0; a < kMmSub; a++)
#pragma unroll
        for (int b = 0; b < kMmSub; b++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const uint32_t m = m0 + wm + 32u * a + 8u * (r >> 2) + 4u * h + (r & 3);
                const uint32_t n = n0 + wn + 32u * b + i;
                if (m < M && n < N) {
                    const uint64_t o = (uint64_t)m * N + n;
                    if constexpr (EPI == kEpiF32)
                        reinterpret_cast<float *>(out)[o] = acc[a][b][r];
                    else
                        reinterpret_cast<uint16_t *>(out)[o] = (uint16_t)mm_bf16_bits(acc[a][b][r]);
                }
            }
}

} // namespace mxq
