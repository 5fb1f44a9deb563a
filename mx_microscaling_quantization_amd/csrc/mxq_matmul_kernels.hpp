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
// MFMA mapping (v_mfma_scale_f32_16x16x128_f8f6f4, measured on gfx950):
//   lane l = i + 16 g supplies row i of A (column i of B) and, in its 32
//   operand bytes, K = 64 * (b >> 4) + 16 g + (b & 15) for byte b; lane group
//   g's scale byte covers K block g (K in [32 g, 32 g + 32)); the result
//   register r of lane l is D[4 g + r][i].
// With one K step = 32 operand rows = 8 row quads (4 rows each), the lane's
// operand is exactly two 16-byte pieces: row quad g (VGPRs 0..3) and row
// quad 4 + g (VGPRs 4..7) of its container column -- one of our 8x4 blocks
// split into halves. So LDS holds each tile container-major: for container
// c, 8 row quads of 16 bytes (row quad q = the 4 containers' bytes of rows
// 4q..4q+3 at column c); a lane reads its operand with two 16-byte loads.
// The row quads of container c are stored in slot q ^ ((c >> 1) & 7): the
// 16 lanes of one lane group then read 16 distinct 16-byte bank groups.
//
// Tiling: a 256-thread workgroup computes a 256 x 256 tile of out; each of
// its 4 waves a 128 x 128 quarter as 8 x 8 MFMAs (accumulators in AGPRs).
// The K loop steps 128 (32 operand rows); each step stages both operand
// tiles (256 containers x 128 bytes each) and their 4 x 256 scale bytes in
// LDS, double buffered: the next step's global loads are in flight during
// this step's 64 MFMAs per wave. A thread fetches 4 rows x 16 bytes (4
// containers) per piece and writes them transposed -- 4 container-major
// 16-byte row quads -- with no extra instructions. Workgroups are renumbered
// so that the 32 CUs of one XCD (which receive every eighth workgroup) work
// on a compact block of tiles and share operand panels in their L2. Tails
// in M, N and K are zero-filled (E8M0 127) so every MFMA runs with all 64
// lanes active.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq_quantize_kernels.hpp"

namespace mxq {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMmTile = 256;        // output tile edge (M and N)
constexpr int kMmWaveTile = 128;    // per-wave output edge
constexpr int kMmSub = kMmWaveTile / 16;   // 8 MFMA tiles per wave edge
constexpr int kMmStepRows = 32;     // operand rows per K step (K = 128)
constexpr int kMmThreads = 256;
constexpr int kMmXcds = 8;
constexpr int kMmGroupRows = 4;     // tile rows walked together (L2 reuse)
constexpr int kMmStashA = 2;        // row tile that writes the next A tile (next: its loads)
constexpr int kMmStashB = 4;        // row tile that writes the next B tile (next: its loads)

// MFMA operand-format code of an element format (cbsz / blgp field).
template <int FMT> struct MfmaFmt;
template <> struct MfmaFmt<kOutE4M3FN> { static constexpr int value = 0; };
template <> struct MfmaFmt<kOutE5M2> { static constexpr int value = 1; };

// LDS stage: A tile, B tile (256 containers x 8 row quads x 16 bytes each),
// then the 4 x 256 E8M0 bytes of A and of B ([K block][container]).
constexpr uint32_t kMmTileBytes = kMmTile * 128;
constexpr uint32_t kMmScaleBytes = 4 * kMmTile;
constexpr uint32_t kMmStageBytes = 2 * kMmTileBytes + 2 * kMmScaleBytes;
constexpr uint32_t kMmBufferFlags = 0x00020000u;   // raw untyped buffer, 32-bit data format

// Row quad q of container c is stored in slot q ^ ((c >> 1) & 7).
__device__ __forceinline__ uint32_t mm_slot(uint32_t c, uint32_t q) { return q ^ ((c >> 1) & 7u); }

// Global side of one operand. Thread t stages row quad t & 7 (rows
// 4 (t & 7) + u, u = 0..3, of each K step) of container groups t >> 3 and
// (t >> 3) + 32 (4 containers = 16 bytes each; the second group 512 bytes
// further), and 4 E8M0 bytes of K block (wave) at containers 4 (t & 63)..+3.
// Loads go through a raw buffer descriptor rebased on each K step whose
// size ends at row P: rows past the end read as zero without a branch.
// Columns past C read bytes of another row (or zeros); they only reach
// results outside the output, which are not stored.
struct MmSource {
    const uint8_t *data;        // column c0 of row 0
    const uint8_t *scale;       // column c0 of scale row 0
    uint64_t pitch;             // 4 C bytes
    uint32_t C, scale_cols;     // containers; scale bytes left in a row from c0
    uint32_t col_bytes;         // 4 c0: bytes of a row before the tile
    uint32_t voff[4];           // lane offset of row 4 (t & 7) + u within a step
};

struct MmFetch {
    u32x4_t w[2][4];   // [container group][row in quad]
    uint32_t scale;    // 4 E8M0 bytes
};

__device__ __forceinline__ void mm_source(MmSource &src, const uint8_t *data, const uint8_t *scale, uint32_t C,
                                          uint32_t c0, uint32_t tid)
{
    src.pitch = 4ull * C;
    src.data = data + 4ull * c0;
    src.scale = scale + c0;
    src.C = C;
    src.scale_cols = C - c0;
    src.col_bytes = 4u * c0;
    const uint32_t rq = tid & 7u, cg = tid >> 3;
#pragma unroll
    for (int u = 0; u < 4; u++)
        src.voff[u] = (4u * rq + u) * (uint32_t)src.pitch + 16u * cg;
}

// Global loads of K step `step` into registers.
__device__ __forceinline__ void mm_fetch(MmFetch &f, const MmSource &src, uint32_t P, uint32_t step, uint32_t wave,
                                         uint32_t dense, uint32_t lane)
{
    // The range starts at column c0 of the step's first row and ends at the
    // operand's last byte when the step reaches row P. A step at or past row
    // P gets an empty range at row 0: no memory is touched.
    const bool in_range = step * kMmStepRows < P;
    const uint32_t rows_left = in_range ? min(P - step * kMmStepRows, (uint32_t)kMmStepRows) : 0u;
    const uint32_t bytes = in_range ? rows_left * (uint32_t)src.pitch - src.col_bytes : 0u;
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(src.data + (in_range ? (uint64_t)step * kMmStepRows * src.pitch : 0ull)), (short)0, (int)bytes,
        kMmBufferFlags);
#pragma unroll
    for (int u = 0; u < 4; u++)
#pragma unroll
        for (int hh = 0; hh < 2; hh++)
            f.w[hh][u] = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rd, src.voff[u] + 512u * hh, 0, 0));
    // scale row of K block kb; blocks past P / 8 read as zero bytes (their data is zero)
    const uint32_t kb = step * 4 + wave;
    const bool kb_ok = kb < P / 8;
    const uint32_t srow = !kb_ok ? 0u : dense ? kb : (kb & 3u) + 32u * (kb >> 2);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(src.scale + (uint64_t)srow * src.C), (short)0, kb_ok ? (int)src.scale_cols : 0, kMmBufferFlags);
    f.scale = __builtin_amdgcn_raw_buffer_load_b32(rs, 4u * lane, 0, 0);
}

// Registers -> LDS, transposed to container-major row quads. `at` is the
// lane's byte address of container 4 (t >> 3) in the tile plus its slot for
// containers x = 0, 1; `at2` the same for x = 2, 3.
__device__ __forceinline__ void mm_stash(const MmFetch &f, uint8_t *tile, uint8_t *stile, uint32_t at, uint32_t at2,
                                         uint32_t tid)
{
#pragma unroll
    for (int hh = 0; hh < 2; hh++)
#pragma unroll
        for (int x = 0; x < 4; x++) {
            const uint32_t addr = (x < 2 ? at : at2) + 128u * (x & 1) + 16384u * hh;
            *reinterpret_cast<u32x4_t *>(tile + addr) =
                u32x4_t{f.w[hh][0][x], f.w[hh][1][x], f.w[hh][2][x], f.w[hh][3][x]};
        }
    *reinterpret_cast<uint32_t *>(stile + 4u * tid) = f.scale;
}

// A lane's operand for containers base + i + 16 t: with base a multiple of
// 16 the slots (c >> 1) & 7 = (i >> 1) & 7 do not depend on t, and the two
// 16-byte pieces (row quads g and g + 4) sit 64 bytes apart in the same
// container; t moves the address by 16 containers (2048 bytes).
__device__ __forceinline__ i32x8_t mm_operand(const uint8_t *tile, uint32_t lo, uint32_t hi, int t)
{
    const u32x4_t a = *reinterpret_cast<const u32x4_t *>(tile + lo + 2048u * t);
    const u32x4_t b = *reinterpret_cast<const u32x4_t *>(tile + hi + 2048u * t);
    return i32x8_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

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

// Quantize-on-produce ("MX-FP8 Microscaling Legalization", The pipeline
// coupling): the wave's 128 x 128 sums, rounded to bf16, are quantized as the
// quantize kernel would quantize that bf16 tensor -- 8-row x 4-column blocks
// of the M x N result, the same conversions and special-code pass -- and
// written as MX data (pitch N, or N / 2 for FP4) and E8M0 bytes.
//
// Lane (i, g) holds column 16 b + i, rows 4 g .. 4 g + 3 of sub-tile (a, b).
// Within each quad of lanes (4 consecutive columns) the bf16 values are
// transposed so that lane k of the quad holds row 4 g + k, columns 4 q ..
// 4 q + 3: one x4 container. A block (rows 8 h .. 8 h + 7, the quad's
// columns) is then the quad's 4 lanes in lane groups 2 h and 2 h + 1, and
// its maximum is a reduction over lanes xor 1, xor 2 and xor 16. Every lane
// runs the shuffles (full EXEC); only the stores are predicated.
template <int OUT>
__device__ __forceinline__ void mm_quantize_epilogue(const f32x4_t (&acc)[kMmSub][kMmSub], uint32_t row0,
                                                     uint32_t col0, uint32_t M, uint32_t N, uint32_t lane,
                                                     uint8_t *__restrict__ data, uint8_t *__restrict__ scale,
                                                     int emax_bias, uint32_t dense)
{
    const uint32_t i = lane & 15u, g = lane >> 4, k = lane & 3u, quad = lane & ~3u;
#pragma unroll
    for (int a = 0; a < kMmSub; a++)
#pragma unroll
        for (int b = 0; b < kMmSub; b++) {
            const uint32_t c01 = mm_bf16_bits(acc[a][b][0]) | mm_bf16_bits(acc[a][b][1]) << 16;
            const uint32_t c23 = mm_bf16_bits(acc[a][b][2]) | mm_bf16_bits(acc[a][b][3]) << 16;
            uint32_t h[4];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const uint32_t d01 = (uint32_t)__shfl((int)c01, (int)(quad | j));
                const uint32_t d23 = (uint32_t)__shfl((int)c23, (int)(quad | j));
                h[j] = ((k & 2u) ? d23 : d01) >> (16u * (k & 1u)) & 0xFFFFu;
            }
            uint32_t w[2] = {h[0] | h[1] << 16, h[2] | h[3] << 16};

            const uint32_t m2 = pk_max_u16(w[0] & 0x7FFF7FFFu, w[1] & 0x7FFF7FFFu);
            uint32_t mag = max(m2 & 0xFFFFu, m2 >> 16);
            mag = max(mag, (uint32_t)__shfl_xor((int)mag, 1));
            mag = max(mag, (uint32_t)__shfl_xor((int)mag, 2));
            mag = max(mag, (uint32_t)__shfl_xor((int)mag, 16));
            uint32_t e[1] = {block_e8m0<kInBF16>(mag, emax_bias)};
            const float sc = e8m0_to_scale(e[0]);
            const bool special = mag > InfBits<kInBF16>::value || e[0] == 254u;

            const uint32_t row = row0 + 16u * a + 4u * g + k;
            const uint32_t col = col0 + 16u * b + 4u * (i >> 2);
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
                if (k == 0 && (g & 1u) == 0) {   // the block's first row writes its E8M0
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
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kMmStageBytes];
    constexpr int F = MfmaFmt<FMT>::value;

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t i = lane & 15u, g = lane >> 4;

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
    mm_source(src_a, lhs, lhs_scale, M, m0, tid);
    mm_source(src_b, rhs, rhs_scale, N, n0, tid);

    // lane-constant LDS addresses (relative to a tile)
    const uint32_t rq = tid & 7u, cg = tid >> 3;
    const uint32_t st0 = 512u * cg + 16u * mm_slot(4u * cg, rq);
    const uint32_t st1 = 512u * cg + 256u + 16u * mm_slot(4u * cg + 2u, rq);
    const uint32_t a_lo = (wm + i) * 128u + 16u * mm_slot(i, g), a_hi = a_lo ^ 64u;
    const uint32_t b_lo = (wn + i) * 128u + 16u * mm_slot(i, g), b_hi = b_lo ^ 64u;
    const uint32_t a_sc = g * kMmTile + wm + i, b_sc = g * kMmTile + wn + i;

    f32x4_t acc[kMmSub][kMmSub];
#pragma unroll
    for (int a = 0; a < kMmSub; a++)
#pragma unroll
        for (int b = 0; b < kMmSub; b++)
            acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Software pipeline, per K step s (stage s & 1 holds step s). Each row
    // tile issues 8 MFMAs and reads the next row tile's A operand; besides,
    //   row tile 2 / 4: write step s + 1's A / B tile (in registers since
    //     step s - 1) into the other stage, one 16-byte LDS write per MFMA;
    //   row tile 3 / 5: issue the global loads of step s + 2 into the freed
    //     registers, one load per MFMA;
    //   row tile 7: one barrier (every wave has written step s + 1 and read
    //     its last operand of step s), then step s + 1's B operands and
    //     first A operand are read between the last 8 MFMAs.
    // With one wave per SIMD and in-order issue, a burst of loads or LDS
    // writes would stall the matrix core, so sched_group_barrier spreads
    // them between the MFMAs; sched_barrier fences the row tiles.
    MmFetch fa, fb;
    mm_fetch(fa, src_a, P, 0, wave, dense, lane);
    mm_fetch(fb, src_b, P, 0, wave, dense, lane);
    mm_stash(fa, lds, lds + 2 * kMmTileBytes, st0, st1, tid);
    mm_stash(fb, lds + kMmTileBytes, lds + 2 * kMmTileBytes + kMmScaleBytes, st0, st1, tid);
    if (nsteps > 1) {
        mm_fetch(fa, src_a, P, 1, wave, dense, lane);
        mm_fetch(fb, src_b, P, 1, wave, dense, lane);
    }
    __syncthreads();

    i32x8_t bop[kMmSub];
    int bsc[kMmSub];
    i32x8_t aop = mm_operand(lds, a_lo, a_hi, 0);
    int asc = lds[2 * kMmTileBytes + a_sc];
#pragma unroll
    for (int b = 0; b < kMmSub; b++) {
        bop[b] = mm_operand(lds + kMmTileBytes, b_lo, b_hi, b);
        bsc[b] = lds[2 * kMmTileBytes + kMmScaleBytes + b_sc + 16u * b];
    }

    for (uint32_t s = 0; s < nsteps; s++) {
        const uint8_t *cur = lds + (s & 1) * kMmStageBytes;
        uint8_t *nxt = lds + ((s + 1) & 1) * kMmStageBytes;
#pragma unroll
        for (int a = 0; a < kMmSub; a++) {
            __builtin_amdgcn_sched_barrier(0);
            if (a == kMmSub - 1) {
                __syncthreads();
                __builtin_amdgcn_sched_barrier(0);
            }
            i32x8_t an = aop;
            int ans = asc;
            // (on the last step the reads of the other stage are unused)
            if (a + 1 < kMmSub) {
                an = mm_operand(cur, a_lo, a_hi, a + 1);
                ans = cur[2 * kMmTileBytes + a_sc + 16u * (a + 1)];
            } else {
                an = mm_operand(nxt, a_lo, a_hi, 0);
                ans = nxt[2 * kMmTileBytes + a_sc];
            }
            // The loop body is one basic block, so nothing here is
            // conditional: on the last step the stash writes the other stage
            // (free since the previous barrier, never read again) and the
            // loads past the end read nothing.
            if (a == kMmStashA)
                mm_stash(fa, nxt, nxt + 2 * kMmTileBytes, st0, st1, tid);
            if (a == kMmStashA + 1)
                mm_fetch(fa, src_a, P, s + 2, wave, dense, lane);
            if (a == kMmStashB)
                mm_stash(fb, nxt + kMmTileBytes, nxt + 2 * kMmTileBytes + kMmScaleBytes, st0, st1, tid);
            if (a == kMmStashB + 1)
                mm_fetch(fb, src_b, P, s + 2, wave, dense, lane);
#pragma unroll
            for (int b = 0; b < kMmSub; b++) {
                acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop[b], acc[a][b], F, F, 0, asc,
                                                                             0, bsc[b]);
                if (a == kMmSub - 1) {
                    bop[b] = mm_operand(nxt + kMmTileBytes, b_lo, b_hi, b);
                    bsc[b] = nxt[2 * kMmTileBytes + kMmScaleBytes + b_sc + 16u * b];
                }
            }
            // instruction order inside the row tile (masks: 0x008 MFMA,
            // 0x100 LDS read, 0x200 LDS write, 0x020 global load, 0x002 VALU)
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);          // next A operand first
#pragma unroll
            for (int b = 0; b < kMmSub; b++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (a == kMmSub - 1) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // next step's B operand b
                } else if (a == kMmStashA || a == kMmStashB) {
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // gather one row quad
                    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // and write it
                } else if (a == kMmStashA + 1 || a == kMmStashB + 1) {
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
            }
            aop = an;
            asc = ans;
        }
    }

    if constexpr (EPI >= kEpiMx) {
        mm_quantize_epilogue<EPI - kEpiMx>(acc, m0 + wm, n0 + wn, M, N, lane, reinterpret_cast<uint8_t *>(out),
                                           out_scale, emax_bias, dense);
        return;
    }
    // result register r of lane (i, g) in sub-tile (a, b) is
    // out[m0 + wm + 16a + 4g + r][n0 + wn + 16b + i]
#pragma unroll
    for (int a = 0; a < kMmSub; a++)
#pragma unroll
        for (int b = 0; b < kMmSub; b++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const uint32_t m = m0 + wm + 16u * a + 4u * g + r;
                const uint32_t n = n0 + wn + 16u * b + i;
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
