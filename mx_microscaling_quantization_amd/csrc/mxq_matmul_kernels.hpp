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
// One of our 8x4 blocks (K block kb of 32 values = 8 u32 containers, rows
// 8 kb .. 8 kb + 7 at column 4c) therefore lands as two 16-byte halves:
// rows 8kb..8kb+3 in lane group 2 (kb & 1), rows 8kb+4..8kb+7 in lane group
// 2 (kb & 1) + 1, at bytes 16 (kb >> 1) .. 16 (kb >> 1) + 15. A lane reads
// its operand as 8 u32: VGPR 4h + q = row 8 (2h + (g >> 1)) + 4 (g & 1) + q.
//
// Tiling: a 256-thread workgroup computes a 128 x 128 tile of out; each of
// its 4 waves a 64 x 64 quarter as 4 x 4 MFMAs. The K loop steps 128 (32
// operand rows); each step stages both operand tiles (32 rows x 512 bytes)
// and their 4 x 128 scale bytes in LDS, double buffered so the next step's
// global loads are in flight while this step's MFMAs run. LDS rows are
// padded to 528 bytes: the four lane groups read rows 4 apart, which then
// fall 16 banks apart. Tails in M, N and K are zero-filled (with E8M0 127)
// so every MFMA runs with all 64 lanes active.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq_quantize_kernels.hpp"

namespace mxq {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMmTile = 128;        // output tile edge (M and N)
constexpr int kMmStepRows = 32;     // operand rows per K step (K = 128)
constexpr int kMmRowBytes = 4 * kMmTile;          // 512 bytes of one tile row
constexpr int kMmLdsPitch = kMmRowBytes + 16;     // padded LDS row
constexpr int kMmThreads = 256;

// MFMA operand-format code of an element format (cbsz / blgp field).
template <int FMT> struct MfmaFmt;
template <> struct MfmaFmt<kOutE4M3FN> { static constexpr int value = 0; };
template <> struct MfmaFmt<kOutE5M2> { static constexpr int value = 1; };

struct MmStage {
    uint8_t a[kMmStepRows][kMmLdsPitch];
    uint8_t b[kMmStepRows][kMmLdsPitch];
    uint8_t sa[4][kMmTile];
    uint8_t sb[4][kMmTile];
};

// Global -> registers for one K step of one operand tile: 1024 16-byte
// chunks (32 rows x 32 chunks) and 4 x 128 scale bytes, spread over the
// workgroup. Out-of-range chunks read as zero codes; out-of-range scales as
// 127 (so a zero element times its scale stays exactly zero).
struct MmFetch {
    u32x4_t chunk[4];
    uint32_t scale; // 4 scale bytes (threads 0..127 only)
};

__device__ __forceinline__ void mm_fetch(MmFetch &f, const uint8_t *__restrict__ data,
                                         const uint8_t *__restrict__ scale, uint32_t P, uint32_t C,
                                         uint32_t c0, uint32_t step, uint32_t dense, uint32_t tid)
{
    const uint64_t pitch = 4ull * C;      // operand row bytes
#pragma unroll
    for (int u = 0; u < 4; u++) {
        const uint32_t id = tid + kMmThreads * u;
        const uint32_t r = id >> 5, x = id & 31;
        const uint32_t row = step * kMmStepRows + r;
        const uint32_t col = 4u * c0 + 16u * x;           // byte column of the chunk
        if (row < P && col < 4u * C)                       // C % 4 == 0: a chunk is all in or all out
            f.chunk[u] = load<1>(reinterpret_cast<const u32x4_t *>(data + row * pitch + col));
        else
            f.chunk[u] = u32x4_t{0u, 0u, 0u, 0u};
    }
    // scales: thread t < 128 fetches 4 bytes: K block (t >> 5), columns c0 + 4 (t & 31) ..
    f.scale = 0x7F7F7F7Fu;
    if (tid < 128) {
        const uint32_t kb = step * 4 + (tid >> 5);
        const uint32_t c = c0 + 4u * (tid & 31);
        if (kb < P / 8 && c < C) {
            const uint64_t srow = dense ? (uint64_t)kb : (uint64_t)(kb & 3u) + 32u * (uint64_t)(kb >> 2);
            f.scale = load<1>(reinterpret_cast<const uint32_t *>(scale + srow * C + c));
        }
    }
}

__device__ __forceinline__ void mm_stash(const MmFetch &f, uint8_t (*tile)[kMmLdsPitch], uint8_t (*stile)[kMmTile],
                                         uint32_t tid)
{
#pragma unroll
    for (int u = 0; u < 4; u++) {
        const uint32_t id = tid + kMmThreads * u;
        const uint32_t r = id >> 5, x = id & 31;
        *reinterpret_cast<u32x4_t *>(&tile[r][16 * x]) = f.chunk[u];
    }
    if (tid < 128)
        *reinterpret_cast<uint32_t *>(&stile[tid >> 5][4 * (tid & 31)]) = f.scale;
}

// One lane's MFMA operand for tile-local container column c from a staged
// tile: VGPR 4h + q holds row 8 (2h + (g >> 1)) + 4 (g & 1) + q.
__device__ __forceinline__ i32x8_t mm_operand(const uint8_t (*tile)[kMmLdsPitch], uint32_t c, uint32_t g)
{
    i32x8_t v;
    const uint32_t base = 4u * (g & 1u) + 8u * (g >> 1);
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
        for (int q = 0; q < 4; q++)
            v[4 * h + q] = *reinterpret_cast<const int *>(&tile[base + 16u * h + q][4u * c]);
    return v;
}

template <int FMT, int RES>
__global__ __launch_bounds__(kMmThreads) void scaled_matmul_kernel(
    const uint8_t *__restrict__ lhs, const uint8_t *__restrict__ lhs_scale, const uint8_t *__restrict__ rhs,
    const uint8_t *__restrict__ rhs_scale, uint32_t P, uint32_t M, uint32_t N, uint32_t tiles_n, uint32_t dense,
    void *__restrict__ out)
{
    __shared__ MmStage stage[2];
    constexpr int F = MfmaFmt<FMT>::value;

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63, wave = tid >> 6;
    const uint32_t i = lane & 15, g = lane >> 4;
    const uint32_t m0 = (blockIdx.x / tiles_n) * kMmTile;
    const uint32_t n0 = (blockIdx.x % tiles_n) * kMmTile;
    const uint32_t wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    const uint32_t nsteps = (P + kMmStepRows - 1) / kMmStepRows;

    f32x4_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
        for (int b = 0; b < 4; b++)
            acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    MmFetch fa, fb;
    mm_fetch(fa, lhs, lhs_scale, P, M, m0, 0, dense, tid);
    mm_fetch(fb, rhs, rhs_scale, P, N, n0, 0, dense, tid);
    mm_stash(fa, stage[0].a, stage[0].sa, tid);
    mm_stash(fb, stage[0].b, stage[0].sb, tid);
    __syncthreads();

    for (uint32_t s = 0; s < nsteps; s++) {
        const MmStage &cur = stage[s & 1];
        const bool more = s + 1 < nsteps;
        if (more) {
            mm_fetch(fa, lhs, lhs_scale, P, M, m0, s + 1, dense, tid);
            mm_fetch(fb, rhs, rhs_scale, P, N, n0, s + 1, dense, tid);
        }
        i32x8_t bop[4];
        int bsc[4];
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const uint32_t c = wn + 16u * b + i;
            bop[b] = mm_operand(cur.b, c, g);
            bsc[b] = cur.sb[g][c];
        }
#pragma unroll
        for (int a = 0; a < 4; a++) {
            const uint32_t c = wm + 16u * a + i;
            const i32x8_t aop = mm_operand(cur.a, c, g);
            const int asc = cur.sa[g][c];
#pragma unroll
            for (int b = 0; b < 4; b++)
                acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop[b], acc[a][b], F, F, 0, asc,
                                                                             0, bsc[b]);
        }
        if (more) {
            MmStage &nxt = stage[(s + 1) & 1];
            mm_stash(fa, nxt.a, nxt.sa, tid);
            mm_stash(fb, nxt.b, nxt.sb, tid);
        }
        __syncthreads();
    }

    // result register r of lane (i, g) in sub-tile (a, b) is
    // out[m0 + wm + 16a + 4g + r][n0 + wn + 16b + i]
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
        for (int b = 0; b < 4; b++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const uint32_t m = m0 + wm + 16u * a + 4u * g + r;
                const uint32_t n = n0 + wn + 16u * b + i;
                if (m < M && n < N) {
                    const uint64_t o = (uint64_t)m * N + n;
                    if constexpr (RES == 0) {
                        reinterpret_cast<float *>(out)[o] = acc[a][b][r];
                    } else {
                        const uint32_t bits = __float_as_uint(acc[a][b][r]);
                        uint32_t rb;
                        if ((bits & 0x7FFFFFFFu) > 0x7F800000u)
                            rb = (bits >> 16) | 0x40u;
                        else
                            rb = (bits + 0x7FFFu + ((bits >> 16) & 1u)) >> 16;
                        reinterpret_cast<uint16_t *>(out)[o] = (uint16_t)rb;
                    }
                }
            }
}

} // namespace mxq
