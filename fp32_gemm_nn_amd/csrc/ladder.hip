// The vector-ALU technique ladder: the itan.pw RTX 4090 SGEMM page's steps
// (section 3), each rewritten for CDNA4's 64-wide waves and computed with
// plain FP32 fused multiply-adds on the vector ALUs instead of the matrix
// cores. They are reachable only through mi_sgemm_with_config, as baselines
// for the page's progression and as an independent check of the MFMA path;
// mi_sgemm never selects them.
//
// Every rung computes C = alpha*op(A)*op(B) + beta*C for any shape, op pair,
// leading dimension and alignment: out-of-range rows, columns and k terms are
// selected to zero (never multiplied in), stores are masked to i < M, j < N,
// and C is not read when beta == 0. Each output's k sum runs in ascending k,
// one FMA per term, so results are run-to-run identical.
//
// Packed FP32 (two FMAs per instruction) is switched off for this build, so
// the inner loops are plain v_fmac_f32. Their ceiling is the FP32 vector
// rate of 256 FLOP per clock per CU (256 CUs x 2.4 GHz: 157.3 TFLOP/s, the
// same figure as the FP32 matrix cores): the top rung runs 88.9 TFLOP/s at
// 4096^3 on MI355X, more than a 16-lane-per-SIMD unpacked rate (78.6) would
// allow.

#include "ladder.h"

#include <stddef.h>

namespace misgemm_ladder {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// op(A)(i, k) and op(B)(k, j) of the stored row-major matrices.
template <bool TA>
__device__ __forceinline__ float op_a(const LadderArgs &g, int i, int k) {
    return TA ? g.A[(size_t)k * g.lda + i] : g.A[(size_t)i * g.lda + k];
}
template <bool TB>
__device__ __forceinline__ float op_b(const LadderArgs &g, int k, int j) {
    return TB ? g.B[(size_t)j * g.ldb + k] : g.B[(size_t)k * g.ldb + j];
}

// C(i, j) <- alpha*s + beta*C(i, j); C is not read when beta == 0.
__device__ __forceinline__ void put_c(const LadderArgs &g, int i, int j, float s) {
    float *p = g.C + (size_t)i * g.ldc + j;
    const float o = g.alpha * s;
    *p = g.beta != 0.0f ? fmaf(g.beta, *p, o) : o;
}

// Four adjacent outputs of row i starting at column j: one 16-byte access
// when all four are in range and C allows it, else element by element.
__device__ __forceinline__ void put_c4(const LadderArgs &g, int i, int j, const float (&s)[4]) {
    if (i >= g.M) return;
    if (g.vec_c && j + 3 < g.N) {
        f32x4 *p = reinterpret_cast<f32x4 *>(g.C + (size_t)i * g.ldc + j);
        f32x4 v;
        if (g.beta != 0.0f) {
            const f32x4 c = *p;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = fmaf(g.beta, c[e], g.alpha * s[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = g.alpha * s[e];
        }
        *p = v;
        return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (j + e < g.N) put_c(g, i, j + e, s[e]);
}

// ---------------------------------------------------------------------------
// Rung 0 (section 3.1). One thread per output, its k sum read straight from
// global memory. The page's fix for uncoalesced reads is to give consecutive
// threads consecutive columns; here the 64 lanes of a wave take 64 adjacent
// columns of one row, so op(B) 'N' and C are accessed in 256-byte runs and
// op(A) 'N' is one broadcast address per wave.
template <bool TA, bool TB>
__global__ __launch_bounds__(256) void valu_naive(LadderArgs g) {
    const long long cols = (g.N + 63) / 64, tiles = cols * ((g.M + 3) / 4);
    for (long long t = blockIdx.x; t < tiles; t += gridDim.x) {
        const int j = (int)(t % cols) * 64 + (int)(threadIdx.x & 63);
        const int i = (int)(t / cols) * 4 + (int)(threadIdx.x >> 6);
        if (i >= g.M || j >= g.N) continue;
        float s = 0.0f;
        for (int k = 0; k < g.K; ++k) s = fmaf(op_a<TA>(g, i, k), op_b<TB>(g, k, j), s);
        put_c(g, i, j, s);
    }
}

// ---------------------------------------------------------------------------
// Rung 1 (section 3.2). A 32 x 32 tile of C per workgroup (16 waves), one
// output per thread; each 32-wide k step stages a 32 x 32 block of op(A) and
// of op(B) in LDS. Each block is fetched along its stored contiguous axis and
// written transposed when that axis is not the one the inner product walks;
// rows are padded by one float so those transposed writes do not collide.
template <bool TA, bool TB>
__global__ __launch_bounds__(1024) void valu_lds32(LadderArgs g) {
    constexpr int T = 32;
    __shared__ float as[T][T + 1];   // [m][k]
    __shared__ float bs[T][T + 1];   // [k][n]
    const int tx = threadIdx.x % T, ty = threadIdx.x / T;
    const long long tiles_n = (g.N + T - 1) / T, tiles = tiles_n * ((g.M + T - 1) / T);
    for (long long t = blockIdx.x; t < tiles; t += gridDim.x) {
        const int m0 = (int)(t / tiles_n) * T, n0 = (int)(t % tiles_n) * T;
        float s = 0.0f;
        for (int k0 = 0; k0 < g.K; k0 += T) {
            if (!TA) {
                const int i = m0 + ty, k = k0 + tx;
                as[ty][tx] = (i < g.M && k < g.K) ? g.A[(size_t)i * g.lda + k] : 0.0f;
            } else {
                const int k = k0 + ty, i = m0 + tx;
                as[tx][ty] = (i < g.M && k < g.K) ? g.A[(size_t)k * g.lda + i] : 0.0f;
            }
            if (!TB) {
                const int k = k0 + ty, j = n0 + tx;
                bs[ty][tx] = (k < g.K && j < g.N) ? g.B[(size_t)k * g.ldb + j] : 0.0f;
            } else {
                const int j = n0 + ty, k = k0 + tx;
                bs[tx][ty] = (k < g.K && j < g.N) ? g.B[(size_t)j * g.ldb + k] : 0.0f;
            }
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < T; ++kk) s = fmaf(as[ty][kk], bs[kk][tx], s);
            __syncthreads();
        }
        if (m0 + ty < g.M && n0 + tx < g.N) put_c(g, m0 + ty, n0 + tx, s);
    }
}

// ---------------------------------------------------------------------------
// Rung 2 (section 3.3, 1-D block tiling). A 64 x 64 tile of C per workgroup
// of 512 threads, k in steps of 8; each thread accumulates 8 outputs of one
// column in registers, so one LDS read of op(B) serves 8 FMAs. A wave is one
// 8-row band: its op(A) reads are broadcasts.
template <bool TA, bool TB>
__global__ __launch_bounds__(512) void valu_block1d(LadderArgs g) {
    constexpr int BM = 64, BN = 64, BK = 8, TM = 8;
    __shared__ float as[BM][BK + 1];   // [m][k]
    __shared__ float bs[BK][BN];       // [k][n]
    const int tid = threadIdx.x, tx = tid % BN, ty = tid / BN;
    const long long tiles_n = (g.N + BN - 1) / BN, tiles = tiles_n * ((g.M + BM - 1) / BM);
    for (long long t = blockIdx.x; t < tiles; t += gridDim.x) {
        const int m0 = (int)(t / tiles_n) * BM, n0 = (int)(t % tiles_n) * BN;
        float acc[TM];
#pragma unroll
        for (int r = 0; r < TM; ++r) acc[r] = 0.0f;
        for (int k0 = 0; k0 < g.K; k0 += BK) {
            // One element of each 512-element block per thread, along the
            // stored contiguous axis.
            if (!TA) {
                const int r = tid / BK, c = tid % BK, i = m0 + r, k = k0 + c;
                as[r][c] = (i < g.M && k < g.K) ? g.A[(size_t)i * g.lda + k] : 0.0f;
            } else {
                const int r = tid / BM, c = tid % BM, k = k0 + r, i = m0 + c;
                as[c][r] = (i < g.M && k < g.K) ? g.A[(size_t)k * g.lda + i] : 0.0f;
            }
            if (!TB) {
                const int r = tid / BN, c = tid % BN, k = k0 + r, j = n0 + c;
                bs[r][c] = (k < g.K && j < g.N) ? g.B[(size_t)k * g.ldb + j] : 0.0f;
            } else {
                const int r = tid / BK, c = tid % BK, j = n0 + r, k = k0 + c;
                bs[c][r] = (k < g.K && j < g.N) ? g.B[(size_t)j * g.ldb + k] : 0.0f;
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < BK; ++k) {
                const float b = bs[k][tx];
#pragma unroll
                for (int r = 0; r < TM; ++r) acc[r] = fmaf(as[ty * TM + r][k], b, acc[r]);
            }
            __syncthreads();
        }
        const int j = n0 + tx;
        if (j < g.N)
#pragma unroll
            for (int r = 0; r < TM; ++r)
                if (m0 + ty * TM + r < g.M) put_c(g, m0 + ty * TM + r, j, acc[r]);
    }
}

// ---------------------------------------------------------------------------
// Rung 3 (section 3.4, 2-D block tiling). A 128 x 128 tile of C per
// workgroup of 256 threads, k in steps of 8; each thread owns an 8 x 8 block
// of C (rows 8*ty.., columns 8*tx..) and per k step reads 8 values of op(A)
// and 8 of op(B) from LDS for 64 FMAs. Element-wise loads, one LDS buffer,
// a barrier before and after each step's reads.
template <bool TA, bool TB>
__global__ __launch_bounds__(256) void valu_block2d(LadderArgs g) {
    constexpr int BM = 128, BN = 128, BK = 8, TM = 8, TN = 8, NT = 256;
    __shared__ float as[BM][BK + 1];   // [m][k]
    __shared__ float bs[BK][BN + 4];   // [k][n]
    const int tid = threadIdx.x, tx = tid % (BN / TN), ty = tid / (BN / TN);
    const long long tiles_n = (g.N + BN - 1) / BN, tiles = tiles_n * ((g.M + BM - 1) / BM);
    for (long long t = blockIdx.x; t < tiles; t += gridDim.x) {
        const int m0 = (int)(t / tiles_n) * BM, n0 = (int)(t % tiles_n) * BN;
        float acc[TM][TN];
#pragma unroll
        for (int r = 0; r < TM; ++r)
#pragma unroll
            for (int c = 0; c < TN; ++c) acc[r][c] = 0.0f;
        for (int k0 = 0; k0 < g.K; k0 += BK) {
#pragma unroll
            for (int e = tid; e < BM * BK; e += NT) {
                if (!TA) {
                    const int r = e / BK, c = e % BK, i = m0 + r, k = k0 + c;
                    as[r][c] = (i < g.M && k < g.K) ? g.A[(size_t)i * g.lda + k] : 0.0f;
                } else {
                    const int r = e / BM, c = e % BM, k = k0 + r, i = m0 + c;
                    as[c][r] = (i < g.M && k < g.K) ? g.A[(size_t)k * g.lda + i] : 0.0f;
                }
                if (!TB) {
                    const int r = e / BN, c = e % BN, k = k0 + r, j = n0 + c;
                    bs[r][c] = (k < g.K && j < g.N) ? g.B[(size_t)k * g.ldb + j] : 0.0f;
                } else {
                    const int r = e / BK, c = e % BK, j = n0 + r, k = k0 + c;
                    bs[c][r] = (k < g.K && j < g.N) ? g.B[(size_t)j * g.ldb + k] : 0.0f;
                }
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < BK; ++k) {
                float a[TM], b[TN];
#pragma unroll
                for (int r = 0; r < TM; ++r) a[r] = as[ty * TM + r][k];
#pragma unroll
                for (int c = 0; c < TN; ++c) b[c] = bs[k][tx * TN + c];
#pragma unroll
                for (int r = 0; r < TM; ++r)
#pragma unroll
                    for (int c = 0; c < TN; ++c) acc[r][c] = fmaf(a[r], b[c], acc[r][c]);
            }
            __syncthreads();
        }
#pragma unroll
        for (int r = 0; r < TM; ++r)
#pragma unroll
            for (int h = 0; h < TN / 4; ++h) {
                const float s[4] = {acc[r][4 * h], acc[r][4 * h + 1], acc[r][4 * h + 2], acc[r][4 * h + 3]};
                put_c4(g, m0 + ty * TM + r, n0 + tx * TN + 4 * h, s);
            }
    }
}

// ---------------------------------------------------------------------------
// Rung 4 (sections 3.5, 3.7, 3.8). The 2-D tile of rung 3 with
//   * 16-byte global loads: per k step each thread fetches four consecutive
//     elements of op(A) and four of op(B) along their stored contiguous axes
//     (element-wise with zero fill on edge tiles, unaligned operands and the
//     last partial k step);
//   * op(A) written to LDS transposed, k-major ([k][m]), so that both
//     operands are read along m / n; op(B) stored [k][n] (a k-contiguous
//     stored B is transposed the same way);
//   * two LDS buffers: the next step's global loads are issued before the
//     current step's FMAs and written to the other buffer afterwards, so one
//     barrier per step suffices (the double buffering without warp tiles of
//     section 3.7);
//   * vector LDS reads without bank conflicts: a thread's 8 x 8 outputs are
//     rows {4ty + i, 64 + 4ty + i} x columns {4tx + j, 64 + 4tx + j}, i, j < 4,
//     so the 16 column groups of a wave read 16 adjacent 16-byte runs of a
//     k row of op(B), and its 4 row groups read 4 broadcast runs of op(A).
template <bool TA, bool TB>
__global__ __launch_bounds__(256) void valu_vec2d(LadderArgs g) {
    constexpr int BM = 128, BN = 128, BK = 8;
    constexpr int AS = BM + 4, BS = BN + 4;   // row strides; keep 16-byte alignment
    __shared__ __attribute__((aligned(16))) float as[2][BK * AS];   // [k][m]
    __shared__ __attribute__((aligned(16))) float bs[2][BK * BS];   // [k][n]
    const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
    // This thread's four-element load of each block, in stored coordinates:
    // 'N' A / 'T' B (k contiguous): row tid / 2 of the 128, k offset 4 * (tid % 2);
    // 'T' A / 'N' B (m / n contiguous): k row tid / 32, offset 4 * (tid % 32).
    const int a_r = TA ? tid / 32 : tid / 2, a_c = TA ? 4 * (tid % 32) : 4 * (tid % 2);
    const int b_r = TB ? tid / 2 : tid / 32, b_c = TB ? 4 * (tid % 2) : 4 * (tid % 32);
    const long long tiles_n = (g.N + BN - 1) / BN, tiles = tiles_n * ((g.M + BM - 1) / BM);
    for (long long t = blockIdx.x; t < tiles; t += gridDim.x) {
        const int m0 = (int)(t / tiles_n) * BM, n0 = (int)(t % tiles_n) * BN;
        const bool interior = g.vec_ab && m0 + BM <= g.M && n0 + BN <= g.N;
        float ra[4], rb[4];
        auto fetch = [&](int k0) {
            if (interior && k0 + BK <= g.K) {
                const f32x4 va = TA ? *reinterpret_cast<const f32x4 *>(g.A + (size_t)(k0 + a_r) * g.lda + m0 + a_c)
                                    : *reinterpret_cast<const f32x4 *>(g.A + (size_t)(m0 + a_r) * g.lda + k0 + a_c);
                const f32x4 vb = TB ? *reinterpret_cast<const f32x4 *>(g.B + (size_t)(n0 + b_r) * g.ldb + k0 + b_c)
                                    : *reinterpret_cast<const f32x4 *>(g.B + (size_t)(k0 + b_r) * g.ldb + n0 + b_c);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ra[e] = va[e];
                    rb[e] = vb[e];
                }
                return;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (TA) {
                    const int k = k0 + a_r, i = m0 + a_c + e;
                    ra[e] = (k < g.K && i < g.M) ? g.A[(size_t)k * g.lda + i] : 0.0f;
                } else {
                    const int i = m0 + a_r, k = k0 + a_c + e;
                    ra[e] = (k < g.K && i < g.M) ? g.A[(size_t)i * g.lda + k] : 0.0f;
                }
                if (TB) {
                    const int j = n0 + b_r, k = k0 + b_c + e;
                    rb[e] = (k < g.K && j < g.N) ? g.B[(size_t)j * g.ldb + k] : 0.0f;
                } else {
                    const int k = k0 + b_r, j = n0 + b_c + e;
                    rb[e] = (k < g.K && j < g.N) ? g.B[(size_t)k * g.ldb + j] : 0.0f;
                }
            }
        };
        auto stash = [&](int buf) {
            float *a = as[buf], *b = bs[buf];
            if (TA) {
                *reinterpret_cast<f32x4 *>(a + a_r * AS + a_c) = f32x4{ra[0], ra[1], ra[2], ra[3]};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) a[(a_c + e) * AS + a_r] = ra[e];   // transposed write
            }
            if (TB) {
#pragma unroll
                for (int e = 0; e < 4; ++e) b[(b_c + e) * BS + b_r] = rb[e];   // transposed write
            } else {
                *reinterpret_cast<f32x4 *>(b + b_r * BS + b_c) = f32x4{rb[0], rb[1], rb[2], rb[3]};
            }
        };

        float acc[8][8];
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[r][c] = 0.0f;

        const int steps = (g.K + BK - 1) / BK;
        fetch(0);
        stash(0);
        __syncthreads();
        for (int s = 0; s < steps; ++s) {
            const int cur = s & 1;
            if (s + 1 < steps) fetch((s + 1) * BK);
            const float *a = as[cur], *b = bs[cur];
#pragma unroll
            for (int k = 0; k < BK; ++k) {
                const f32x4 a0 = *reinterpret_cast<const f32x4 *>(a + k * AS + 4 * ty);
                const f32x4 a1 = *reinterpret_cast<const f32x4 *>(a + k * AS + 64 + 4 * ty);
                const f32x4 b0 = *reinterpret_cast<const f32x4 *>(b + k * BS + 4 * tx);
                const f32x4 b1 = *reinterpret_cast<const f32x4 *>(b + k * BS + 64 + 4 * tx);
                const float av[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                const float bv[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
                for (int r = 0; r < 8; ++r)
#pragma unroll
                    for (int c = 0; c < 8; ++c) acc[r][c] = fmaf(av[r], bv[c], acc[r][c]);
            }
            // The other buffer was last read in step s - 1, before the
            // barrier that ended it.
            if (s + 1 < steps) stash(cur ^ 1);
            __syncthreads();
        }

#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int i = m0 + (r < 4 ? 4 * ty + r : 64 + 4 * ty + r - 4);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float s4[4] = {acc[r][4 * h], acc[r][4 * h + 1], acc[r][4 * h + 2], acc[r][4 * h + 3]};
                put_c4(g, i, n0 + 64 * h + 4 * tx, s4);
            }
        }
    }
}

// Workgroups: one per tile up to a cap; the kernels loop over the rest.
constexpr long long kMaxWorkgroups = 1 << 20;

unsigned grid_for(long long tiles) { return (unsigned)(tiles < kMaxWorkgroups ? tiles : kMaxWorkgroups); }

template <bool TA, bool TB>
hipError_t launch_t(int rung, const LadderArgs &a, hipStream_t stream) {
    auto tiles = [&](int bm, int bn) { return (long long)((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
    switch (rung) {
        case kNaive:
            hipLaunchKernelGGL((valu_naive<TA, TB>), dim3(grid_for(tiles(4, 64))), dim3(256), 0, stream, a);
            break;
        case kLds32:
            hipLaunchKernelGGL((valu_lds32<TA, TB>), dim3(grid_for(tiles(32, 32))), dim3(1024), 0, stream, a);
            break;
        case kBlock1d:
            hipLaunchKernelGGL((valu_block1d<TA, TB>), dim3(grid_for(tiles(64, 64))), dim3(512), 0, stream, a);
            break;
        case kBlock2d:
            hipLaunchKernelGGL((valu_block2d<TA, TB>), dim3(grid_for(tiles(128, 128))), dim3(256), 0, stream, a);
            break;
        default:
            hipLaunchKernelGGL((valu_vec2d<TA, TB>), dim3(grid_for(tiles(128, 128))), dim3(256), 0, stream, a);
            break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch(int rung, bool ta, bool tb, const LadderArgs &a, hipStream_t stream) {
    if (rung < 0 || rung >= kNumRungs) return hipErrorInvalidValue;
    if (!ta && !tb) return launch_t<false, false>(rung, a, stream);
    if (!ta && tb) return launch_t<false, true>(rung, a, stream);
    if (ta && !tb) return launch_t<true, false>(rung, a, stream);
    return launch_t<true, true>(rung, a, stream);
}

}  // namespace misgemm_ladder
