// HBM-bound kernels for products with few rows of C (sgemm_skinny16 and the
// split-K band kernel sgemm_skinny_band), and the small helper kernels
// zero_ints and scale_c.
// Internal to libmisgemm: compiled only as part of misgemm.hip, whose header comment
// describes the kernels and the configurations built from them.
#ifndef MISGEMM_SKINNY_KERNELS_H
#define MISGEMM_SKINNY_KERNELS_H

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "tile_common.h"

namespace {

// ---------------------------------------------------------------------------
// Skinny kernel: few rows of C (M <= 32 is its intended class), where the cost
// is one pass over op(B) from HBM (4KN bytes against 2MKN flops: under 20
// flop/byte for M <= 32, below the MI355X ridge of 157.3 TFLOP/s / 8 TB/s).
//
// One workgroup owns 16 columns of C and 16*MB rows (MB = 1 or 2), over all
// of K. Its kSkinnyWaves waves split K into contiguous runs of 16-row chunks
// and each keeps a 16 x 16 FP32 accumulator block per row block, fed by
// v_mfma_f32_16x16x4_f32. Lane (c, q) = (lane % 16, lane / 16) supplies
// column c of op(B) and row c of op(A) for k slot q; within a chunk, MFMA j
// takes k = k0 + 4q + j (a k-permutation shared by both operands), so the
// lane's four A values are one 16-byte load and, for B stored k-contiguous
// ('T'), so are its four B values. B ('N') is read one element per lane in
// exactly the MFMA layout: each load instruction covers 4 rows x 64 bytes.
// kSkinnyUnroll chunks of loads are in flight per wave before their MFMAs.
// The waves' partial blocks are summed through LDS in wave order (a fixed
// order: repeated calls give identical bits), then alpha/beta are applied
// and the block is stored with masks for M and N.
constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyUnroll = 8;

// Loads of one group of U chunks (k rows kc*16 .. (kc+U)*16) for one lane,
// zero where out of range.
template <int U, int MB, bool TA, bool TB>
struct SkinnyFrag {
    float b[U][4];
    float a[U][MB][4];

    __device__ __forceinline__ void load(const GemmArgs &g, const float *bcol, bool col_ok, int m0, int c,
                                         int q, int kc, int kc1, bool vec) {
        const int M = g.M, K = g.K, lda = g.lda, ldb = g.ldb;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool chunk_ok = kc + u < kc1;
            const int kq = (kc + u) * 16 + 4 * q;            // this lane's first k in the chunk
            const bool full = chunk_ok && kq + 4 <= K;
            if (TB && vec && full && col_ok) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(bcol + kq);
#pragma unroll
                for (int j = 0; j < 4; ++j) b[u][j] = v[j];
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int k = kq + j;
                    const bool ok = chunk_ok && col_ok && k < K;
                    b[u][j] = ok ? (TB ? bcol[k] : bcol[(size_t)k * ldb]) : 0.0f;
                }
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int row = m0 + 16 * mb + c;
                const bool row_ok = row < M;
                if (!TA && vec && full && row_ok) {
                    const f32x4 v = *reinterpret_cast<const f32x4 *>(g.A + (size_t)row * lda + kq);
#pragma unroll
                    for (int j = 0; j < 4; ++j) a[u][mb][j] = v[j];
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int k = kq + j;
                        const bool ok = chunk_ok && row_ok && k < K;
                        a[u][mb][j] = ok ? (TA ? g.A[(size_t)k * lda + row] : g.A[(size_t)row * lda + k]) : 0.0f;
                    }
                }
            }
        }
    }

    __device__ __forceinline__ void mma(f32x4 (&acc)[MB]) const {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u][mb][j], b[u][j], acc[mb], 0, 0, 0);
    }
};

template <int MB, bool TA, bool TB>
__global__ __launch_bounds__(64 * kSkinnyWaves) void sgemm_skinny16(GemmArgs g) {
    constexpr int NT = 64 * kSkinnyWaves, U = kSkinnyUnroll;
    __shared__ float red[kSkinnyWaves][MB][256];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int c = lane & 15, q = lane >> 4;
    // Column slabs: the j-th workgroup on XCD x takes slab prefix(x) + j, so
    // each XCD reads one contiguous band of columns and its L2 lines are
    // shared by neighbouring slabs.
    const int total = gridDim.x, bid = blockIdx.x;
    const int xq = total / kXcds, xr = total % kXcds, x = bid % kXcds;
    const int slab = x * xq + (x < xr ? x : xr) + bid / kXcds;
    const int n0 = slab * 16, m0 = blockIdx.y * 16 * MB;
    const int M = g.M, N = g.N, K = g.K;
    const bool vec = g.vec_ab != 0;

    const int nchunks = (K + 15) / 16;
    const int per = (nchunks + kSkinnyWaves - 1) / kSkinnyWaves;
    const int kc0 = w * per;
    const int kc1 = min(nchunks, kc0 + per);
    const bool col_ok = n0 + c < N;
    // op(B)(k, n0 + c): B[k*ldb + n0 + c] ('N') or B[(n0 + c)*ldb + k] ('T').
    const float *bcol = TB ? g.B + (size_t)(col_ok ? n0 + c : 0) * g.ldb : g.B + (col_ok ? n0 + c : 0);

    f32x4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // Two register buffers: the loads of the next U chunks are in flight while
    // the MFMAs of the current ones run.
    SkinnyFrag<U, MB, TA, TB> f0, f1;
    f0.load(g, bcol, col_ok, m0, c, q, kc0, kc1, vec);
    for (int kc = kc0; kc < kc1; kc += 2 * U) {
        f1.load(g, bcol, col_ok, m0, c, q, kc + U, kc1, vec);
        f0.mma(acc);
        if (kc + 2 * U >= kc1) {
            f1.mma(acc);
            break;
        }
        f0.load(g, bcol, col_ok, m0, c, q, kc + 2 * U, kc1, vec);
        f1.mma(acc);
    }

    // Accumulator element r of lane (c, q) is block row 4q + r, column c.
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[w][mb][(4 * q + r) * 16 + c] = acc[mb][r];
    __syncthreads();

    const float alpha = g.alpha, beta = g.beta;
    for (int t = tid; t < MB * 256; t += NT) {
        const int mb = t >> 8, rc = t & 255;
        const int row = m0 + 16 * mb + (rc >> 4), col = n0 + (rc & 15);
        float s = 0.0f;
#pragma unroll
        for (int v = 0; v < kSkinnyWaves; ++v) s += red[v][mb][rc];
        if (row < M && col < N) {
            float *p = g.C + (size_t)row * g.ldc + col;
            const float o = alpha * s;
            *p = (beta != 0.0f) ? fmaf(beta, *p, o) : o;
        }
    }
}

// ---------------------------------------------------------------------------
// Skinny kernel with K split over workgroups. A 16-column slab per workgroup
// (above) reads B in 64-byte pieces, which HBM serves at well under its
// streaming rate; here a workgroup owns a band of kBandCols = 128 columns
// (512-byte rows) and 1/S of K, so S workgroups share a band and the grid
// still fills the chip.
//
// Lane (c, q) = (lane % 16, lane / 16). Within a 16-row chunk, MFMA step j
// takes k = k0 + 4q + j for both operands (a k-permutation). For B stored
// n-contiguous ('N') the lane loads four columns n0 + 64h + 4c .. +3 of row
// k as one 16-byte load (h = 0, 1 picks the half band), and MFMA block
// (h, e) takes column n0 + 64h + 4c + e: one load instruction covers
// 4 rows x 256 bytes and feeds four 16x16x4 MFMAs. For B stored k-contiguous
// ('T'), block b takes columns n0 + 16b + c and the lane's four k values
// are one 16-byte load.
//
// Reduction, in a fixed order at every level: the waves of a
// workgroup split its k range and are summed through LDS in wave order; with
// S > 1 each workgroup then writes its partial block to the workspace and
// increments the band's counter; the one that brings the counter to S sums
// the S partials in split order, applies alpha/beta, stores C and resets the
// counter for the next call. No workgroup waits on another, so no grid-wide
// residency is assumed.
constexpr int kBandCols = 128;
constexpr int kBandWaves = 8;
constexpr int kMaxSplits = 32;
// Waves per workgroup. One row block: sixteen on the unguarded path (more
// loads in flight per CU; its fragments fit 128 registers), eight on the
// guarded one. Two row blocks: eight on the unguarded path (one chunk per
// buffer; the 8 x 16 KB LDS partial blocks fit), four on the guarded one, so
// each wave may use 512 registers (its fragments need ~260).
template <int MB, bool FAST> constexpr int band_waves() {
    return MB == 1 ? (FAST ? 2 * kBandWaves : kBandWaves) : (FAST ? kBandWaves : kBandWaves / 2);
}
// 16-row chunks per register buffer: one on the unguarded path, else two.
template <int MB, bool FAST> constexpr int band_chunks() { return FAST ? 1 : 2; }

struct SplitArgs {
    GemmArgs g;
    float *ws;            // [tile][split][16*MB*kBandCols] partial blocks
    int *counters;        // one per tile; zero between calls
    int splits;           // S
    int rows_per_split;   // multiple of 16
};

template <int MB, bool TA, bool TB, bool FAST>
struct BandFrag {
    static constexpr int kBandChunks = band_chunks<MB, FAST>();
    f32x4 b[kBandChunks][8];
    float a[kBandChunks][MB][4];

    // Chunk u covers k0 = kc + 16u .. +15, valid below kend. FAST: the host
    // has checked that every band lies inside N, every chunk below kend and
    // the pointers allow 16-byte loads, so no load of B is checked; rows of A
    // at or beyond M (A is small and stays in cache) read as zero.
    __device__ __forceinline__ void load(const GemmArgs &g, int m0, int n0, int c, int q, int kc, int kend,
                                         bool vec) {
        const int M = g.M, N = g.N, lda = g.lda, ldb = g.ldb;
#pragma unroll
        for (int u = 0; u < kBandChunks; ++u) {
            const int kq = kc + 16 * u + 4 * q;
            if constexpr (FAST) {
                if (!TB) {
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            b[u][4 * h + j] =
                                *reinterpret_cast<const f32x4 *>(g.B + (size_t)(kq + j) * ldb + n0 + 64 * h + 4 * c);
                } else {
#pragma unroll
                    for (int blk = 0; blk < 8; ++blk)
                        b[u][blk] = *reinterpret_cast<const f32x4 *>(g.B + (size_t)(n0 + 16 * blk + c) * ldb + kq);
                }
            } else if constexpr (!TB) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int col = n0 + 64 * h + 4 * c;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int k = kq + j;
                        const float *p = g.B + (size_t)k * ldb + col;
                        if (vec && k < kend && col + 3 < N) {
                            b[u][4 * h + j] = *reinterpret_cast<const f32x4 *>(p);
                        } else {
                            f32x4 t;
#pragma unroll
                            for (int e = 0; e < 4; ++e) t[e] = (k < kend && col + e < N) ? p[e] : 0.0f;
                            b[u][4 * h + j] = t;
                        }
                    }
                }
            } else {
#pragma unroll
                for (int blk = 0; blk < 8; ++blk) {
                    const int n = n0 + 16 * blk + c;
                    const float *p = g.B + (size_t)n * ldb + kq;
                    if (vec && n < N && kq + 3 < kend) {
                        b[u][blk] = *reinterpret_cast<const f32x4 *>(p);
                    } else {
                        f32x4 t;
#pragma unroll
                        for (int e = 0; e < 4; ++e) t[e] = (n < N && kq + e < kend) ? p[e] : 0.0f;
                        b[u][blk] = t;
                    }
                }
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int row = m0 + 16 * mb + c;
                // Unguarded path: load from a row clamped into range (no branch
                // in the streaming loop), then select zero past M.
                const int row_c = row < M ? row : M - 1;
                if (FAST && !TA) {
                    const f32x4 v = *reinterpret_cast<const f32x4 *>(g.A + (size_t)row_c * lda + kq);
#pragma unroll
                    for (int j = 0; j < 4; ++j) a[u][mb][j] = row < M ? v[j] : 0.0f;
                } else if (FAST) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float v = g.A[(size_t)(kq + j) * lda + row_c];
                        a[u][mb][j] = row < M ? v : 0.0f;
                    }
                } else if (!TA && vec && row < M && kq + 3 < kend) {
                    const f32x4 v = *reinterpret_cast<const f32x4 *>(g.A + (size_t)row * lda + kq);
#pragma unroll
                    for (int j = 0; j < 4; ++j) a[u][mb][j] = v[j];
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int k = kq + j;
                        const bool ok = row < M && k < kend;
                        a[u][mb][j] = ok ? (TA ? g.A[(size_t)k * lda + row] : g.A[(size_t)row * lda + k]) : 0.0f;
                    }
                }
            }
        }
    }

    __device__ __forceinline__ void mma(f32x4 (&acc)[MB][8]) const {
#pragma unroll
        for (int u = 0; u < kBandChunks; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int blk = 0; blk < 8; ++blk) {
                        // 'N': block blk = 4h + e takes element e of the row-j load of half h.
                        const float bv = TB ? b[u][blk][j] : b[u][4 * (blk / 4) + j][blk % 4];
                        acc[mb][blk] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u][mb][j], bv, acc[mb][blk], 0, 0, 0);
                    }
    }
};

template <int MB, bool TA, bool TB, bool FAST>
__global__ __launch_bounds__((64 * band_waves<MB, FAST>())) void sgemm_skinny_band(SplitArgs sa) {
    constexpr int W = band_waves<MB, FAST>();
    constexpr int NT = 64 * W;
    constexpr int T = 16 * MB * kBandCols;       // outputs per workgroup
    __shared__ float red[W][T];
    __shared__ int is_last;

    const GemmArgs &g = sa.g;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int c = lane & 15, q = lane >> 4;
    const int S = sa.splits;
    // Launch index -> (band, split): each XCD takes a contiguous run, so the
    // S workgroups of a band share an L2 whenever the run allows.
    const int total = gridDim.x, bid = blockIdx.x;
    const int xq = total / kXcds, xr = total % kXcds, x = bid % kXcds;
    const int logical = x * xq + (x < xr ? x : xr) + bid / kXcds;
    const int band = logical / S, split = logical % S;
    const int n0 = band * kBandCols, m0 = blockIdx.y * 16 * MB;
    const int tile = blockIdx.y * (total / S) + band;
    const int M = g.M, N = g.N, K = g.K;
    const bool vec = g.vec_ab != 0;

    const int ks = split * sa.rows_per_split;
    const int ke = min(K, ks + sa.rows_per_split);
    const int rpw = ((sa.rows_per_split / 16 + W - 1) / W) * 16;
    const int kw0 = ks + w * rpw;
    const int kw1 = min(ke, kw0 + rpw);

    f32x4 acc[MB][8];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) acc[mb][blk] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    constexpr int STEP = 16 * band_chunks<MB, FAST>();
    if (FAST) {
        // One register buffer: sixteen waves per CU keep enough loads in flight.
        BandFrag<MB, TA, TB, FAST> f;
        for (int kc = kw0; kc < kw1; kc += STEP) {
            f.load(g, m0, n0, c, q, kc, kw1, vec);
            f.mma(acc);
        }
    } else if (kw0 < kw1) {
        BandFrag<MB, TA, TB, FAST> f0, f1;
        f0.load(g, m0, n0, c, q, kw0, kw1, vec);
        for (int kc = kw0; kc < kw1; kc += 2 * STEP) {
            if (kc + STEP < kw1) f1.load(g, m0, n0, c, q, kc + STEP, kw1, vec);
            f0.mma(acc);
            if (kc + STEP >= kw1) break;
            if (kc + 2 * STEP < kw1) f0.load(g, m0, n0, c, q, kc + 2 * STEP, kw1, vec);
            f1.mma(acc);
        }
    }

    // Canonical block layout: index = row * kBandCols + col.
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) {
            const int col = TB ? 16 * blk + c : 64 * (blk / 4) + 4 * c + (blk % 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) red[w][(16 * mb + 4 * q + r) * kBandCols + col] = acc[mb][blk][r];
        }
    __syncthreads();

    const float alpha = g.alpha, beta = g.beta;
    // C values of this thread's outputs, loaded now (beta != 0) so that the
    // workgroup that finishes the band does not wait for them at the end.
    constexpr int PER = (T + NT - 1) / NT;
    float c_in[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int idx = tid + NT * i;
        const int row = m0 + idx / kBandCols, col = n0 + idx % kBandCols;
        c_in[i] = (beta != 0.0f && idx < T && row < M && col < N) ? g.C[(size_t)row * g.ldc + col] : 0.0f;
    }
    auto finish = [&](int i, int idx, float sum) {
        const int row = m0 + idx / kBandCols, col = n0 + idx % kBandCols;
        if (row < M && col < N) {
            const float o = alpha * sum;
            g.C[(size_t)row * g.ldc + col] = (beta != 0.0f) ? fmaf(beta, c_in[i], o) : o;
        }
    };

    if (S == 1) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = tid + NT * i;
            if (idx >= T) break;
            float sum = 0.0f;
#pragma unroll
            for (int v = 0; v < W; ++v) sum += red[v][idx];
            finish(i, idx, sum);
        }
        return;
    }

    // Partials are written and read with device-scope relaxed atomics, i.e.
    // stores written through to, and loads served from, the point where all
    // XCDs are coherent; each thread's stores have completed (s_waitcnt 0)
    // before the barrier that precedes the counter increment, and the last
    // workgroup only loads after it has seen the count. This avoids the
    // whole-L2 write-back and invalidate a device-scope fence costs here.
    float *part = sa.ws + ((size_t)tile * S + split) * T;
    for (int idx = tid; idx < T; idx += NT) {
        float sum = 0.0f;
#pragma unroll
        for (int v = 0; v < W; ++v) sum += red[v][idx];
        __hip_atomic_store(part + idx, sum, __ATOMIC_RELAXED, kExchangeScope);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
        is_last = __hip_atomic_fetch_add(&sa.counters[tile], 1, __ATOMIC_RELAXED, kExchangeScope) == S - 1;
    __syncthreads();
    if (!is_last) return;
    // The loads of eight splits, for all of this thread's outputs, are issued
    // before any of them is summed or stored (a store to C ahead of the next
    // output's loads would make those loads wait a round trip of their own);
    // each output's sum runs in split order.
    const float *parts = sa.ws + (size_t)tile * S * T;
    float sum[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) sum[i] = 0.0f;
    for (int sp0 = 0; sp0 < S; sp0 += 8) {
        float v[PER][8];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = tid + NT * i;
            const float *p = parts + (size_t)sp0 * T + idx;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[i][u] = (idx < T && sp0 + u < S)
                              ? __hip_atomic_load(p + (size_t)u * T, __ATOMIC_RELAXED, kExchangeScope)
                              : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < PER; ++i)
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (sp0 + u < S) sum[i] += v[i][u];
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int idx = tid + NT * i;
        if (idx < T) finish(i, idx, sum[i]);
    }
    if (tid == 0) __hip_atomic_store(&sa.counters[tile], 0, __ATOMIC_RELAXED, kExchangeScope);
}

__global__ __launch_bounds__(256) void zero_ints(int *p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0;
}

// C <- beta * C (beta == 0: C <- 0 without reading C), for alpha == 0 or K == 0.
__global__ __launch_bounds__(256) void scale_c(float *C, int M, int N, int ldc, float beta) {
    const int col = blockIdx.x * 256 + threadIdx.x;
    if (col >= N) return;
    for (int row = blockIdx.y; row < M; row += gridDim.y) {
        float *p = C + (size_t)row * ldc + col;
        *p = (beta == 0.0f) ? 0.0f : beta * *p;
    }
}

}  // namespace

#endif  // MISGEMM_SKINNY_KERNELS_H
