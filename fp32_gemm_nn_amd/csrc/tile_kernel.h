// The MFMA tile kernel sgemm_mfma32: MFMA fragments for 32 x 32 and 16 x 16
// blocks, instruction-order hints, and the kernel with its k-loop, k-group and
// split-K / stream-K reductions and epilogue.
// Internal to libmisgemm: compiled only as part of misgemm.hip, whose header comment
// describes the kernels and the configurations built from them.
#ifndef MISGEMM_TILE_KERNEL_H
#define MISGEMM_TILE_KERNEL_H

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <type_traits>

#include "tile_common.h"

namespace {

// MFMA operands of one q-group (four consecutive k-steps of a k-tile) for one
// wave: a[blk][e] and b[blk][e] feed step e of the 32x32x2 MFMA for block blk.
template <class CFG, bool TA, bool TB>
struct Frag {
    static constexpr int FM = CFG::FM, FN = CFG::FN, WTM = CFG::WTM, WTN = CFG::WTN, HB = CFG::BK / 2;
    float a[FM][4];
    float b[FN][4];

    // Float offset inside a k-contiguous LDS row of the lane's q-group: k =
    // lh*HB + 4q, at its swizzled chunk position in the DL layout (the row is
    // li plus a multiple of 8, so its swizzle depends on li alone).
    static __device__ __forceinline__ int kofs(int li, int lh, int q) {
        if constexpr (CFG::DL) {
            constexpr int CPR = CFG::BK / 4;
            return (((lh * HB + 4 * q) / 4) ^ (CPR >= 8 ? li & 7 : (li / 2) & 3)) * 4;
        } else {
            return lh * HB + 4 * q;
        }
    }

    // as/bs: LDS tiles of one k-tile, row strides AS/BS (lds0, the start of
    // the workgroup's LDS, is not needed by this layout).
    template <int AS, int BS>
    __device__ __forceinline__ void read(const float *, const float *as, const float *bs, int q, int wm, int wn,
                                         int li, int lh) {
        if (!TA) {
            // k-contiguous A tile [m][k]: block blk, lane row li is m = 32*blk + li.
#pragma unroll
            for (int blk = 0; blk < FM; ++blk)
                LdsVec<4>::get(as + (wm * WTM + 32 * blk + li) * AS + kofs(li, lh, q), a[blk]);
        } else {
            // m-contiguous A tile [k][m]: block blk, lane row li is m = FM*li + blk.
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float t[FM];
                LdsVec<FM>::get(as + (lh * HB + 4 * q + e) * AS + wm * WTM + FM * li, t);
#pragma unroll
                for (int blk = 0; blk < FM; ++blk) a[blk][e] = t[blk];
            }
        }
        if (TB) {
            // k-contiguous B tile [n][k]: block blk, lane column li is n = 32*blk + li.
#pragma unroll
            for (int blk = 0; blk < FN; ++blk)
                LdsVec<4>::get(bs + (wn * WTN + 32 * blk + li) * BS + kofs(li, lh, q), b[blk]);
        } else {
            // n-contiguous B tile [k][n]: block blk, lane column li is n = FN*li + blk.
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float t[FN];
                LdsVec<FN>::get(bs + (lh * HB + 4 * q + e) * BS + wn * WTN + FN * li, t);
#pragma unroll
                for (int blk = 0; blk < FN; ++blk) b[blk][e] = t[blk];
            }
        }
    }

    __device__ __forceinline__ void mma(f32x16 (&acc)[FM][FN]) const {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][e], b[j][e], acc[i][j], 0, 0, 0);
    }
};

// MFMA operands of one 16-deep q-group for one wave on 16 x 16 blocks:
// a[blk][s] and b[blk][s] feed step s of v_mfma_f32_16x16x4_f32. Lane (c, g)
// = (lane % 16, lane / 16) supplies row / column c of a block and, at step s,
// k = 16q + 4g + s (a k-permutation shared by both operands): one 16-byte
// read gives a k-contiguous operand's four steps. m/n-contiguous operands
// use the column permutation m = FM*c + block (n = FN*c + block), one read of
// FM (FN) adjacent floats per step.
template <class CFG, bool TA, bool TB>
struct Frag16 {
    static constexpr int FM = CFG::FM, FN = CFG::FN, WTM = CFG::WTM, WTN = CFG::WTN;
    static_assert(!TA || (FM >= 1 && FM <= 4), "one LdsVec read covers a row's FM blocks");
    static_assert(TB || (FN >= 1 && FN <= 4), "one LdsVec read covers a row's FN blocks");
    float a[FM][4];
    float b[FN][4];

    // Float offset of the lane's four k values inside a k-contiguous LDS row
    // (row c plus a multiple of 16), at its swizzled chunk position in the
    // unpadded layout.
    static __device__ __forceinline__ int kofs(int c, int g, int q) {
        if constexpr (CFG::SWZ) {
            return ((4 * q + g) ^ (c & 7)) * 4;
        } else {
            return 16 * q + 4 * g;
        }
    }

    // The lane's 16-byte k-run for q-group q in row `row` of a k-contiguous
    // tile. Swizzled rows are 32 floats per 8 chunks, and every tile buffer
    // starts a whole number of rows into `lds0`, so an odd q-group's run is
    // the even one's with float-offset bit 4 flipped: formed with one XOR at
    // the read rather than held as a second address across the k-loop (the
    // offset from lds0 includes the round's buffer, so it is not hoisted).
    // Rows 16 apart (the next block) keep the same chunk position, so adding
    // 16 rows after the flip is exact.
    template <int STRIDE>
    static __device__ __forceinline__ const float *krun(const float *lds0, const float *tile, int row, int c, int g,
                                                          int q) {
        if constexpr (CFG::SWZ) {
            static_assert(STRIDE % 32 == 0, "swizzled rows hold whole groups of 8 chunks");
            const float *p = tile + row * STRIDE + kofs(c, g, q & ~1);
            return (q & 1) ? lds0 + ((int)(p - lds0) ^ 16) : p;
        } else {
            return tile + row * STRIDE + kofs(c, g, q);
        }
    }

    // c, g: the lane's column and group (lane % 16, lane / 16); lds0: the
    // start of the workgroup's LDS, which the tiles lie in.
    template <int AS, int BS>
    __device__ __forceinline__ void read(const float *lds0, const float *as, const float *bs, int q, int wm, int wn,
                                         int c, int g) {
        const int k0 = 16 * q + 4 * g;
        if (!TA) {
            // Blocks are 16 rows apart: one address, immediate offsets.
            const float *pa = krun<AS>(lds0, as, wm * WTM + c, c, g, q);
#pragma unroll
            for (int blk = 0; blk < FM; ++blk) LdsVec<4>::get(pa + 16 * blk * AS, a[blk]);
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                float t[FM];
                LdsVec<FM>::get(as + (k0 + s) * AS + wm * WTM + FM * c, t);
#pragma unroll
                for (int blk = 0; blk < FM; ++blk) a[blk][s] = t[blk];
            }
        }
        if (TB) {
            const float *pb = krun<BS>(lds0, bs, wn * WTN + c, c, g, q);
#pragma unroll
            for (int blk = 0; blk < FN; ++blk) LdsVec<4>::get(pb + 16 * blk * BS, b[blk]);
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                float t[FN];
                LdsVec<FN>::get(bs + (k0 + s) * BS + wn * WTN + FN * c, t);
#pragma unroll
                for (int blk = 0; blk < FN; ++blk) b[blk][s] = t[blk];
            }
        }
    }

    __device__ __forceinline__ void mma(f32x4 (&acc)[FM][FN]) const {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][s], b[j][s], acc[i][j], 0, 0, 0);
    }
};

// Instruction-order hints for the straight-line k-tile iteration (one
// scheduling region ending at the barrier): the next tile's global loads are
// spread over the first MFMAs, each q-group's fragment reads for the next
// group over the MFMAs of the current one, and the LDS writes of the next
// tile over the last group. Masks: 0x008 MFMA, 0x020 VMEM read, 0x100 DS read,
// 0x200 DS write.
template <int MASK, int N>
__device__ __forceinline__ void hint_pairs() {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(MASK, 1, 0);
    }
}

// Global loads of the next tile per q-group: all in the first group when they
// fit beside its fragment reads, else spread over the groups before the last.
template <int MFMA_PER_Q, int Q, int GLOADS, int DSREADS>
constexpr int gloads_in_group(int q) {
    if (GLOADS + DSREADS <= MFMA_PER_Q) return q == 0 ? GLOADS : 0;
    const int per = (GLOADS + Q - 2) / (Q - 1);
    const int before = per * q;
    if (q >= Q - 1 || before >= GLOADS) return 0;
    return GLOADS - before < per ? GLOADS - before : per;
}

template <int MFMA_PER_Q, int Q, int GLOADS, int DSREADS, int DSWRITES>
constexpr bool hints_fit() {
    if (DSWRITES > MFMA_PER_Q || Q < 2) return false;
    for (int q = 0; q + 1 < Q; ++q)
        if (gloads_in_group<MFMA_PER_Q, Q, GLOADS, DSREADS>(q) + DSREADS > MFMA_PER_Q) return false;
    int total = 0;
    for (int q = 0; q < Q; ++q) total += gloads_in_group<MFMA_PER_Q, Q, GLOADS, DSREADS>(q);
    return total == GLOADS;
}

template <int MFMA_PER_Q, int Q, int GLOADS, int DSREADS, int DSWRITES, int q = 0>
__device__ __forceinline__ void schedule_iteration() {
    if constexpr (hints_fit<MFMA_PER_Q, Q, GLOADS, DSREADS, DSWRITES>() && q < Q) {
        constexpr int gl = gloads_in_group<MFMA_PER_Q, Q, GLOADS, DSREADS>(q);
        constexpr int dr = q + 1 < Q ? DSREADS : 0;
        constexpr int dw = q + 1 < Q ? 0 : DSWRITES;
        hint_pairs<0x020, gl>();
        hint_pairs<0x100, dr>();
        hint_pairs<0x200, dw>();
        __builtin_amdgcn_sched_group_barrier(0x008, MFMA_PER_Q - gl - dr - dw, 0);
        schedule_iteration<MFMA_PER_Q, Q, GLOADS, DSREADS, DSWRITES, q + 1>();
    }
}

// Register-staged tiles up to 256 x 128, and the 192 x 192 tile, fetch every
// complete k-tile with clamped loads, so edge tiles keep the straight-line
// rounds (the 256 x 256 tile has no registers to spare for the clamped
// offsets).
template <class CFG>
constexpr bool kClampEdge = !CFG::DL && CFG::BM * CFG::BN <= 192 * 192;

// SCALAR: the instantiation launched when A or B cannot be read with 16-byte
// loads (pointer or leading dimension not a multiple of 4 floats); its
// straight-line rounds fetch with clamped 4-byte loads. A separate kernel, so
// that the 16-byte path keeps its own register allocation.
template <class CFG, bool TA, bool TB, bool SCALAR = false>
__global__ __launch_bounds__(CFG::NT) __attribute__((amdgpu_waves_per_eu(CFG::WAVES_PER_EU)))
void sgemm_mfma32(GemmArgs g) {
    static_assert(!SCALAR || kClampEdge<CFG>, "only clamping tiles have a 4-byte straight-line path");
    constexpr int BM = CFG::BM, BN = CFG::BN, BK = CFG::BK, NTG = CFG::NTG, KG = CFG::KG;
    constexpr int FM = CFG::FM, FN = CFG::FN, WTM = CFG::WTM, WTN = CFG::WTN;
    constexpr int Q = BK / CFG::QK;             // q-groups per k-tile
    constexpr int AR = CFG::ACC_REGS, MBLK = CFG::MBLK;
    using AccT = std::conditional_t<CFG::MI16, f32x4, f32x16>;
    static_assert(Q % 2 == 0, "fragment buffers alternate, so the q-group count must be even");
    // Stored tile shapes: A is BM x BK ('N', k contiguous) or BK x BM ('T',
    // m contiguous); B is BK x BN ('N', n contiguous) or BN x BK ('T').
    using ACopy = TileCopy<TA ? BK : BM, TA ? BM : BK, NTG, CFG::DL, CFG::SWZ && !TA, CFG::SWZ>;
    using BCopy = TileCopy<TB ? BN : BK, TB ? BK : BN, NTG, CFG::DL, CFG::SWZ && TB, CFG::SWZ>;
    using F = std::conditional_t<CFG::MI16, Frag16<CFG, TA, TB>, Frag<CFG, TA, TB>>;
    constexpr int A_FLOATS = ACopy::LDS_FLOATS, B_FLOATS = BCopy::LDS_FLOATS;
    constexpr int AS = ACopy::STRIDE, BS = BCopy::STRIDE;
    constexpr int GROUP_FLOATS = 2 * (A_FLOATS + B_FLOATS);
    // The k-group reduction reuses the tile buffers: KG groups x waves x
    // FM*FN accumulator blocks x AR registers x 64 lanes.
    constexpr int RED_FLOATS = KG > 1 ? KG * (NTG / 64) * FM * FN * AR * 64 : 0;
    static_assert(RED_FLOATS <= KG * GROUP_FLOATS, "reduction does not fit the tile buffers");

    __shared__ __attribute__((aligned(16))) float lds[KG * GROUP_FLOATS];

    __shared__ int is_last;
    const int ktiles = (g.K + BK - 1) / BK;

    // Tile (tm, tn), k-tiles [kt_begin, kt_end), into C; or, when sg.nseg > 1,
    // into a partial block that the last of the tile's segments to finish
    // adds up in segment order before the epilogue.
    auto run_tile = [&](const int tm, const int tn, const int kt_begin, const int kt_end, const SegInfo &sg) {
        // Thread coordinates. A stream-K workgroup walks several tiles: the
        // empty asm makes the thread id opaque per tile, so the addresses
        // derived from it are recomputed per tile instead of being hoisted
        // out of the tile loop and held live across every k-loop.
        int tid = threadIdx.x;
        if constexpr (CFG::STREAMK) asm volatile("" : "+v"(tid));
        // The k-group and the wave are the same for every lane of a wave:
        // read from the first lane, they live in scalar registers, so the
        // k-loop's trip count and the per-wave offsets are scalar too.
        const int grp = KG == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid / NTG);   // k-group
        const int gtid = KG == 1 ? tid : tid % NTG;                                // thread within it
        const int lane = gtid & 63, wave = __builtin_amdgcn_readfirstlane(gtid >> 6);
        // Lane column and group: (lane % 32, lane / 32) for 32 x 32 blocks,
        // (lane % 16, lane / 16) for 16 x 16 blocks.
        const int li = CFG::MI16 ? (lane & 15) : (lane & 31), lh = CFG::MI16 ? (lane >> 4) : (lane >> 5);
        const int wm = wave / CFG::WAVES_N, wn = wave % CFG::WAVES_N;
        // This group's buffer i of A at a_lds + i*A_FLOATS, of B at b_lds + i*B_FLOATS.
        float *const a_lds = lds + grp * GROUP_FLOATS;
        float *const b_lds = a_lds + 2 * A_FLOATS;
        const int m0 = tm * BM, n0 = tn * BN;
        const int M = g.M, N = g.N, K = g.K;
        const bool vec = g.vec_ab != 0;
        // Interior workgroup: every complete k-tile can be fetched unguarded.
        // Clamping tiles take the straight-line rounds for edge tiles too, and
        // their SCALAR instantiation for any alignment.
        const bool interior = (m0 + BM <= M) && (n0 + BN <= N);
        constexpr bool CLAMP_EDGE = kClampEdge<CFG>;
        const bool wg_fast = SCALAR || (vec && (interior || CLAMP_EDGE));
        const int kfull = K / BK;
        const int kfast_end = min(kfull, kt_end);
        const int rounds = kt_end > kt_begin ? (kt_end - kt_begin + KG - 1) / KG : 0;

        // Base of the tile at k = 0 in each stored matrix, and the per-k-tile step.
        const float *a_ptr = TA ? g.A + m0 : g.A + (size_t)m0 * g.lda;
        const float *b_ptr = TB ? g.B + (size_t)n0 * g.ldb : g.B + n0;
        const size_t a_step = TA ? (size_t)BK * g.lda : (size_t)BK;
        const size_t b_step = TB ? (size_t)BK : (size_t)BK * g.ldb;
        const int a_rows = TA ? K : M - m0, a_cols = TA ? M - m0 : K;
        const int b_rows = TB ? N - n0 : K, b_cols = TB ? K : N - n0;

        ACopy ca;
        BCopy cb;
        // A complete k-tile (kt < kfull) of a wg_fast workgroup: unguarded
        // loads, clamped at the M and N edges (the k extent is whole). The
        // clamps do nothing in an interior tile and are loop-invariant, so the
        // straight-line rounds carry no branch.
        auto fetch_fast = [&](int kt) {
            if constexpr (CLAMP_EDGE) {
                ca.template load_clamped<!SCALAR>(a_ptr + kt * a_step, g.lda, TA ? BK : a_rows, TA ? a_cols : BK,
                                                  gtid);
                cb.template load_clamped<!SCALAR>(b_ptr + kt * b_step, g.ldb, TB ? b_rows : BK, TB ? BK : b_cols,
                                                  gtid);
            } else {
                ca.load(a_ptr + kt * a_step, g.lda, 0, 0, false, true, gtid);
                cb.load(b_ptr + kt * b_step, g.ldb, 0, 0, false, true, gtid);
            }
        };
        auto fetch_any = [&](int kt) {
            if constexpr (CLAMP_EDGE) {
                if (wg_fast && kt < kfull) {
                    fetch_fast(kt);
                    return;
                }
                if (wg_fast) {
                    // The k tail (kt == kfull, K not a multiple of BK): clamped
                    // loads with the elements past K zeroed. The thread id is
                    // made opaque so that these addresses are formed here
                    // rather than held through the k-loop.
                    int ltid = gtid;
                    asm volatile("" : "+v"(ltid));
                    const int kleft = K - kt * BK;
                    ca.template load_ktail<!SCALAR, TA>(a_ptr + kt * a_step, g.lda, TA ? kleft : a_rows,
                                                        TA ? a_cols : kleft, ltid);
                    cb.template load_ktail<!SCALAR, !TB>(b_ptr + kt * b_step, g.ldb, TB ? b_rows : kleft,
                                                         TB ? kleft : b_cols, ltid);
                    return;
                }
            }
            const int k0 = kt * BK;
            // Complete k-tiles of interior workgroups unguarded (the only ones
            // left fast without edge clamping), the rest guarded. Rows/cols
            // left counted from this k-tile's origin.
            const bool guard = CLAMP_EDGE || !(wg_fast && kt < kfull);
            // Tiles that clamp their edges reach this only when their operands
            // allow no 16-byte loads and they have no 4-byte straight-line
            // form: with the thread id made opaque here its element addresses
            // are formed when needed instead of being held through the k-loop.
            int ltid = gtid;
            if constexpr (CLAMP_EDGE) asm volatile("" : "+v"(ltid));
            ca.load(a_ptr + kt * a_step, g.lda, TA ? a_rows - k0 : a_rows, TA ? a_cols : a_cols - k0, guard,
                    vec, ltid);
            cb.load(b_ptr + kt * b_step, g.ldb, TB ? b_rows : b_rows - k0, TB ? b_cols - k0 : b_cols, guard,
                    vec, ltid);
        };

        AccT acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < AR; ++r) acc[i][j][r] = 0.0f;

        F f0, f1;
        // Group grp takes k-tiles kt_begin + grp, + KG, ... In round r its k-tile
        // is t = kt_begin + r*KG + grp. Invariant at the top of round r: the
        // group's LDS buffer r&1 holds k-tile t (when t < kt_end) and f0 holds
        // its q-group 0.
        if (kt_begin + grp < kt_end) {
            fetch_any(kt_begin + grp);
            ca.store(a_lds, gtid);
            cb.store(b_lds, gtid);
        }
        __syncthreads();
        if (kt_begin + grp < kt_end) f0.template read<AS, BS>(lds, a_lds, b_lds, 0, wm, wn, li, lh);

        // Straight-line rounds (this and the next k-tile complete and in
        // range) first, then the guarded ones, as two loops; the condition
        // holds for a prefix of the rounds, and both kinds end on one barrier.
        int r = 0;
        if (wg_fast) {
            for (; kt_begin + (r + 1) * KG + grp < kfast_end; ++r) {
                const int cur = r & 1, nxt = cur ^ 1;
                const float *as = a_lds + cur * A_FLOATS;
                const float *bs = b_lds + cur * B_FLOATS;
                float *as_n = a_lds + nxt * A_FLOATS;
                float *bs_n = b_lds + nxt * B_FLOATS;
                const int kt_next = kt_begin + (r + 1) * KG + grp;
                if constexpr (CFG::DL) {
                    // The other buffer was last read before the previous
                    // round's barrier, so the next tile can land in it now.
                    ca.load_direct(a_ptr + kt_next * a_step, g.lda, as_n, gtid);
                    cb.load_direct(b_ptr + kt_next * b_step, g.ldb, bs_n, gtid);
                    asm volatile("" ::: "memory");
                } else {
                    fetch_fast(kt_next);
                }
#pragma unroll
                for (int q = 0; q < Q; q += 2) {
                    f1.template read<AS, BS>(lds, as, bs, q + 1, wm, wn, li, lh);
                    f0.mma(acc);
                    if (q + 2 < Q) {
                        f0.template read<AS, BS>(lds, as, bs, q + 2, wm, wn, li, lh);
                    } else if constexpr (!CFG::DL) {
                        ca.store(as_n, gtid);
                        cb.store(bs_n, gtid);
                    }
                    f1.mma(acc);
                }
                // DS reads per q-group: FM (or FN) 16-byte reads of a k-contiguous
                // tile, four narrow reads of an m/n-contiguous one. Direct loads
                // are issued before the round's first reads and leave no writes.
                // A 4-byte fetch issues four loads per chunk.
                constexpr int COPIES = CFG::DL ? 0 : ACopy::PER_THREAD + BCopy::PER_THREAD;
                schedule_iteration<4 * FM * FN, Q, SCALAR ? 4 * COPIES : COPIES, (TA ? 4 : FM) + (TB ? FN : 4),
                                   COPIES>();
                // Direct loads complete (vmcnt) before the barrier publishes them.
                if constexpr (CFG::DL) __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                f0.template read<AS, BS>(lds, as_n, bs_n, 0, wm, wn, li, lh);
            }
        }
        for (; r < rounds; ++r) {
            const int t = kt_begin + r * KG + grp, tn_ = t + KG;
            const int cur = r & 1, nxt = cur ^ 1;
            const float *as = a_lds + cur * A_FLOATS;
            const float *bs = b_lds + cur * B_FLOATS;
            float *as_n = a_lds + nxt * A_FLOATS;
            float *bs_n = b_lds + nxt * B_FLOATS;
            const bool has_cur = t < kt_end, has_next = tn_ < kt_end;
            if (has_next) fetch_any(tn_);
            if (has_cur) {
#pragma unroll
                for (int q = 0; q < Q; q += 2) {
                    f1.template read<AS, BS>(lds, as, bs, q + 1, wm, wn, li, lh);
                    f0.mma(acc);
                    if (q + 2 < Q) f0.template read<AS, BS>(lds, as, bs, q + 2, wm, wn, li, lh);
                    f1.mma(acc);
                }
            }
            if (has_next) {
                ca.store(as_n, gtid);
                cb.store(bs_n, gtid);
            }
            __syncthreads();
            if (has_next) f0.template read<AS, BS>(lds, as_n, bs_n, 0, wm, wn, li, lh);
        }

        // k-groups without a split: every group writes its accumulators to LDS
        // (the tile buffers are free after the last barrier), and group g then
        // sums accumulator registers r = g, g + KG, ... of all KG groups, in
        // group order (the same sum, in the same order, on every call), and
        // stores those outputs; the reduction and the stores are shared by all
        // the workgroup's waves.
        static_assert(KG == 1 || AR % KG == 0, "k-groups split the accumulator registers evenly");
        if constexpr (KG > 1 && !CFG::SPLIT) {
            constexpr int WAVES = NTG / 64;
            constexpr int BLOCKS = FM * FN;
            // Register r of block b of wave w of group s at ((s*WAVES + w)*AR + r)*BLOCKS + b, times 64 lanes.
            float *mine = lds + (grp * WAVES + wave) * AR * BLOCKS * 64 + lane;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < AR; ++r) mine[(r * BLOCKS + i * FN + j) * 64] = acc[i][j][r];
            __syncthreads();
#pragma unroll
            for (int r = 0; r < AR; ++r) {
                if (r % KG != grp) continue;
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const float *src = lds + wave * AR * BLOCKS * 64 + lane + (r * BLOCKS + i * FN + j) * 64;
                        float sum = src[0];
#pragma unroll
                        for (int s2 = 1; s2 < KG; ++s2) sum += src[s2 * WAVES * AR * BLOCKS * 64];
                        acc[i][j][r] = sum;
                    }
            }
        } else if constexpr (KG > 1) {
            // With a split, group 0 takes the partial block on: groups 1..KG-1
            // hand their accumulators to it, and it adds them in group order.
            constexpr int SLOT = FM * FN * AR * 64;            // floats per wave
            constexpr int WAVES = NTG / 64;
            if (grp > 0) {
                float *dst = lds + ((grp - 1) * WAVES + wave) * SLOT + lane;
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int r = 0; r < AR; ++r) dst[((i * FN + j) * AR + r) * 64] = acc[i][j][r];
            }
            __syncthreads();
            if (grp == 0)
#pragma unroll
            for (int g2 = 1; g2 < KG; ++g2) {
                const float *src = lds + ((g2 - 1) * WAVES + wave) * SLOT + lane;
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int r = 0; r < AR; ++r) acc[i][j][r] += src[((i * FN + j) * AR + r) * 64];
            }
        }

        if constexpr (CFG::SPLIT || CFG::STREAMK) if (sg.nseg > 1) {
            // Split-K over workgroups: store this partial tile (group 0's
            // accumulators, in register order) to the workspace with device-scope
            // stores, count in, and let the workgroup that completes the count sum
            // the partials in split order before the epilogue. Same protocol as the
            // skinny band kernel; every wave of the workgroup reaches each barrier.
            constexpr int REGS = FM * FN * AR;
            constexpr size_t PART = (size_t)BM * BN;
            const int S = sg.nseg;
            const size_t tile_id = (size_t)sg.counter;
            float *mine = g.ws + (size_t)sg.slot(sg.seg) * PART + (size_t)wave * REGS * 64 + lane;
            if (grp == 0) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int r = 0; r < AR; ++r)
                            __hip_atomic_store(mine + ((i * FN + j) * AR + r) * 64, acc[i][j][r], __ATOMIC_RELAXED,
                                               kExchangeScope);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (tid == 0)
                is_last = __hip_atomic_fetch_add(&g.counters[tile_id], 1, __ATOMIC_RELAXED, kExchangeScope) ==
                          S - 1;
            __syncthreads();
            if (!is_last) return;
            const float *base = g.ws + (size_t)wave * REGS * 64 + lane;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < AR; ++r) acc[i][j][r] = 0.0f;
            // SB splits' loads in flight at a time (about 64 registers); the sum
            // runs in split order.
            constexpr int SB = (REGS >= 64 || CFG::WAVES_PER_EU > 2) ? 1 : 64 / REGS;
            for (int sp0 = 0; sp0 < S; sp0 += SB) {
                float v[SB][FM][FN][AR];
#pragma unroll
                for (int u = 0; u < SB; ++u)
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j)
#pragma unroll
                            for (int r = 0; r < AR; ++r)
                                v[u][i][j][r] = (grp == 0 && sp0 + u < S)
                                                    ? __hip_atomic_load(base + (size_t)sg.slot(sp0 + u) * PART +
                                                                            ((i * FN + j) * AR + r) * 64,
                                                                        __ATOMIC_RELAXED, kExchangeScope)
                                                    : 0.0f;
#pragma unroll
                for (int u = 0; u < SB; ++u)
                    if (sp0 + u < S)
#pragma unroll
                        for (int i = 0; i < FM; ++i)
#pragma unroll
                            for (int j = 0; j < FN; ++j)
#pragma unroll
                                for (int r = 0; r < AR; ++r) acc[i][j][r] += v[u][i][j][r];
            }
            if (tid == 0) __hip_atomic_store(&g.counters[tile_id], 0, __ATOMIC_RELAXED, kExchangeScope);
        }
        if (CFG::SPLIT && grp > 0) return;

        // Epilogue. Accumulator element r of block (i, j) in lane (li, lh) is
        // block row 8*(r/4) + 4*lh + r%4 (32 x 32 blocks) or 4*lh + r (16 x 16
        // blocks), block column li. With k-groups and no split, group g stores
        // the registers r = g (mod KG) it has summed.
        const float alpha = g.alpha, beta = g.beta;
        float *const cw = g.C + (size_t)(m0 + wm * WTM) * g.ldc + (n0 + wn * WTN);
        const int rows_left = M - (m0 + wm * WTM), cols_left = N - (n0 + wn * WTN);
        const int ldc = g.ldc;
        // k-group tiles (a quarter or half of the row runs (i, r) per lane)
        // and the 256 x 256 tiles (one tile per CU; batching measured no
        // faster there) store run by run, reading C with each store where
        // beta != 0.
        constexpr bool RUN_BY_RUN = (KG > 1 && !CFG::SPLIT) || CFG::BM * CFG::BN >= 256 * 256;
        // Staged through LDS (B transposed): every wave's block, unpadded,
        // within the tile buffers.
        constexpr bool STAGE_C = TB && !RUN_BY_RUN && KG == 1 && (NTG / 64) * WTM * WTN <= GROUP_FLOATS &&
                                 (WTM * WTN) % 256 == 0 && WTN % 32 == 0;
        if constexpr (RUN_BY_RUN) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
#pragma unroll
                for (int r = 0; r < AR; ++r) {
                    if constexpr (KG > 1 && !CFG::SPLIT)
                        if (r % KG != grp) continue;
                    const int ib = CFG::MI16 ? 4 * lh + r : 8 * (r / 4) + 4 * lh + (r % 4);
                    const int row = TA ? FM * ib + i : MBLK * i + ib;
                    if (row >= rows_left) continue;
                    float *crow = cw + (size_t)row * ldc;
                    if (!TB) {
                        const int col = FN * li;
                        float out[FN];
#pragma unroll
                        for (int j = 0; j < FN; ++j) out[j] = alpha * acc[i][j][r];
                        store_run<FN>(crow + col, out, beta, g.vec_c && col + FN <= cols_left, cols_left - col);
                    } else {
#pragma unroll
                        for (int j = 0; j < FN; ++j) {
                            const int col = MBLK * j + li;
                            if (col < cols_left) {
                                float *p = crow + col;
                                const float o = alpha * acc[i][j][r];
                                *p = (beta != 0.0f) ? fmaf(beta, *p, o) : o;
                            }
                        }
                    }
                }
            }
        } else {
            // B transposed and C read (beta != 0): a lane's FN outputs of a row
            // sit MBLK columns apart and would be loaded and stored as 4-byte
            // accesses. Each wave writes its block to its own part of the tile
            // buffers (free once the k-loop has ended on a barrier), reads it
            // back as rows of 16-byte runs, loads all of its C runs, and stores
            // the runs, 256 contiguous bytes per 16 lanes. (With beta == 0 the
            // staging costs more than the 4-byte stores: 2048^3 NT 132.7 vs
            // 130.4 us.)
            bool staged = false;
            if constexpr (STAGE_C) {
                if (beta != 0.0f) {
                    constexpr int RUNS4 = WTM * WTN / 256;    // 16-byte runs per lane
                    // The 16-float halves of each 32-column group swap places on
                    // rows whose bit SH is set: the four rows one write instruction
                    // covers (4*lh apart, or 4*FM*lh with A transposed) then fall on
                    // both halves of the banks, and a 16-byte run never straddles a
                    // half.
                    constexpr int SH = TA ? (FM == 1 ? 2 : (FM == 2 ? 3 : 4)) : 2;
                    auto sidx = [&](int row, int col) { return row * WTN + (col ^ (((row >> SH) & 1) << 4)); };
                    float *st = lds + wave * WTM * WTN;
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int r = 0; r < AR; ++r) {
                            const int ib = CFG::MI16 ? 4 * lh + r : 8 * (r / 4) + 4 * lh + (r % 4);
                            const int row = TA ? FM * ib + i : MBLK * i + ib;
#pragma unroll
                            for (int j = 0; j < FN; ++j) st[sidx(row, MBLK * j + li)] = acc[i][j][r];
                        }
                    __syncthreads();
                    float out[RUNS4][4], cin[RUNS4][4];
#pragma unroll
                    for (int u = 0; u < RUNS4; ++u) {
                        const int flat = (u * 64 + lane) * 4, row = flat / WTN, col = flat % WTN;
                        LdsVec<4>::get(st + sidx(row, col), out[u]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            out[u][e] *= alpha;
                            cin[u][e] = 0.0f;
                        }
                        if (row < rows_left)
                            load_run<4>(cw + (size_t)row * ldc + col, cin[u], g.vec_c && col + 4 <= cols_left,
                                        cols_left - col);
                    }
#pragma unroll
                    for (int u = 0; u < RUNS4; ++u) {
                        const int flat = (u * 64 + lane) * 4, row = flat / WTN, col = flat % WTN;
                        if (row < rows_left)
                            put_run<4>(cw + (size_t)row * ldc + col, out[u], cin[u], beta,
                                       g.vec_c && col + 4 <= cols_left, cols_left - col);
                    }
                    // A stream-K workgroup's next tile writes the tile buffers next.
                    if constexpr (CFG::STREAMK) __syncthreads();
                    staged = true;
                }
            }
            if (!staged) {
                // Row runs (i, r) are stored in turn when C is not read (beta ==
                // 0). When it is, they go in batches of up to 32 values, and every
                // C load of a batch is issued before the batch's first store, so
                // the loads wait once, together. (Loaded and stored run by run,
                // each load would wait for the store before it: nothing tells the
                // compiler that the rows do not overlap.)
                constexpr int RUNS = FM * AR;
                constexpr int BATCH = 32 / FN < 1 ? 1 : (32 / FN > RUNS ? RUNS : 32 / FN);
                // !TB: FN adjacent columns FN*li .. FN*li + FN-1; TB: columns MBLK*j + li.
                const int col0 = FN * li;
                const bool whole = g.vec_c && col0 + FN <= cols_left;
                // Output row of run (i, r) within the wave's block, or -1 beyond M.
                auto run_row = [&](int i, int r) {
                    const int ib = CFG::MI16 ? 4 * lh + r : 8 * (r / 4) + 4 * lh + (r % 4);
                    const int row = TA ? FM * ib + i : MBLK * i + ib;
                    return row < rows_left ? row : -1;
                };
                // Run (i, r) from acc and cin (C's values there; unused when beta == 0).
                auto put = [&](int i, int r, int row, const float (&cin)[FN]) {
                    float *crow = cw + (size_t)row * ldc;
                    if (!TB) {
                        float out[FN];
#pragma unroll
                        for (int j = 0; j < FN; ++j) out[j] = alpha * acc[i][j][r];
                        put_run<FN>(crow + col0, out, cin, beta, whole, cols_left - col0);
                    } else {
#pragma unroll
                        for (int j = 0; j < FN; ++j) {
                            const int col = MBLK * j + li;
                            if (col < cols_left) {
                                const float o = alpha * acc[i][j][r];
                                crow[col] = beta != 0.0f ? fmaf(beta, cin[j], o) : o;
                            }
                        }
                    }
                };
                if (beta == 0.0f) {
                    float none[FN];
#pragma unroll
                    for (int j = 0; j < FN; ++j) none[j] = 0.0f;
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int r = 0; r < AR; ++r) {
                            const int row = run_row(i, r);
                            if (row >= 0) put(i, r, row, none);
                        }
                } else {
#pragma unroll
                    for (int b0 = 0; b0 < RUNS; b0 += BATCH) {
                        float cin[BATCH][FN];
#pragma unroll
                        for (int u = 0; u < BATCH; ++u) {
#pragma unroll
                            for (int j = 0; j < FN; ++j) cin[u][j] = 0.0f;
                            if (b0 + u >= RUNS) continue;
                            const int row = run_row((b0 + u) / AR, (b0 + u) % AR);
                            if (row < 0) continue;
                            const float *crow = cw + (size_t)row * ldc;
                            if (!TB) {
                                load_run<FN>(crow + col0, cin[u], whole, cols_left - col0);
                            } else {
#pragma unroll
                                for (int j = 0; j < FN; ++j) {
                                    const int col = MBLK * j + li;
                                    if (col < cols_left) cin[u][j] = crow[col];
                                }
                            }
                        }
#pragma unroll
                        for (int u = 0; u < BATCH; ++u) {
                            if (b0 + u >= RUNS) continue;
                            const int row = run_row((b0 + u) / AR, (b0 + u) % AR);
                            if (row >= 0) put((b0 + u) / AR, (b0 + u) % AR, row, cin[u]);
                        }
                    }
                }
            }
        }
    };

    if constexpr (CFG::STREAMK) {
        static_assert(KG == 1 && !CFG::SPLIT, "stream-K runs one k-group");
        // The first sk_tiles tiles (fewer than the grid) are shared out:
        // iteration i is k-tile i % ktiles of tile i / ktiles (tiles in the
        // grouped order), and workgroup w owns [start(w), start(w+1));
        // workgroups on one XCD own consecutive shares. The rest, whole waves of
        // the grid, follow whole, one per workgroup per wave.
        // A tile cut between workgroups w0..w1 has one segment per workgroup.
        // Workgroup w keeps the partial of its first tile in slot 2w and of
        // its last in slot 2w+1; segment j > 0 of a tile always starts its
        // workgroup's share, so its slot is 2(w0+j).
        const long long G = gridDim.x;
        const int tiles = g.tiles_m * g.tiles_n, sk_tiles = tiles - g.sk_dp_tiles;
        const long long total = (long long)sk_tiles * ktiles;
        auto start = [&](long long w) { return w * total / G; };
        auto owner = [&](long long i) { return ((i + 1) * G + total - 1) / total - 1; };
        const int w = xcd_logical();
        long long it = start(w);
        const long long it_end = start(w + 1);
        while (it < it_end) {
            const int t = (int)(it / ktiles);
            const long long t0 = (long long)t * ktiles;
            const int kb = (int)(it - t0);
            const int ke = (int)min((long long)ktiles, kb + (it_end - it));
            SegInfo sg;
            sg.counter = t;
            sg.sstep = 2;
            if (kb == 0 && ke == ktiles) {
                sg.nseg = 1;
                sg.seg = 0;
                sg.s0 = sg.sbase = 0;
            } else {
                const int w0 = (int)owner(t0), w1 = (int)owner(t0 + ktiles - 1);
                sg.nseg = w1 - w0 + 1;
                sg.seg = w - w0;
                sg.sbase = 2 * w0;
                sg.s0 = 2 * w0 + (start(w0) < t0 ? 1 : 0);
            }
            int tm, tn;
            tile_of(t, g.tiles_m, g.tiles_n, tm, tn);
            run_tile(tm, tn, kb, ke, sg);
            it += ke - kb;
        }
        // Whole tiles, one per workgroup per wave: the workgroups of a wave
        // sweep k together, so the A and B panels they share stay in L2.
        for (int t = sk_tiles + w; t < tiles; t += (int)G) {
            SegInfo sg;
            sg.counter = t;
            sg.nseg = 1;
            sg.seg = 0;
            sg.s0 = sg.sbase = 0;
            sg.sstep = 2;
            int tm, tn;
            tile_of(t, g.tiles_m, g.tiles_n, tm, tn);
            run_tile(tm, tn, 0, ktiles, sg);
        }
    } else {
        int tm, tn, split;
        tile_coords(g.tiles_m, g.tiles_n, CFG::SPLIT ? g.splits : 1, tm, tn, split);
        SegInfo sg;
        sg.nseg = CFG::SPLIT ? g.splits : 1;
        sg.seg = split;
        sg.counter = tm * g.tiles_n + tn;
        sg.s0 = sg.sbase = sg.counter * sg.nseg;
        sg.sstep = 1;
        const int kt_begin = CFG::SPLIT ? split * g.kt_per_split : 0;
        const int kt_end = CFG::SPLIT ? min(ktiles, kt_begin + g.kt_per_split) : ktiles;
        run_tile(tm, tn, kt_begin, kt_end, sg);
    }
}

}  // namespace

#endif  // MISGEMM_TILE_KERNEL_H
