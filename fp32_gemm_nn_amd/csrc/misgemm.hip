// misgemm -- FP32 SGEMM on CDNA4 (gfx950) matrix cores, behind a C ABI.
//
// C = alpha*op(A)*op(B) + beta*C, row-major, op in {N, T}: the BLAS SGEMM of
// the itan.pw RTX 4090 SGEMM page (overview), with the row-major sum of the
// problem definition of "【CUDA】Sgemm单精度矩阵乘法" (klklkl10086.github.io).
//
// Kernel shape (one workgroup per BM x BN tile of C):
//   * The k range is walked in BK-wide tiles. Each tile of op(A) (BM x BK) and
//     op(B) (BK x BN) is fetched with 16-byte global loads along whichever
//     axis is contiguous in memory and stored unchanged into one of two LDS
//     buffers, so one barrier per k-tile suffices (the double buffering of the
//     itan.pw page, sections 3.6-3.7: the write-after-read barrier goes away
//     when consecutive tiles live in different buffers). The next tile's
//     global loads are issued before the current tile's matrix instructions.
//   * Each wave owns a (BM/WAVES_M) x (BN/WAVES_N) block of C held in
//     accumulator registers as FM x FN blocks of 32 x 32 (the register tile of
//     the same page, section 3.4, moved onto the matrix cores), and issues
//     v_mfma_f32_32x32x2_f32: full FP32 inputs, products and sums. MI16
//     configurations hold 16 x 16 blocks instead and issue
//     v_mfma_f32_16x16x4_f32 (see Frag16).
//   * k-permutation: inside a k-tile, the two 32-lane halves of a wave feed the
//     MFMA's two k slots from the two halves of the tile (slot h of step s is
//     k = h*BK/2 + s). Any permutation of k applied to both operands only
//     reorders the sum, and this one makes each lane's successive k values
//     adjacent, so one ds_read_b128 feeds four MFMAs from a k-contiguous LDS
//     tile -- the role played by the transposed A tile of section 3.5.
//   * Operands whose contiguous axis is m or n (A transposed, B not
//     transposed) stay m/n-contiguous in LDS. For those, MFMA block b of a wave
//     takes columns FN*c + b (c = lane column), so one ds_read of FN adjacent
//     floats serves all FN blocks at once, and each lane ends up holding FN
//     adjacent outputs of a row, which the epilogue stores as one vector.
//   * LDS rows are padded by 4 floats (the padding remedy of section 3.8); the
//     16-byte reads of the k-contiguous tiles are then bank-conflict free.
//   * Edges: a workgroup whose tile, or whose current k-tile, crosses M, N or
//     K takes a guarded load path that reads only in-range elements and
//     selects zero for the rest (the zero-fill of the klklkl10086 page,
//     01-Shared Memory Tiling); stores are masked to i < M, j < N.
//   * Epilogue: C = alpha*acc + beta*C fused into the store (itan.pw page,
//     sections 3.4-3.5); when beta == 0, C is not read.
//   * Workgroup order: consecutive workgroups are dealt round-robin to the 8
//     XCDs, each with its own L2. The launch index is remapped so each XCD
//     receives one contiguous run of tiles, walked in column groups of
//     kGroupM tile rows, so tiles sharing A rows and B columns meet in the
//     same L2.
//
// Ways of dividing the k range (compile-time per configuration):
//   * k-groups (KG > 1): KG groups of waves in one workgroup take alternate
//     k-tiles, each with its own LDS buffers, and are summed through LDS in
//     group order.
//   * Split-K over workgroups (SPLIT): S workgroups share one tile's k range;
//     each stores its partial tile, and the last to finish sums the S
//     partials in split order (see sgemm_mfma32).
//   * Stream-K (STREAMK): one or two workgroups per CU each take an equal
//     share of all (tile, k-tile) iterations, with the same exchange for the
//     tiles cut between workgroups; all but the last wave of tiles run whole.
// No workgroup ever waits for another, and every sum has a fixed order, so
// repeated calls give identical bits. The skinny kernels (M <= 32, bound by
// HBM) are described with their code.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "misgemm.h"
#include "ladder.h"

namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kXcds = 8;
constexpr int kGroupM = 8;
// Memory scope of the split-K exchange (partial blocks, counters): the
// workgroups that meet there all run on this GPU.
constexpr int kExchangeScope = __HIP_MEMORY_SCOPE_AGENT;
constexpr int kLdsPad = 4;

struct GemmArgs {
    const float *A;
    const float *B;
    float *C;
    int M, N, K;
    int lda, ldb, ldc;
    float alpha, beta;
    int tiles_m, tiles_n;
    int vec_ab;   // A and B: 16-byte aligned base, lda and ldb multiples of 4
    int vec_c;    // C: 16-byte aligned base, ldc multiple of 4
    // Split-K over workgroups (tile kernels): `splits` workgroups per tile,
    // each taking `kt_per_split` consecutive k-tiles; with splits > 1 their
    // partial tiles meet in `ws` and `counters` (one counter per tile).
    int splits, kt_per_split;
    // Stream-K: the last sk_dp_tiles tiles (a multiple of the grid) are taken
    // whole, one per workgroup per wave, after the shared-out ones.
    int sk_dp_tiles;
    float *ws;
    int *counters;
};

// BM x BN x BK macro tile; WAVES_M x WAVES_N waves share each k-tile; KG such
// groups of waves take alternate k-tiles (split-K inside the workgroup), each
// with its own LDS buffers, and are summed at the end in group order.
template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int KG_ = 1, int EU_ = 0, bool SPLIT_ = false,
          bool STREAMK_ = false, bool DL_ = false, bool MI16_ = false>
struct TileCfg {
    // MI16: blocks of 16 x 16 on v_mfma_f32_16x16x4_f32 (four accumulator
    // registers each, 16-deep q-groups) instead of 32 x 32 on
    // v_mfma_f32_32x32x2_f32 (sixteen registers, 8-deep q-groups). At one
    // wave per SIMD a small wave tile runs faster as 16 x 16 blocks (64 x 64
    // tile at 1024^3: 22.6 vs 27.5 us).
    static constexpr bool MI16 = MI16_;
    static constexpr int MBLK = MI16 ? 16 : 32;      // block edge
    static constexpr int ACC_REGS = MI16 ? 4 : 16;   // accumulator registers per block
    static constexpr int QK = MI16 ? 16 : 8;         // k per q-group
    // DL: the straight-line rounds move tiles global -> LDS directly
    // (global_load_lds_dwordx4), with unpadded, chunk-swizzled LDS rows.
    static constexpr bool DL = DL_;
    // SPLIT: the kernel carries the split-K-over-workgroups reduction.
    static constexpr bool SPLIT = SPLIT_;
    // STREAMK: one workgroup per CU walks an equal share of all (tile,
    // k-tile) iterations; tiles cut between workgroups use the same reduction.
    static constexpr bool STREAMK = STREAMK_;
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, KG = KG_;
    static constexpr int NTG = 64 * WAVES_M * WAVES_N;   // threads per k-group
    static constexpr int NT = NTG * KG;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    static constexpr int FM = WTM / MBLK, FN = WTN / MBLK;
    // Waves per SIMD the register allocation must allow: at least two (two
    // workgroups per CU where LDS allows), more when one workgroup alone
    // places more than two waves on each SIMD.
    static constexpr int WAVES_PER_EU = EU_ ? EU_ : (NT / 256 > 2 ? NT / 256 : 2);
    static_assert(WTM % MBLK == 0 && WTN % MBLK == 0, "wave tile must be whole blocks");
    static_assert(BK % (2 * QK) == 0, "fragment buffers alternate, so a k-tile holds an even number of q-groups");
};

// n adjacent floats from LDS (n = 1, 2, 4), as one ds_read.
template <int n> struct LdsVec;
template <> struct LdsVec<1> {
    static __device__ __forceinline__ void get(const float *p, float *out) { out[0] = *p; }
};
template <> struct LdsVec<2> {
    static __device__ __forceinline__ void get(const float *p, float *out) {
        f32x2 v = *reinterpret_cast<const f32x2 *>(p);
        out[0] = v[0]; out[1] = v[1];
    }
};
template <> struct LdsVec<4> {
    static __device__ __forceinline__ void get(const float *p, float *out) {
        f32x4 v = *reinterpret_cast<const f32x4 *>(p);
        out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
    }
};

// One R x CC tile of a stored row-major matrix, moved global -> registers ->
// LDS in 16-byte chunks. Thread t handles chunks t, t+NT, ...; a chunk is four
// consecutive columns of one row. LDS layout: [R][CC + kLdsPad].
//
// DL layout (for direct global -> LDS loads, which write a wave's 64 chunks
// to 1 KB of consecutive LDS): rows are unpadded, [R][CC]. When SWZ (a
// k-contiguous tile, read as 16-byte runs down 8 consecutive rows), chunk c
// of row r sits at chunk position c ^ swz(r) -- r mod 8 for rows of 8 or
// more chunks, (r / 2) mod 4 for rows of 4 -- so those 8 reads fall on 8
// different 16-byte bank groups, as the padding achieves otherwise.
template <int R, int CC, int NT, bool DL = false, bool SWZ = false>
struct TileCopy {
    static constexpr int CPR = CC / 4;                  // chunks per row
    static constexpr int CHUNKS = R * CPR;
    static constexpr int PER_THREAD = CHUNKS / NT;
    static constexpr int STRIDE = DL ? CC : CC + kLdsPad;
    static constexpr int LDS_FLOATS = R * STRIDE;
    static_assert(CC % 4 == 0 && CHUNKS % NT == 0, "tile must split evenly over the threads");
    static_assert(!SWZ || (DL && (CPR == 4 || CPR % 8 == 0)), "swizzle is for 16-wide or multiple-of-32-wide k-contiguous rows");
    static_assert(!DL || NT % 64 == 0, "direct loads are issued per wave");

    // Chunk position of chunk c in row r (SWZ), and its LDS float offset.
    static __device__ __forceinline__ int swz(int r) { return SWZ ? (CPR >= 8 ? r & 7 : (r / 2) & 3) : 0; }
    static __device__ __forceinline__ int at(int r, int c) { return r * STRIDE + ((c / 4) ^ swz(r)) * 4; }

    f32x4 v[PER_THREAD];

    // base points at stored element (r0, c0); rows_left / cols_left count the
    // in-range rows and columns from there (may exceed R / CC).
    __device__ __forceinline__ void load(const float *__restrict__ base, int ld, int rows_left,
                                         int cols_left, bool guard, bool vec, int tid) {
        if (!guard) {
#pragma unroll
            for (int j = 0; j < PER_THREAD; ++j) {
                const int idx = tid + NT * j;
                const int r = idx / CPR, c = (idx % CPR) * 4;
                v[j] = *reinterpret_cast<const f32x4 *>(base + (size_t)r * ld + c);
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < PER_THREAD; ++j) {
            const int idx = tid + NT * j;
            const int r = idx / CPR, c = (idx % CPR) * 4;
            const float *p = base + (size_t)r * ld + c;
            if (vec && r < rows_left && c + 3 < cols_left) {
                v[j] = *reinterpret_cast<const f32x4 *>(p);
            } else {
                f32x4 t;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    t[e] = (r < rows_left && c + e < cols_left) ? p[e] : 0.0f;
                v[j] = t;
            }
        }
    }

    __device__ __forceinline__ void store(float *lds, int tid) const {
#pragma unroll
        for (int j = 0; j < PER_THREAD; ++j) {
            const int idx = tid + NT * j;
            const int r = idx / CPR, c = (idx % CPR) * 4;
            *reinterpret_cast<f32x4 *>(lds + at(r, c)) = v[j];
        }
    }

    // DL layout, unguarded tile: each wave's j-th instruction fills LDS chunk
    // positions NT*j + 64*wave .. +63 (lane l the l-th), from the chunks that
    // belong there. The caller follows the batch with a compiler memory
    // barrier (the LDS writes are invisible to the compiler) and waits for
    // vmcnt before the workgroup barrier that publishes the tile.
    __device__ __forceinline__ void load_direct(const float *__restrict__ base, int ld, float *lds, int tid) const {
#pragma unroll
        for (int j = 0; j < PER_THREAD; ++j) {
            const int idx = tid + NT * j;
            const int r = idx / CPR, p = idx % CPR;
            const int c = p ^ swz(r);
            __builtin_amdgcn_global_load_lds(base + (size_t)r * ld + 4 * c, lds + 4 * (NT * j + (tid & ~63)), 16, 0,
                                             0);
        }
    }
};

template <int n> struct VecOf;
template <> struct VecOf<2> { using type = f32x2; };
template <> struct VecOf<4> { using type = f32x4; };

// C <- out + beta*C over n adjacent elements of one row, as one vector access
// when `whole` (all n in range and aligned), else element by element for the
// first `valid` of them. beta == 0: C is not read.
template <int n>
__device__ __forceinline__ void store_run(float *p, const float (&out)[n], float beta, bool whole, int valid) {
    if constexpr (n == 2 || n == 4) {
        if (whole) {
            using V = typename VecOf<n>::type;
            V *vp = reinterpret_cast<V *>(p);
            V v;
            if (beta != 0.0f) {
                const V c = *vp;
#pragma unroll
                for (int b = 0; b < n; ++b) v[b] = fmaf(beta, c[b], out[b]);
            } else {
#pragma unroll
                for (int b = 0; b < n; ++b) v[b] = out[b];
            }
            *vp = v;
            return;
        }
    }
#pragma unroll
    for (int b = 0; b < n; ++b)
        if (b < valid) p[b] = (beta != 0.0f) ? fmaf(beta, p[b], out[b]) : out[b];
}

// Launch index -> (tile row, tile column). Workgroup b runs on XCD b % 8; the
// j-th workgroup of XCD x is given logical tile prefix(x) + j, so each XCD
// walks one contiguous run of logical tiles. Logical tiles are ordered in
// groups of kGroupM tile rows, column by column within a group.
// With split-K, the S workgroups of a tile are adjacent in logical order (so
// usually on one XCD): logical = tile * S + split.
__device__ __forceinline__ int xcd_logical() {
    const int bid = blockIdx.x;
    const int total = gridDim.x;
    const int q = total / kXcds, rem = total % kXcds;
    const int x = bid % kXcds, j = bid / kXcds;
    return x * q + (x < rem ? x : rem) + j;
}

__device__ __forceinline__ void tile_of(int logical, int tiles_m, int tiles_n, int &tm, int &tn) {
    const int per_group = kGroupM * tiles_n;
    const int group = logical / per_group;
    const int first_m = group * kGroupM;
    const int gsz = min(tiles_m - first_m, kGroupM);
    const int in_g = logical - group * per_group;
    tm = first_m + in_g % gsz;
    tn = in_g / gsz;
}

__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int splits, int &tm, int &tn, int &split) {
    const int logical_ws = xcd_logical();
    split = logical_ws % splits;
    tile_of(logical_ws / splits, tiles_m, tiles_n, tm, tn);
}

// One tile's share of the k-range in a split product: segment seg of nseg (in
// k order), the tile's counter, and where segment j keeps its partial block:
// workspace slot s0 for j = 0, sbase + j*sstep after that.
struct SegInfo {
    int nseg, seg, counter;
    int s0, sbase, sstep;
    __device__ __forceinline__ int slot(int j) const { return j == 0 ? s0 : sbase + j * sstep; }
};

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

    // as/bs: LDS tiles of one k-tile, row strides AS/BS.
    template <int AS, int BS>
    __device__ __forceinline__ void read(const float *as, const float *bs, int q, int wm, int wn, int li, int lh) {
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
    static_assert(!TA || FM == 1 || FM == 2 || FM == 4, "one LDS read covers a row's FM blocks");
    static_assert(TB || FN == 1 || FN == 2 || FN == 4, "one LDS read covers a row's FN blocks");
    float a[FM][4];
    float b[FN][4];

    // Float offset of the lane's four k values inside a k-contiguous LDS row
    // (row c plus a multiple of 16), at its swizzled chunk position in the DL
    // layout.
    static __device__ __forceinline__ int kofs(int c, int g, int q) {
        if constexpr (CFG::DL) {
            return ((4 * q + g) ^ (c & 7)) * 4;
        } else {
            return 16 * q + 4 * g;
        }
    }

    // c, g: the lane's column and group (lane % 16, lane / 16).
    template <int AS, int BS>
    __device__ __forceinline__ void read(const float *as, const float *bs, int q, int wm, int wn, int c, int g) {
        const int k0 = 16 * q + 4 * g;
        if (!TA) {
#pragma unroll
            for (int blk = 0; blk < FM; ++blk)
                LdsVec<4>::get(as + (wm * WTM + 16 * blk + c) * AS + kofs(c, g, q), a[blk]);
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
#pragma unroll
            for (int blk = 0; blk < FN; ++blk)
                LdsVec<4>::get(bs + (wn * WTN + 16 * blk + c) * BS + kofs(c, g, q), b[blk]);
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

template <class CFG, bool TA, bool TB>
__global__ __launch_bounds__(CFG::NT) __attribute__((amdgpu_waves_per_eu(CFG::WAVES_PER_EU)))
void sgemm_mfma32(GemmArgs g) {
    constexpr int BM = CFG::BM, BN = CFG::BN, BK = CFG::BK, NTG = CFG::NTG, KG = CFG::KG;
    constexpr int FM = CFG::FM, FN = CFG::FN, WTM = CFG::WTM, WTN = CFG::WTN;
    constexpr int Q = BK / CFG::QK;             // q-groups per k-tile
    constexpr int AR = CFG::ACC_REGS, MBLK = CFG::MBLK;
    using AccT = std::conditional_t<CFG::MI16, f32x4, f32x16>;
    static_assert(Q % 2 == 0, "fragment buffers alternate, so the q-group count must be even");
    // Stored tile shapes: A is BM x BK ('N', k contiguous) or BK x BM ('T',
    // m contiguous); B is BK x BN ('N', n contiguous) or BN x BK ('T').
    using ACopy = TileCopy<TA ? BK : BM, TA ? BM : BK, NTG, CFG::DL, CFG::DL && !TA>;
    using BCopy = TileCopy<TB ? BN : BK, TB ? BK : BN, NTG, CFG::DL, CFG::DL && TB>;
    using F = std::conditional_t<CFG::MI16, Frag16<CFG, TA, TB>, Frag<CFG, TA, TB>>;
    constexpr int A_FLOATS = ACopy::LDS_FLOATS, B_FLOATS = BCopy::LDS_FLOATS;
    constexpr int AS = ACopy::STRIDE, BS = BCopy::STRIDE;
    constexpr int GROUP_FLOATS = 2 * (A_FLOATS + B_FLOATS);
    // The k-group reduction reuses the tile buffers: KG-1 groups x waves x
    // FM*FN accumulator blocks x 16 registers x 64 lanes.
    constexpr int RED_FLOATS = (KG - 1) * (NTG / 64) * FM * FN * AR * 64;
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
        const int grp = KG == 1 ? 0 : tid / NTG;    // k-group
        const int gtid = KG == 1 ? tid : tid % NTG;  // thread within it
        const int lane = gtid & 63, wave = gtid >> 6;
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
        const bool wg_fast = (m0 + BM <= M) && (n0 + BN <= N) && vec;
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
        auto fetch_fast = [&](int kt) {
            ca.load(a_ptr + kt * a_step, g.lda, 0, 0, false, true, gtid);
            cb.load(b_ptr + kt * b_step, g.ldb, 0, 0, false, true, gtid);
        };
        auto fetch_any = [&](int kt) {
            const int k0 = kt * BK;
            const bool guard = !(wg_fast && kt < kfull);
            // Rows/cols left counted from this k-tile's origin.
            ca.load(a_ptr + kt * a_step, g.lda, TA ? a_rows - k0 : a_rows, TA ? a_cols : a_cols - k0,
                    guard, vec, gtid);
            cb.load(b_ptr + kt * b_step, g.ldb, TB ? b_rows : b_rows - k0, TB ? b_cols - k0 : b_cols,
                    guard, vec, gtid);
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
        if (kt_begin + grp < kt_end) f0.template read<AS, BS>(a_lds, b_lds, 0, wm, wn, li, lh);

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
                    f1.template read<AS, BS>(as, bs, q + 1, wm, wn, li, lh);
                    f0.mma(acc);
                    if (q + 2 < Q) {
                        f0.template read<AS, BS>(as, bs, q + 2, wm, wn, li, lh);
                    } else if constexpr (!CFG::DL) {
                        ca.store(as_n, gtid);
                        cb.store(bs_n, gtid);
                    }
                    f1.mma(acc);
                }
                // DS reads per q-group: FM (or FN) 16-byte reads of a k-contiguous
                // tile, four narrow reads of an m/n-contiguous one. Direct loads
                // are issued before the round's first reads and leave no writes.
                constexpr int COPIES = CFG::DL ? 0 : ACopy::PER_THREAD + BCopy::PER_THREAD;
                schedule_iteration<4 * FM * FN, Q, COPIES, (TA ? 4 : FM) + (TB ? FN : 4), COPIES>();
                // Direct loads complete (vmcnt) before the barrier publishes them.
                if constexpr (CFG::DL) __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                f0.template read<AS, BS>(as_n, bs_n, 0, wm, wn, li, lh);
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
                    f1.template read<AS, BS>(as, bs, q + 1, wm, wn, li, lh);
                    f0.mma(acc);
                    if (q + 2 < Q) f0.template read<AS, BS>(as, bs, q + 2, wm, wn, li, lh);
                    f1.mma(acc);
                }
            }
            if (has_next) {
                ca.store(as_n, gtid);
                cb.store(bs_n, gtid);
            }
            __syncthreads();
            if (has_next) f0.template read<AS, BS>(as_n, bs_n, 0, wm, wn, li, lh);
        }

        if constexpr (KG > 1) {
            // Groups 1..KG-1 hand their accumulators to group 0 through LDS (the
            // tile buffers are free after the last barrier); group 0 adds them in
            // group order, so the sum is the same on every call.
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
            // Without split-K no barrier follows, so the other groups are done.
            if (!CFG::SPLIT && grp > 0) return;
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
        if (grp > 0) return;

        // Epilogue. Accumulator element r of block (i, j) in lane (li, lh) is
        // block row 8*(r/4) + 4*lh + r%4 (32 x 32 blocks) or 4*lh + r (16 x 16
        // blocks), block column li.
        const float alpha = g.alpha, beta = g.beta;
        float *const cw = g.C + (size_t)(m0 + wm * WTM) * g.ldc + (n0 + wn * WTN);
        const int rows_left = M - (m0 + wm * WTM), cols_left = N - (n0 + wn * WTN);
        const int ldc = g.ldc;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int r = 0; r < AR; ++r) {
                const int ib = CFG::MI16 ? 4 * lh + r : 8 * (r / 4) + 4 * lh + (r % 4);
                const int row = TA ? FM * ib + i : MBLK * i + ib;
                if (row >= rows_left) continue;
                float *crow = cw + (size_t)row * ldc;
                if (!TB) {
                    // FN adjacent columns FN*li .. FN*li + FN-1.
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
    };

    if constexpr (CFG::STREAMK) {
        static_assert(KG == 1 && !CFG::SPLIT, "stream-K runs one k-group");
        // The first sk_tiles tiles are shared out: iteration i is k-tile
        // i % ktiles of tile i / ktiles (tiles in the grouped order), and
        // workgroup w owns [start(w), start(w+1)); workgroups on one XCD own
        // consecutive shares. The rest follow whole, one per workgroup per wave.
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
    // The loads of eight splits are issued before they are summed; the sum
    // runs in split order.
    const float *parts = sa.ws + (size_t)tile * S * T;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int idx = tid + NT * i;
        if (idx >= T) break;
        float sum = 0.0f;
        for (int sp0 = 0; sp0 < S; sp0 += 8) {
            const float *p = parts + (size_t)sp0 * T + idx;
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = sp0 + i < S ? __hip_atomic_load(p + (size_t)i * T, __ATOMIC_RELAXED, kExchangeScope)
                                   : 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (sp0 + i < S) sum += v[i];
        }
        finish(i, idx, sum);
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

// ---------------------------------------------------------------------------
// Configuration table.

using CfgL = TileCfg<128, 128, 32, 2, 2>;        // 4 waves, 64 x 64 per wave
using CfgS = TileCfg<64, 64, 32, 2, 2>;          // 4 waves, 32 x 32 per wave
using CfgS2 = TileCfg<64, 64, 32, 2, 2, 2>;      // 8 waves: 2 k-groups of 4
using CfgS4 = TileCfg<64, 64, 32, 2, 2, 4>;      // 16 waves: 4 k-groups of 4
using CfgL2 = TileCfg<128, 128, 32, 2, 2, 2>;    // 8 waves: 2 k-groups of 4
using CfgL24 = TileCfg<128, 128, 32, 2, 4, 1, 4>;   // 8 waves, 64 x 32 per wave, 2 per CU
using CfgL42 = TileCfg<128, 128, 32, 4, 2, 1, 4>;   // 8 waves, 32 x 64 per wave, 2 per CU
using CfgW = TileCfg<256, 128, 32, 4, 2>;        // 8 waves, 64 x 64 per wave
using CfgT = TileCfg<128, 256, 32, 2, 4>;        // 8 waves, 64 x 64 per wave
using CfgT16 = TileCfg<128, 256, 16, 2, 2>;      // 4 waves, 64 x 128 per wave, 2 per CU
using CfgQ32 = TileCfg<256, 256, 32, 4, 2>;      // 8 waves, 64 x 128 per wave, 1 per CU
// Split-K over workgroups (for grids with fewer tiles than CU slots).
using CfgL42K = TileCfg<128, 128, 32, 4, 2, 1, 0, true>;   // one per CU
using CfgSK = TileCfg<64, 64, 32, 2, 2, 1, 0, true>;
using CfgLK = TileCfg<128, 128, 32, 2, 2, 1, 0, true>;
// Stream-K: one workgroup per CU (two waves per SIMD), or two (four).
using CfgL42S1 = TileCfg<128, 128, 32, 4, 2, 1, 2, false, true>;
using CfgL42S2 = TileCfg<128, 128, 32, 4, 2, 1, 4, false, true>;
using CfgWS = TileCfg<256, 128, 32, 4, 2, 1, 0, false, true>;   // one workgroup per CU
using CfgTS = TileCfg<128, 256, 32, 2, 4, 1, 0, false, true>;
// Direct global -> LDS loads in the straight-line rounds.
using CfgQ32D = TileCfg<256, 256, 32, 4, 2, 1, 0, false, false, true>;
using CfgL42D = TileCfg<128, 128, 32, 4, 2, 1, 4, false, false, true>;
// 16 x 16 MFMA blocks.
using Cfg16S = TileCfg<64, 64, 32, 2, 2, 1, 0, false, false, false, true>;
using Cfg16S2 = TileCfg<64, 64, 32, 2, 2, 2, 0, false, false, false, true>;
using Cfg16S4 = TileCfg<64, 64, 32, 2, 2, 4, 0, false, false, false, true>;
using Cfg16SK = TileCfg<64, 64, 32, 2, 2, 1, 0, true, false, false, true>;
using Cfg16L42 = TileCfg<128, 128, 32, 4, 2, 1, 4, false, false, false, true>;
using Cfg16L42S1 = TileCfg<128, 128, 32, 4, 2, 1, 2, false, true, false, true>;
using Cfg16L = TileCfg<128, 128, 32, 2, 2, 1, 0, false, false, false, true>;
using Cfg16W = TileCfg<256, 128, 32, 4, 2, 1, 0, false, false, false, true>;
using Cfg16L42D = TileCfg<128, 128, 32, 4, 2, 1, 4, false, false, true, true>;
using Cfg16S4D = TileCfg<64, 64, 32, 2, 2, 4, 0, false, false, true, true>;

// Config ids: the index of each entry of kConfigs below.
enum ConfigId : int {
    kCfg128 = 0,
    kCfg64 = 1,
    kCfgSkinny16 = 2,
    kCfgBand = 3,
    kCfg64Kg2 = 4,
    kCfg64Kg4 = 5,
    kCfg128Kg2 = 6,
    kCfg128W24 = 7,
    kCfg128W42 = 8,
    kCfg256x128 = 9,
    kCfg128x256 = 10,
    kCfg128W42Split = 11,
    kCfg64Split = 12,
    kCfg128Split = 13,
    kCfg128x256x16 = 14,
    kCfg256x256 = 15,
    kCfgStreamK1 = 16,
    kCfgStreamK2 = 17,
    kCfgStreamK256x128 = 18,
    kCfgStreamK128x256 = 19,
    // The vector-ALU technique ladder (ladder.hip), forced only.
    kCfgLadderFirst = 20,
    kCfgLadderLast = kCfgLadderFirst + misgemm_ladder::kNumRungs - 1,
    kCfg256x256Dl = 25,
    kCfg128W42Dl = 26,
    kCfg16x64 = 27,
    kCfg16x64Kg2 = 28,
    kCfg16x64Kg4 = 29,
    kCfg16x64Split = 30,
    kCfg16x128W42 = 31,
    kCfg16StreamK1 = 32,
    kCfg16x128 = 33,
    kCfg16x256x128 = 34,
    kCfg16x128W42Dl = 35,
    kCfg16x64Kg4Dl = 36,
};

struct ConfigInfo {
    const char *name;
    int bm, bn, nt;
};

constexpr ConfigInfo kConfigs[] = {
    {"mfma32_128x128x32_w2x2", CfgL::BM, CfgL::BN, CfgL::NT},
    {"mfma32_64x64x32_w2x2", CfgS::BM, CfgS::BN, CfgS::NT},
    {"skinny_mfma16_16cols_splitk8", 32, 16, 64 * kSkinnyWaves},
    {"skinny_mfma16_band128_splitk", 32, kBandCols, 64 * kBandWaves},
    {"mfma32_64x64x32_w2x2_kg2", CfgS2::BM, CfgS2::BN, CfgS2::NT},
    {"mfma32_64x64x32_w2x2_kg4", CfgS4::BM, CfgS4::BN, CfgS4::NT},
    {"mfma32_128x128x32_w2x2_kg2", CfgL2::BM, CfgL2::BN, CfgL2::NT},
    {"mfma32_128x128x32_w2x4", CfgL24::BM, CfgL24::BN, CfgL24::NT},
    {"mfma32_128x128x32_w4x2", CfgL42::BM, CfgL42::BN, CfgL42::NT},
    {"mfma32_256x128x32_w4x2", CfgW::BM, CfgW::BN, CfgW::NT},
    {"mfma32_128x256x32_w2x4", CfgT::BM, CfgT::BN, CfgT::NT},
    {"mfma32_128x128x32_w4x2_splitk", CfgL42K::BM, CfgL42K::BN, CfgL42K::NT},
    {"mfma32_64x64x32_w2x2_splitk", CfgSK::BM, CfgSK::BN, CfgSK::NT},
    {"mfma32_128x128x32_w2x2_splitk", CfgLK::BM, CfgLK::BN, CfgLK::NT},
    {"mfma32_128x256x16_w2x2", CfgT16::BM, CfgT16::BN, CfgT16::NT},
    {"mfma32_256x256x32_w4x2", CfgQ32::BM, CfgQ32::BN, CfgQ32::NT},
    {"mfma32_128x128x32_w4x2_streamk_1wg", CfgL42S1::BM, CfgL42S1::BN, CfgL42S1::NT},
    {"mfma32_128x128x32_w4x2_streamk_2wg", CfgL42S2::BM, CfgL42S2::BN, CfgL42S2::NT},
    {"mfma32_256x128x32_w4x2_streamk", CfgWS::BM, CfgWS::BN, CfgWS::NT},
    {"mfma32_128x256x32_w2x4_streamk", CfgTS::BM, CfgTS::BN, CfgTS::NT},
    {"valu_naive", 4, 64, 256},
    {"valu_lds32x32", 32, 32, 1024},
    {"valu_block1d_64x64x8_tm8", 64, 64, 512},
    {"valu_block2d_128x128x8_8x8", 128, 128, 256},
    {"valu_vec2d_128x128x8_8x8_dbuf", 128, 128, 256},
    {"mfma32_256x256x32_w4x2_dl", CfgQ32D::BM, CfgQ32D::BN, CfgQ32D::NT},
    {"mfma32_128x128x32_w4x2_dl", CfgL42D::BM, CfgL42D::BN, CfgL42D::NT},
    {"mfma16_64x64x32_w2x2", Cfg16S::BM, Cfg16S::BN, Cfg16S::NT},
    {"mfma16_64x64x32_w2x2_kg2", Cfg16S2::BM, Cfg16S2::BN, Cfg16S2::NT},
    {"mfma16_64x64x32_w2x2_kg4", Cfg16S4::BM, Cfg16S4::BN, Cfg16S4::NT},
    {"mfma16_64x64x32_w2x2_splitk", Cfg16SK::BM, Cfg16SK::BN, Cfg16SK::NT},
    {"mfma16_128x128x32_w4x2", Cfg16L42::BM, Cfg16L42::BN, Cfg16L42::NT},
    {"mfma16_128x128x32_w4x2_streamk_1wg", Cfg16L42S1::BM, Cfg16L42S1::BN, Cfg16L42S1::NT},
    {"mfma16_128x128x32_w2x2", Cfg16L::BM, Cfg16L::BN, Cfg16L::NT},
    {"mfma16_256x128x32_w4x2", Cfg16W::BM, Cfg16W::BN, Cfg16W::NT},
    {"mfma16_128x128x32_w4x2_dl", Cfg16L42D::BM, Cfg16L42D::BN, Cfg16L42D::NT},
    {"mfma16_64x64x32_w2x2_kg4_dl", Cfg16S4D::BM, Cfg16S4D::BN, Cfg16S4D::NT},
};
constexpr int kSkinnyMaxM = 32;
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);
static_assert(kNumConfigs == kCfg16x64Kg4Dl + 1, "one ConfigId per kConfigs entry");
static_assert(kCfgLadderLast + 1 == kCfg256x256Dl, "the ladder ids are contiguous");
static_assert(kConfigs[kCfg128].bm == CfgL::BM && kConfigs[kCfg128].bn == CfgL::BN && kConfigs[kCfg128].nt == CfgL::NT, "kConfigs order");
static_assert(kConfigs[kCfg64].bm == CfgS::BM && kConfigs[kCfg64].bn == CfgS::BN && kConfigs[kCfg64].nt == CfgS::NT, "kConfigs order");
static_assert(kConfigs[kCfg64Kg2].bm == CfgS2::BM && kConfigs[kCfg64Kg2].bn == CfgS2::BN && kConfigs[kCfg64Kg2].nt == CfgS2::NT, "kConfigs order");
static_assert(kConfigs[kCfg64Kg4].bm == CfgS4::BM && kConfigs[kCfg64Kg4].bn == CfgS4::BN && kConfigs[kCfg64Kg4].nt == CfgS4::NT, "kConfigs order");
static_assert(kConfigs[kCfg128Kg2].bm == CfgL2::BM && kConfigs[kCfg128Kg2].bn == CfgL2::BN && kConfigs[kCfg128Kg2].nt == CfgL2::NT, "kConfigs order");
static_assert(kConfigs[kCfg128W24].bm == CfgL24::BM && kConfigs[kCfg128W24].bn == CfgL24::BN && kConfigs[kCfg128W24].nt == CfgL24::NT, "kConfigs order");
static_assert(kConfigs[kCfg128W42].bm == CfgL42::BM && kConfigs[kCfg128W42].bn == CfgL42::BN && kConfigs[kCfg128W42].nt == CfgL42::NT, "kConfigs order");
static_assert(kConfigs[kCfg256x128].bm == CfgW::BM && kConfigs[kCfg256x128].bn == CfgW::BN && kConfigs[kCfg256x128].nt == CfgW::NT, "kConfigs order");
static_assert(kConfigs[kCfg128x256].bm == CfgT::BM && kConfigs[kCfg128x256].bn == CfgT::BN && kConfigs[kCfg128x256].nt == CfgT::NT, "kConfigs order");
static_assert(kConfigs[kCfg128W42Split].bm == CfgL42K::BM && kConfigs[kCfg128W42Split].bn == CfgL42K::BN && kConfigs[kCfg128W42Split].nt == CfgL42K::NT, "kConfigs order");
static_assert(kConfigs[kCfg64Split].bm == CfgSK::BM && kConfigs[kCfg64Split].bn == CfgSK::BN && kConfigs[kCfg64Split].nt == CfgSK::NT, "kConfigs order");
static_assert(kConfigs[kCfg128Split].bm == CfgLK::BM && kConfigs[kCfg128Split].bn == CfgLK::BN && kConfigs[kCfg128Split].nt == CfgLK::NT, "kConfigs order");
static_assert(kConfigs[kCfg128x256x16].bm == CfgT16::BM && kConfigs[kCfg128x256x16].bn == CfgT16::BN && kConfigs[kCfg128x256x16].nt == CfgT16::NT, "kConfigs order");
static_assert(kConfigs[kCfg256x256].bm == CfgQ32::BM && kConfigs[kCfg256x256].bn == CfgQ32::BN && kConfigs[kCfg256x256].nt == CfgQ32::NT, "kConfigs order");
static_assert(kConfigs[kCfgStreamK1].bm == CfgL42S1::BM && kConfigs[kCfgStreamK1].bn == CfgL42S1::BN && kConfigs[kCfgStreamK1].nt == CfgL42S1::NT, "kConfigs order");
static_assert(kConfigs[kCfgStreamK2].bm == CfgL42S2::BM && kConfigs[kCfgStreamK2].bn == CfgL42S2::BN && kConfigs[kCfgStreamK2].nt == CfgL42S2::NT, "kConfigs order");
static_assert(kConfigs[kCfgStreamK256x128].bm == CfgWS::BM && kConfigs[kCfgStreamK256x128].bn == CfgWS::BN && kConfigs[kCfgStreamK256x128].nt == CfgWS::NT, "kConfigs order");
static_assert(kConfigs[kCfgStreamK128x256].bm == CfgTS::BM && kConfigs[kCfgStreamK128x256].bn == CfgTS::BN && kConfigs[kCfgStreamK128x256].nt == CfgTS::NT, "kConfigs order");
static_assert(kConfigs[kCfg256x256Dl].bm == CfgQ32D::BM && kConfigs[kCfg256x256Dl].bn == CfgQ32D::BN && kConfigs[kCfg256x256Dl].nt == CfgQ32D::NT, "kConfigs order");
static_assert(kConfigs[kCfg128W42Dl].bm == CfgL42D::BM && kConfigs[kCfg128W42Dl].bn == CfgL42D::BN && kConfigs[kCfg128W42Dl].nt == CfgL42D::NT, "kConfigs order");
constexpr int kNumCus = 256;

bool op_n(char t) { return t == 'N' || t == 'n'; }
bool op_t(char t) { return t == 'T' || t == 't' || t == 'C' || t == 'c'; }

int check_args(char transA, char transB, int M, int N, int K, float alpha, const float *A, int lda,
               const float *B, int ldb, const float *C, int ldc) {
    if (!op_n(transA) && !op_t(transA)) return MISGEMM_BAD_TRANSA;
    if (!op_n(transB) && !op_t(transB)) return MISGEMM_BAD_TRANSB;
    if (M < 0) return MISGEMM_BAD_M;
    if (N < 0) return MISGEMM_BAD_N;
    if (K < 0) return MISGEMM_BAD_K;
    const int a_cols = op_n(transA) ? K : M;
    const int b_cols = op_n(transB) ? N : K;
    if (lda < (a_cols > 1 ? a_cols : 1)) return MISGEMM_BAD_LDA;
    if (ldb < (b_cols > 1 ? b_cols : 1)) return MISGEMM_BAD_LDB;
    if (ldc < (N > 1 ? N : 1)) return MISGEMM_BAD_LDC;
    if (M == 0 || N == 0) return MISGEMM_SUCCESS;
    const bool reads_ab = alpha != 0.0f && K > 0;
    if (reads_ab && A == nullptr) return MISGEMM_NULL_A;
    if (reads_ab && B == nullptr) return MISGEMM_NULL_B;
    if (C == nullptr) return MISGEMM_NULL_C;
    return MISGEMM_SUCCESS;
}

// Fraction of the busiest CU's workgroup slots that hold work when `tiles`
// workgroups are spread over the CUs, `slots` at a time per CU: 1 when every
// CU gets the same count.
double cu_balance(long long tiles, int slots = 1) {
    const long long cap = (long long)kNumCus * slots;
    const long long rounds = (tiles + cap - 1) / cap;
    return (double)tiles / (double)(rounds * cap);
}

// Timing model of the 64 x 64 x 32 tile (four waves; up to four resident per
// CU, bounded by LDS), in microseconds, for `kgroups` k-groups per workgroup
// (each a set of four waves) or `splits` workgroups per tile:
//   T = 4 + kt * max(0.6 u, 0.88) + 2 ceil(S / 4)   (the last term when S > 1)
// where u = kgroups * ceil(tiles * S / CUs) is the number of four-wave units
// on the busiest CU and kt the k-tiles each unit runs. A k-tile costs a lone
// unit 0.88 us (load latency) and 0.6 us per unit once several share the CU;
// the last workgroup of a split tile sums the partials four at a time, about
// 2 us per batch. The terms are fitted to timings of every split count and
// k-group count on square products from 320^3 to 1152^3 and on long-K
// products (512 x 512 x 4096, 2048 x 256 x 2048) on MI355X; it orders split
// counts and the split / four-k-group choice correctly up to 256 tiles, but
// underrates two k-groups above that.
double model_64x64_us(long long tiles, int ktiles, int kgroups, long long splits) {
    const long long kt_split = (ktiles + splits - 1) / splits;
    const long long kt = (kt_split + kgroups - 1) / kgroups;
    const long long u = kgroups * ((tiles * splits + kNumCus - 1) / kNumCus);
    double t = 4.0 + (double)kt * std::max(0.6 * (double)u, 0.88);
    if (splits > 1) t += 2.0 * (double)((splits + 3) / 4);
    return t;
}

// Split count for the 64 x 64 x 32 split-K tile: the modelled fastest among
// those that keep every workgroup resident at once (at most four per CU) with
// at least two k-tiles per split; one split is always a candidate.
long long splits_64x64(long long tiles, int ktiles) {
    long long best_s = 1;
    double best_t = model_64x64_us(tiles, ktiles, 1, 1);
    for (long long s = 2; s <= std::min<long long>(kMaxSplits, ktiles); ++s) {
        const long long kt = (ktiles + s - 1) / s;
        if ((ktiles + kt - 1) / kt != s) continue;   // same split as a smaller s
        if (kt < 2 || tiles * s > 4LL * kNumCus) continue;
        const double t = model_64x64_us(tiles, ktiles, 1, s);
        if (t < best_t) {
            best_s = s;
            best_t = t;
        }
    }
    return best_s;
}

// Shape class -> configuration, from per-configuration timings of the square
// sweep, the layer shapes and the ragged shape on MI355X (bench.py
// --sweep-configs):
//   M <= 32, N >= 128   skinny band kernel (HBM-bound);
//   >= 256 tiles of 128 x 128: the best-scoring of
//                       256 x 256 with 8 waves (one per CU; B not
//                         transposed)                        1.044 x balance
//                       stream-K 256 x 128 / 128 x 256, one workgroup
//                         per CU (B not transposed)          0.955 (always balanced)
//                       stream-K 128 x 128, two workgroups per CU
//                         (either: >= 8 k-tiles per workgroup) 0.925 (always balanced)
//                       stream-K 128 x 128 of 16 x 16 blocks, one
//                         workgroup per CU (neither transposed) 0.965 (always balanced)
//                       128 x 256 with 4 waves (two workgroups per CU; B
//                         not transposed)                    1.038 x balance over 2 slots per CU
//                       256 x 128 / 128 x 256 with 8 waves (one per CU; B
//                         not transposed)                    1.024 x balance
//                       128 x 128 with 8 waves                   1 x balance
//                       64 x 64                               0.87 x balance
//                       (the factors are their relative speeds on a large,
//                       evenly spread product);
//   144..255 such tiles with >= 20 k-tiles per workgroup: stream-K 128 x 128,
//                       one workgroup per CU;
//   192..255 such tiles otherwise: 128 x 128 with 8 waves;
//   else, by 64 x 64 tiles: >= 512 plain; 257..511 two k-groups, or split-K
//                       over workgroups when those would fill under 75% of
//                       the CU slots; <= 256 four k-groups or split-K,
//                       whichever the 64 x 64 timing model puts first.
// The 128 x 128 (8 waves), one-workgroup stream-K 128 x 128 and 64 x 64
// tiles run as 16 x 16 MFMA blocks; the larger tiles as 32 x 32 blocks.
int select_config(char transA, char transB, int M, int N, int K) {
    // Few rows: the band kernel streams op(B) once; below one 128-column band
    // its padding costs more than a tile kernel (32 x 64 x 64: 8.9 vs 5.6 us).
    if (M <= kSkinnyMaxM && N >= kBandCols) return kCfgBand;
    auto tiles = [&](int bm, int bn) { return (long long)((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    const long long t128 = tiles(128, 128), t64 = tiles(64, 64);
    // Stream-K work: 128 x 128 x 32 iterations.
    const long long sk_iters = t128 * ((K + 31) / 32);
    // The 128 x 128 and 64 x 64 tiles run as 16 x 16 MFMA blocks, 2-18%
    // faster than as 32 x 32 blocks for every op pair (1024^3: 22 vs 24 us;
    // 2048 x 4096 x 1024 TN: 132 vs 144 us).
    const int cfg128 = kCfg16x128W42;
    if (t128 >= kNumCus) {
        const bool ta = op_t(transA), tb = op_t(transB);
        // Big tiles (one workgroup per CU) lose to 128 x 128 (two per CU)
        // when K is short and the grid fills the chip only once; with both
        // transposed, 256 x 128 is the one that gains (the register-staged
        // 256 x 256 and 128 x 256 x 16 tiles do not).
        const bool big_ok = !(K < 2048 && t128 < 4 * kNumCus);
        const bool tt = ta && tb;
        const bool wide = !tt && M < N;    // 128 x 256 rather than 256 x 128
        // With both transposed, the 256 x 256 tile with direct-to-LDS loads
        // (the register-staged one spills): 960 vs 989 us for 256 x 128 at 4096^3.
        const double s_q = big_ok ? (tt ? 1.065 : 1.044) * cu_balance(tiles(256, 256)) : -1.0;
        const double s_b4 = big_ok ? (tt ? 1.0 : 1.038) * cu_balance(tiles(128, 256), 2) : -1.0;
        const double s_b8 = big_ok ? (tt ? 1.034 : 1.024) * cu_balance(wide ? tiles(128, 256) : tiles(256, 128)) : -1.0;
        const double s_128 = cu_balance(t128), s_64 = 0.87 * cu_balance(t64);
        // Stream-K fills every CU slot whatever the tile count: with the
        // 256 x 128 / 128 x 256 tile where big tiles pay, else 128 x 128.
        const bool sk_ok = sk_iters >= 8LL * 2 * kNumCus;
        const double s_skb = (sk_ok && big_ok) ? 0.955 : -1.0;
        const double s_sk = sk_ok ? 0.925 : -1.0;
        // With neither operand transposed, stream-K over 128 x 128 tiles of
        // 16 x 16 blocks, one workgroup per CU, beats the big-tile stream-K
        // (n = 2304: 193 vs 202 us; 3840: 839 vs 854).
        const double s_sk16 = (sk_ok && !ta && !tb) ? 0.965 : -1.0;
        const double best =
            fmax(fmax(fmax(s_q, fmax(s_skb, s_sk)), fmax(s_b4, s_b8)), fmax(fmax(s_128, s_64), s_sk16));
        if (best == s_q) return tt ? kCfg256x256Dl : kCfg256x256;
        if (best == s_sk16) return kCfg16StreamK1;
        if (best == s_skb) return wide ? kCfgStreamK128x256 : kCfgStreamK256x128;
        if (best == s_sk) return kCfgStreamK2;
        if (best == s_b4) return kCfg128x256x16;
        if (best == s_b8) return wide ? kCfg128x256 : kCfg256x128;
        return best == s_128 ? cfg128 : kCfg16x64;
    }
    // 144..255 tiles of 128 x 128 with at least 20 k-tiles per workgroup:
    // stream-K, one workgroup per CU.
    if (t128 >= 144 && sk_iters >= 20LL * kNumCus) return kCfg16StreamK1;
    if (t128 >= 3 * kNumCus / 4) return cfg128;
    if (t64 >= 2 * kNumCus) return kCfg16x64;
    // 257..511 tiles of 64 x 64: two k-groups unless their workgroups would
    // leave the CU slots badly filled; then split-K over workgroups, whose
    // smaller workgroups spread more evenly.
    if (t64 > kNumCus) return (double)t64 / (2 * kNumCus) >= 0.75 ? kCfg16x64Kg2 : kCfg16x64Split;
    // Up to 256 tiles of 64 x 64: four k-groups or split-K over workgroups,
    // whichever the timing model puts first.
    const int ktiles = (K + 31) / 32;
    const double t_split = model_64x64_us(t64, ktiles, 1, splits_64x64(t64, ktiles));
    return t_split < model_64x64_us(t64, ktiles, 4, 1) ? kCfg16x64Split : kCfg16x64Kg4;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <class CFG, bool TA, bool TB>
hipError_t launch_t(const GemmArgs &g, unsigned workgroups, hipStream_t stream) {
    dim3 grid(workgroups);
    dim3 block(CFG::NT);
    hipLaunchKernelGGL((sgemm_mfma32<CFG, TA, TB>), grid, block, 0, stream, g);
    return hipGetLastError();
}

// Workspace for the split-K reduction, one per (device, stream) so that calls
// on different streams never share partials or counters. Allocated on the
// first call that needs it and kept until the process ends.
constexpr size_t kWsFloats = size_t(16) << 20;  // 64 MiB of partial blocks
constexpr int kWsCounters = 1 << 16;

struct Workspace {
    float *partials = nullptr;
    int *counters = nullptr;
};

std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

// Returns nullptr if no workspace can be had (the caller then runs unsplit).
// The device a stream's work runs on (the current device for the null
// stream): its workspace lives there, whatever device is current.
bool stream_device(hipStream_t stream, int &dev) {
    if (stream == nullptr) return hipGetDevice(&dev) == hipSuccess;
    hipDevice_t d = 0;
    if (hipStreamGetDevice(stream, &d) != hipSuccess) return false;
    dev = d;
    return true;
}

// Makes `dev` current for its lifetime and restores the caller's device.
struct DeviceGuard {
    int saved = -1;
    bool ok = false;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&saved) != hipSuccess) return;
        ok = saved == dev || hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceGuard() {
        if (saved >= 0) (void)hipSetDevice(saved);
    }
};

const Workspace *get_workspace(hipStream_t stream) {
    int dev = 0;
    if (!stream_device(stream, dev)) return nullptr;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    auto key = std::make_pair(dev, stream);
    auto it = g_ws.find(key);
    if (it != g_ws.end()) return &it->second;
    // No allocation while the stream is being captured into a graph: the
    // captured call runs unsplit instead.
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    if (stream != nullptr &&
        (hipStreamIsCapturing(stream, &capture) != hipSuccess || capture != hipStreamCaptureStatusNone))
        return nullptr;
    DeviceGuard on_dev(dev);
    if (!on_dev.ok) return nullptr;
    Workspace w;
    if (hipMalloc(reinterpret_cast<void **>(&w.partials), kWsFloats * sizeof(float)) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (hipMalloc(reinterpret_cast<void **>(&w.counters), kWsCounters * sizeof(int)) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipFree(w.partials);
        return nullptr;
    }
    hipLaunchKernelGGL(zero_ints, dim3((kWsCounters + 255) / 256), dim3(256), 0, stream, w.counters, kWsCounters);
    if (hipGetLastError() != hipSuccess) {
        (void)hipFree(w.partials);
        (void)hipFree(w.counters);
        return nullptr;
    }
    return &g_ws.emplace(key, w).first->second;
}

// Split factor for the band kernel: enough workgroups to fill every CU's
// workgroup slots once (the LDS partial blocks limit how many fit on a CU),
// at least one 16-row chunk per wave, within the workspace.
int band_splits(int M, int N, int K, int mb, bool fast) {
    const long long bands = (N + kBandCols - 1) / kBandCols;
    const long long yb = (M + 16 * mb - 1) / (16 * mb);
    const long long tiles = bands * yb;
    const int waves = mb == 1 ? (fast ? band_waves<1, true>() : band_waves<1, false>())
                              : (fast ? band_waves<2, true>() : band_waves<2, false>());
    const long long lds_bytes = (long long)waves * 16 * mb * kBandCols * 4;
    const long long per_cu = lds_bytes > 80 * 1024 ? 1 : 2;
    long long S = (per_cu * kNumCus + tiles - 1) / tiles;
    const long long max_by_k = (K + 16 * waves - 1) / (16 * waves);
    if (S > max_by_k) S = max_by_k;
    if (S > kMaxSplits) S = kMaxSplits;
    const long long per_split = 16LL * mb * kBandCols;
    while (S > 1 && tiles * S * per_split > (long long)kWsFloats) --S;
    if (tiles > kWsCounters) S = 1;
    return S < 1 ? 1 : (int)S;
}

template <int MB, bool TA, bool TB, bool FAST>
hipError_t launch_band_t(const SplitArgs &sa, hipStream_t stream) {
    const int bands = (sa.g.N + kBandCols - 1) / kBandCols;
    dim3 grid((unsigned)(bands * sa.splits), (unsigned)((sa.g.M + 16 * MB - 1) / (16 * MB)));
    hipLaunchKernelGGL((sgemm_skinny_band<MB, TA, TB, FAST>), grid, dim3((64 * band_waves<MB, FAST>())), 0, stream, sa);
    return hipGetLastError();
}

template <int MB, bool FAST>
hipError_t launch_band_mb(bool ta, bool tb, const SplitArgs &sa, hipStream_t stream) {
    if (!ta && !tb) return launch_band_t<MB, false, false, FAST>(sa, stream);
    if (!ta && tb) return launch_band_t<MB, false, true, FAST>(sa, stream);
    if (ta && !tb) return launch_band_t<MB, true, false, FAST>(sa, stream);
    return launch_band_t<MB, true, true, FAST>(sa, stream);
}

hipError_t launch_band(bool ta, bool tb, const GemmArgs &g, hipStream_t stream) {
    const int mb = g.M <= 16 ? 1 : 2;
    SplitArgs sa;
    sa.g = g;
    sa.ws = nullptr;
    sa.counters = nullptr;
    // Unguarded instantiation: whole bands, whole 16-row chunks, 16-byte loads.
    const bool fast = g.vec_ab && g.N % kBandCols == 0 && g.K % 16 == 0;
    int S = band_splits(g.M, g.N, g.K, mb, fast);
    if (S > 1) {
        const Workspace *w = get_workspace(stream);
        if (w == nullptr) {
            S = 1;
        } else {
            sa.ws = w->partials;
            sa.counters = w->counters;
        }
    }
    int rps = (((g.K + 15) / 16 + S - 1) / S) * 16;
    S = (g.K + rps - 1) / rps;
    if (S < 1) S = 1;
    sa.splits = S;
    sa.rows_per_split = rps;
    if (mb == 1) return fast ? launch_band_mb<1, true>(ta, tb, sa, stream) : launch_band_mb<1, false>(ta, tb, sa, stream);
    return fast ? launch_band_mb<2, true>(ta, tb, sa, stream) : launch_band_mb<2, false>(ta, tb, sa, stream);
}

template <int MB, bool TA, bool TB>
hipError_t launch_skinny_t(const GemmArgs &g, hipStream_t stream) {
    dim3 grid((unsigned)((g.N + 15) / 16), (unsigned)((g.M + 16 * MB - 1) / (16 * MB)));
    hipLaunchKernelGGL((sgemm_skinny16<MB, TA, TB>), grid, dim3(64 * kSkinnyWaves), 0, stream, g);
    return hipGetLastError();
}

template <int MB>
hipError_t launch_skinny_mb(bool ta, bool tb, const GemmArgs &g, hipStream_t stream) {
    if (!ta && !tb) return launch_skinny_t<MB, false, false>(g, stream);
    if (!ta && tb) return launch_skinny_t<MB, false, true>(g, stream);
    if (ta && !tb) return launch_skinny_t<MB, true, false>(g, stream);
    return launch_skinny_t<MB, true, true>(g, stream);
}

hipError_t launch_skinny(bool ta, bool tb, const GemmArgs &g, hipStream_t stream) {
    if (g.M <= 16) return launch_skinny_mb<1>(ta, tb, g, stream);
    return launch_skinny_mb<2>(ta, tb, g, stream);
}

template <class CFG>
hipError_t launch_cfg(bool ta, bool tb, GemmArgs &g, hipStream_t stream, int split_slots = 0) {
    g.tiles_m = (g.M + CFG::BM - 1) / CFG::BM;
    g.tiles_n = (g.N + CFG::BN - 1) / CFG::BN;
    const int ktiles = (g.K + CFG::BK - 1) / CFG::BK;
    g.splits = 1;
    g.kt_per_split = ktiles;
    g.sk_dp_tiles = 0;
    g.ws = nullptr;
    g.counters = nullptr;
    if (CFG::SPLIT && split_slots > 0) {
        // Split-K over workgroups: for 64 x 64 tiles the modelled best split;
        // otherwise about one workgroup per CU slot with at least four
        // k-tiles per split. Either within the workspace.
        const long long tiles = (long long)g.tiles_m * g.tiles_n;
        long long S;
        if constexpr (CFG::BM == 64 && CFG::BN == 64) {
            S = splits_64x64(tiles, ktiles);
        } else {
            S = ((long long)kNumCus * split_slots + tiles - 1) / tiles;
            if (S > ktiles / 4) S = ktiles / 4;
        }
        if (S > kMaxSplits) S = kMaxSplits;
        if (S < 1) S = 1;
        while (S > 1 && tiles * S * CFG::BM * CFG::BN > (long long)kWsFloats) --S;
        if (tiles > kWsCounters) S = 1;
        if (S > 1) {
            const Workspace *w = get_workspace(stream);
            if (w == nullptr) {
                S = 1;
            } else {
                g.ws = w->partials;
                g.counters = w->counters;
                g.kt_per_split = (int)((ktiles + S - 1) / S);
                S = (ktiles + g.kt_per_split - 1) / g.kt_per_split;
            }
        }
        g.splits = (int)S;
        if (g.splits == 1) g.kt_per_split = ktiles;
    }
    unsigned workgroups = (unsigned)((long long)g.tiles_m * g.tiles_n * g.splits);
    if constexpr (CFG::STREAMK) {
        // One workgroup per CU, each owning an equal share of the tiles x
        // k-tiles iterations; each keeps at most two partial blocks (its first
        // and last tile) and every tile has one counter. When the shares cut
        // no tile (tiles a multiple of the grid) no workspace is needed; when
        // it is needed but missing, every workgroup takes one whole tile.
        const long long tiles = (long long)g.tiles_m * g.tiles_n;
        const long long per_cu = std::max(1, CFG::WAVES_PER_EU * 4 * 64 / CFG::NT);
        long long G = std::min(tiles * ktiles, (long long)kNumCus * per_cu);
        G = std::min(G, (long long)(kWsFloats / ((size_t)2 * CFG::BM * CFG::BN)));
        if (tiles % G != 0) {
            const Workspace *w = tiles <= kWsCounters ? get_workspace(stream) : nullptr;
            if (w == nullptr) {
                G = tiles;
            } else {
                g.ws = w->partials;
                g.counters = w->counters;
            }
        }
        workgroups = (unsigned)G;
        // All but the last full wave of tiles go data-parallel, so that only
        // one to two waves' worth is shared out (see sgemm_mfma32): shares
        // that start at different k offsets share no A or B panels in L2, and
        // over several waves that costs more than the balance gains (5000^3:
        // 113 TFLOP/s all stream-K, 125 with this split).
        const long long waves = tiles / G;
        g.sk_dp_tiles = (int)(waves > 1 ? (waves - 1) * G : 0);
    }
    if (!ta && !tb) return launch_t<CFG, false, false>(g, workgroups, stream);
    if (!ta && tb) return launch_t<CFG, false, true>(g, workgroups, stream);
    if (ta && !tb) return launch_t<CFG, true, false>(g, workgroups, stream);
    return launch_t<CFG, true, true>(g, workgroups, stream);
}

int run(int config, char transA, char transB, int M, int N, int K, float alpha, const float *A, int lda,
        const float *B, int ldb, float beta, float *C, int ldc, hipStream_t stream) {
    int rc = check_args(transA, transB, M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (rc != MISGEMM_SUCCESS) return rc;
    if (config < -1 || config >= kNumConfigs) return MISGEMM_BAD_CONFIG;
    if (M == 0 || N == 0) return MISGEMM_SUCCESS;
    // Tile-local offsets are 32-bit: row * ld for up to 256 rows plus a column.
    const long long max_ld = lda > ldb ? (lda > ldc ? lda : ldc) : (ldb > ldc ? ldb : ldc);
    if (max_ld * 256 + 256 > 0x7fffffffLL) return MISGEMM_TOO_LARGE;
    // Grid limits: one workgroup per output tile (x), and row blocks of the
    // skinny kernel (y, at most 65535).
    if ((long long)((N + 15) / 16) * ((M + 15) / 16) > 0x7fffffffLL) return MISGEMM_TOO_LARGE;

    if (alpha == 0.0f || K == 0) {
        if (beta == 1.0f) return MISGEMM_SUCCESS;
        dim3 grid((unsigned)((N + 255) / 256), (unsigned)(M < 65535 ? M : 65535));
        hipLaunchKernelGGL(scale_c, grid, dim3(256), 0, stream, C, M, N, ldc, beta);
        return hipGetLastError() == hipSuccess ? MISGEMM_SUCCESS : MISGEMM_LAUNCH_FAILED;
    }

    GemmArgs g;
    g.A = A;
    g.B = B;
    g.C = C;
    g.M = M;
    g.N = N;
    g.K = K;
    g.lda = lda;
    g.ldb = ldb;
    g.ldc = ldc;
    g.alpha = alpha;
    g.beta = beta;
    g.splits = 1;
    g.kt_per_split = 0;
    g.sk_dp_tiles = 0;
    g.ws = nullptr;
    g.counters = nullptr;
    g.vec_ab = aligned16(A) && aligned16(B) && lda % 4 == 0 && ldb % 4 == 0;
    g.vec_c = aligned16(C) && ldc % 4 == 0;
    const bool ta = op_t(transA), tb = op_t(transB);
    if (config < 0) config = select_config(transA, transB, M, N, K);
    if ((config == kCfgSkinny16 || config == kCfgBand) && (M + 2 * 16 - 1) / (2 * 16) > 65535)
        return MISGEMM_TOO_LARGE;
    hipError_t err;
    if (config >= kCfgLadderFirst && config <= kCfgLadderLast) {
        misgemm_ladder::LadderArgs la;
        la.A = A;
        la.B = B;
        la.C = C;
        la.M = M;
        la.N = N;
        la.K = K;
        la.lda = lda;
        la.ldb = ldb;
        la.ldc = ldc;
        la.alpha = alpha;
        la.beta = beta;
        la.vec_ab = g.vec_ab;
        la.vec_c = g.vec_c;
        err = misgemm_ladder::launch(config - kCfgLadderFirst, ta, tb, la, stream);
        return err == hipSuccess ? MISGEMM_SUCCESS : MISGEMM_LAUNCH_FAILED;
    }
    switch (config) {
        case kCfg128: err = launch_cfg<CfgL>(ta, tb, g, stream); break;
        case kCfg64: err = launch_cfg<CfgS>(ta, tb, g, stream); break;
        case kCfgSkinny16: err = launch_skinny(ta, tb, g, stream); break;
        case kCfgBand: err = launch_band(ta, tb, g, stream); break;
        case kCfg64Kg2: err = launch_cfg<CfgS2>(ta, tb, g, stream); break;
        case kCfg64Kg4: err = launch_cfg<CfgS4>(ta, tb, g, stream); break;
        case kCfg128Kg2: err = launch_cfg<CfgL2>(ta, tb, g, stream); break;
        case kCfg128W24: err = launch_cfg<CfgL24>(ta, tb, g, stream); break;
        case kCfg128W42: err = launch_cfg<CfgL42>(ta, tb, g, stream); break;
        case kCfg256x128: err = launch_cfg<CfgW>(ta, tb, g, stream); break;
        case kCfg128x256: err = launch_cfg<CfgT>(ta, tb, g, stream); break;
        case kCfg128W42Split: err = launch_cfg<CfgL42K>(ta, tb, g, stream, 1); break;
        case kCfg64Split: err = launch_cfg<CfgSK>(ta, tb, g, stream, 2); break;
        case kCfg128Split: err = launch_cfg<CfgLK>(ta, tb, g, stream, 1); break;
        case kCfg128x256x16: err = launch_cfg<CfgT16>(ta, tb, g, stream); break;
        case kCfg256x256: err = launch_cfg<CfgQ32>(ta, tb, g, stream); break;
        case kCfgStreamK1: err = launch_cfg<CfgL42S1>(ta, tb, g, stream); break;
        case kCfgStreamK2: err = launch_cfg<CfgL42S2>(ta, tb, g, stream); break;
        case kCfgStreamK256x128: err = launch_cfg<CfgWS>(ta, tb, g, stream); break;
        case kCfg256x256Dl: err = launch_cfg<CfgQ32D>(ta, tb, g, stream); break;
        case kCfg128W42Dl: err = launch_cfg<CfgL42D>(ta, tb, g, stream); break;
        case kCfg16x64: err = launch_cfg<Cfg16S>(ta, tb, g, stream); break;
        case kCfg16x64Kg2: err = launch_cfg<Cfg16S2>(ta, tb, g, stream); break;
        case kCfg16x64Kg4: err = launch_cfg<Cfg16S4>(ta, tb, g, stream); break;
        case kCfg16x64Split: err = launch_cfg<Cfg16SK>(ta, tb, g, stream, 2); break;
        case kCfg16x128W42: err = launch_cfg<Cfg16L42>(ta, tb, g, stream); break;
        case kCfg16StreamK1: err = launch_cfg<Cfg16L42S1>(ta, tb, g, stream); break;
        case kCfg16x128: err = launch_cfg<Cfg16L>(ta, tb, g, stream); break;
        case kCfg16x256x128: err = launch_cfg<Cfg16W>(ta, tb, g, stream); break;
        case kCfg16x128W42Dl: err = launch_cfg<Cfg16L42D>(ta, tb, g, stream); break;
        case kCfg16x64Kg4Dl: err = launch_cfg<Cfg16S4D>(ta, tb, g, stream); break;
        default: err = launch_cfg<CfgTS>(ta, tb, g, stream); break;   // kCfgStreamK128x256
    }
    return err == hipSuccess ? MISGEMM_SUCCESS : MISGEMM_LAUNCH_FAILED;
}

}  // namespace

extern "C" int mi_sgemm(char transA, char transB, int M, int N, int K, float alpha, const float *A, int lda,
                        const float *B, int ldb, float beta, float *C, int ldc, hipStream_t stream) {
    return run(-1, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

extern "C" int mi_sgemm_with_config(int config, char transA, char transB, int M, int N, int K, float alpha,
                                    const float *A, int lda, const float *B, int ldb, float beta, float *C,
                                    int ldc, hipStream_t stream) {
    if (config < 0) {
        int rc = check_args(transA, transB, M, N, K, alpha, A, lda, B, ldb, C, ldc);
        return rc != MISGEMM_SUCCESS ? rc : MISGEMM_BAD_CONFIG;
    }
    return run(config, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

extern "C" int mi_sgemm_select_config(char transA, char transB, int M, int N, int K) {
    if (!op_n(transA) && !op_t(transA)) return MISGEMM_BAD_TRANSA;
    if (!op_n(transB) && !op_t(transB)) return MISGEMM_BAD_TRANSB;
    if (M < 0) return MISGEMM_BAD_M;
    if (N < 0) return MISGEMM_BAD_N;
    if (K < 0) return MISGEMM_BAD_K;
    return select_config(transA, transB, M, N, K);
}

extern "C" int mi_sgemm_release_workspace(hipStream_t stream) {
    int dev = 0;
    if (!stream_device(stream, dev)) return MISGEMM_LAUNCH_FAILED;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    auto it = g_ws.find(std::make_pair(dev, stream));
    if (it == g_ws.end()) return MISGEMM_SUCCESS;
    DeviceGuard on_dev(dev);
    if (!on_dev.ok) return MISGEMM_LAUNCH_FAILED;
    if (hipStreamSynchronize(stream) != hipSuccess) return MISGEMM_LAUNCH_FAILED;
    const hipError_t e1 = hipFree(it->second.partials);
    const hipError_t e2 = hipFree(it->second.counters);
    g_ws.erase(it);
    return (e1 == hipSuccess && e2 == hipSuccess) ? MISGEMM_SUCCESS : MISGEMM_LAUNCH_FAILED;
}

extern "C" int mi_sgemm_config_count(void) { return kNumConfigs; }

extern "C" const char *mi_sgemm_config_name(int config) {
    if (config < 0 || config >= kNumConfigs) return nullptr;
    return kConfigs[config].name;
}

extern "C" const char *mi_sgemm_status_string(int status) {
    switch (status) {
        case MISGEMM_SUCCESS: return "success";
        case MISGEMM_BAD_TRANSA: return "invalid transA (expected N, n, T, t, C or c)";
        case MISGEMM_BAD_TRANSB: return "invalid transB (expected N, n, T, t, C or c)";
        case MISGEMM_BAD_M: return "M < 0";
        case MISGEMM_BAD_N: return "N < 0";
        case MISGEMM_BAD_K: return "K < 0";
        case MISGEMM_NULL_A: return "A is null but would be read";
        case MISGEMM_BAD_LDA: return "lda smaller than the stored row length of A";
        case MISGEMM_NULL_B: return "B is null but would be read";
        case MISGEMM_BAD_LDB: return "ldb smaller than the stored row length of B";
        case MISGEMM_NULL_C: return "C is null";
        case MISGEMM_BAD_LDC: return "ldc < max(1, N)";
        case MISGEMM_BAD_CONFIG: return "unknown kernel configuration id";
        case MISGEMM_TOO_LARGE: return "problem too large (leading dimension beyond 32-bit tile offsets, or grid too large)";
        case MISGEMM_LAUNCH_FAILED: return "HIP kernel launch failed";
        default: return "unknown status";
    }
}
