// Shared pieces of the tile kernels: vector types, launch arguments, the tile
// configuration, global -> LDS tile copies, epilogue stores, the XCD-aware tile
// order and split bookkeeping.
// Internal to libmisgemm: compiled only as part of misgemm.hip, whose header comment
// describes the kernels and the configurations built from them.
#ifndef MISGEMM_TILE_COMMON_H
#define MISGEMM_TILE_COMMON_H

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

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
    // SWZ: LDS rows unpadded, k-contiguous tiles chunk-swizzled (the layout
    // direct loads need), whether the tiles arrive directly or through
    // registers. 16 x 16 blocks use it: their fragment reads conflict on the
    // padded rows and not on these.
    static constexpr bool SWZ = DL_ || MI16_;
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

// n adjacent floats from LDS: one ds_read for n = 1, 2, 4; n = 3 (three
// blocks per lane row) is split by the compiler into a two- and a one-dword read.
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
template <> struct LdsVec<3> {
    static __device__ __forceinline__ void get(const float *p, float *out) { out[0] = p[0]; out[1] = p[1]; out[2] = p[2]; }
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
// Unpadded layout (UNPAD; required for direct global -> LDS loads, which
// write a wave's 64 chunks to 1 KB of consecutive LDS): rows are [R][CC].
// When SWZ (a k-contiguous tile, read as 16-byte runs down 8 consecutive
// rows), chunk c of row r sits at chunk position c ^ swz(r) -- r mod 8 for
// rows of 8 or more chunks, (r / 2) mod 4 for rows of 4 -- so those 8 reads
// fall on 8 different 16-byte bank groups, as the padding achieves otherwise.
template <int R, int CC, int NT, bool DL = false, bool SWZ = false, bool UNPAD = DL>
struct TileCopy {
    static constexpr int CPR = CC / 4;                  // chunks per row
    static constexpr int CHUNKS = R * CPR;
    static constexpr int PER_THREAD = CHUNKS / NT;
    static constexpr int STRIDE = UNPAD ? CC : CC + kLdsPad;
    static constexpr int LDS_FLOATS = R * STRIDE;
    static_assert(CC % 4 == 0 && CHUNKS % NT == 0, "tile must split evenly over the threads");
    static_assert(!DL || UNPAD, "direct loads fill unpadded rows");
    static_assert(!SWZ || (UNPAD && (CPR == 4 || CPR % 8 == 0)), "swizzle is for unpadded 16-wide or multiple-of-32-wide k-contiguous rows");
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

    // A complete k-tile of any tile, without branches: rows at or beyond
    // rows_left read row rows_left - 1 (rows_left and cols_left are >= 1).
    // VEC: 16-byte loads; a chunk starting beyond the last in-range 4-aligned
    // chunk reads that chunk. The caller guarantees a 16-byte aligned base
    // whose column offset is a multiple of 4 and ld % 4 == 0, so a clamped
    // chunk still ends inside its row's ld floats. Otherwise: 4-byte loads,
    // each column clamped to cols_left - 1, for any alignment and ld. The
    // extra values reach only outputs beyond M or N, which are never stored.
    template <bool VEC>
    __device__ __forceinline__ void load_clamped(const float *__restrict__ base, int ld, int rows_left,
                                                 int cols_left, int tid) {
        const int last_c = ((cols_left - 1) >> 2) << 2;
#pragma unroll
        for (int j = 0; j < PER_THREAD; ++j) {
            const int idx = tid + NT * j;
            const int r = idx / CPR, c = (idx % CPR) * 4;
            const int rr = r < rows_left ? r : rows_left - 1;
            if constexpr (VEC) {
                const int cc = c <= last_c ? c : last_c;
                v[j] = *reinterpret_cast<const f32x4 *>(base + (size_t)rr * ld + cc);
            } else {
                const float *p = base + (size_t)rr * ld;
                f32x4 t;
#pragma unroll
                for (int e = 0; e < 4; ++e) t[e] = p[c + e < cols_left ? c + e : cols_left - 1];
                v[j] = t;
            }
        }
    }

    // The k-tail tile (its k extent shorter than the tile's), without
    // branches: loaded as load_clamped does, then every element at or beyond
    // the k extent is set to zero, since those enter the sum of every output.
    // K_ROWS: k runs along the tile's rows (rows_left is the k extent) rather
    // than its columns (cols_left is). A 16-byte chunk that starts below the
    // k extent is read whole: it starts 16-byte aligned inside its row, so it
    // stays inside the row's ld floats and its page.
    template <bool VEC, bool K_ROWS>
    __device__ __forceinline__ void load_ktail(const float *__restrict__ base, int ld, int rows_left, int cols_left,
                                               int tid) {
        const int last_c = ((cols_left - 1) >> 2) << 2;
#pragma unroll
        for (int j = 0; j < PER_THREAD; ++j) {
            const int idx = tid + NT * j;
            const int r = idx / CPR, c = (idx % CPR) * 4;
            const int rr = r < rows_left ? r : rows_left - 1;
            f32x4 t;
            if constexpr (VEC) {
                const int cc = c <= last_c ? c : last_c;
                t = *reinterpret_cast<const f32x4 *>(base + (size_t)rr * ld + cc);
            } else {
                const float *p = base + (size_t)rr * ld;
#pragma unroll
                for (int e = 0; e < 4; ++e) t[e] = p[c + e < cols_left ? c + e : cols_left - 1];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (K_ROWS ? r >= rows_left : c + e >= cols_left) t[e] = 0.0f;
            v[j] = t;
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

// The n adjacent C values of one row that an epilogue batch will update: one
// vector load when `whole`, else the first `valid` elements (the rest zero).
template <int n>
__device__ __forceinline__ void load_run(const float *p, float (&c)[n], bool whole, int valid) {
    if constexpr (n == 2 || n == 4) {
        if (whole) {
            using V = typename VecOf<n>::type;
            const V v = *reinterpret_cast<const V *>(p);
#pragma unroll
            for (int b = 0; b < n; ++b) c[b] = v[b];
            return;
        }
    }
#pragma unroll
    for (int b = 0; b < n; ++b) c[b] = b < valid ? p[b] : 0.0f;
}

// C <- out + beta*c over n adjacent elements of one row, c being those
// elements' values loaded beforehand (unused when beta == 0); one vector store
// when `whole`, else the first `valid` elements.
template <int n>
__device__ __forceinline__ void put_run(float *p, const float (&out)[n], const float (&c)[n], float beta, bool whole,
                                        int valid) {
    float v[n];
#pragma unroll
    for (int b = 0; b < n; ++b) v[b] = beta != 0.0f ? fmaf(beta, c[b], out[b]) : out[b];
    if constexpr (n == 2 || n == 4) {
        if (whole) {
            using V = typename VecOf<n>::type;
            V w;
#pragma unroll
            for (int b = 0; b < n; ++b) w[b] = v[b];
            *reinterpret_cast<V *>(p) = w;
            return;
        }
    }
#pragma unroll
    for (int b = 0; b < n; ++b)
        if (b < valid) p[b] = v[b];
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

}  // namespace

#endif  // MISGEMM_TILE_COMMON_H
