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
//   * Edges: a k-tile that crosses K takes a guarded load path that reads
//     only in-range elements and selects zero for the rest (the zero-fill of
//     the klklkl10086 page, 01-Shared Memory Tiling); so do the edge tiles of
//     the 256 x 256 tiles, and all its tiles when A or B cannot be read with
//     16-byte loads. The other tiles keep the straight-line rounds for every
//     complete k-tile with clamped loads (16-byte, or 4-byte in a separate
//     instantiation for unaligned operands), whose extra values only reach
//     outputs beyond M or N, and load the k tail the same way with the
//     elements past K selected to zero. Stores are masked to i < M, j < N.
//   * Epilogue: C = alpha*acc + beta*C fused into the store (itan.pw page,
//     sections 3.4-3.5); when beta == 0, C is not read, else a batch of C
//     values is loaded before any of them is stored.
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
//
// Files: tile_common.h (tile configuration, global -> LDS copies, stores,
// tile order, split bookkeeping), tile_kernel.h (MFMA fragments and the tile
// kernel), skinny_kernels.h (few-row kernels, helpers), scratch.hip (the
// static device scratch of mi_sgemm_noalloc); this file holds the
// configuration table, shape-class selection, workspace, launch and C ABI.

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
#include "scratch.h"
#include "skinny_kernels.h"
#include "tile_common.h"
#include "tile_kernel.h"

namespace {

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
using Cfg16Q12 = TileCfg<192, 192, 32, 4, 3, 1, 0, false, false, false, true>;   // 12 waves, 48 x 64 per wave
using Cfg16S4W = TileCfg<64, 64, 32, 2, 1, 4, 0, false, false, false, true>;      // 4 k-groups of 2 waves, 32 x 64 per wave
using Cfg16L42S2 = TileCfg<128, 128, 32, 4, 2, 1, 4, false, true, false, true>;   // stream-K, two workgroups per CU
using Cfg16L42K2 = TileCfg<128, 128, 32, 4, 2, 2, 0, false, false, false, true>;   // 2 k-groups of 8 waves

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
    kCfg16x192W43 = 37,
    kCfg16x64W21Kg4 = 38,
    kCfg16StreamK2 = 39,
    kCfg16x128W42Kg2 = 40,
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
    {"mfma16_192x192x32_w4x3", Cfg16Q12::BM, Cfg16Q12::BN, Cfg16Q12::NT},
    {"mfma16_64x64x32_w2x1_kg4", Cfg16S4W::BM, Cfg16S4W::BN, Cfg16S4W::NT},
    {"mfma16_128x128x32_w4x2_streamk_2wg", Cfg16L42S2::BM, Cfg16L42S2::BN, Cfg16L42S2::NT},
    {"mfma16_128x128x32_w4x2_kg2", Cfg16L42K2::BM, Cfg16L42K2::BN, Cfg16L42K2::NT},
};
constexpr int kSkinnyMaxM = 32;
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);
static_assert(kNumConfigs == kCfg16x128W42Kg2 + 1, "one ConfigId per kConfigs entry");
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
    // One round of 128 x 128 tiles (at most one per CU) with long k (K >= 2048):
    // two k-groups of eight waves per tile (four waves per SIMD), 0.5-2.5%
    // faster than one group (2048^3 NN 131.0 -> 129.6 us, TN 2048 x 2048 x 8192
    // 498.9 -> 486.8); at K <= 1024, or with two tiles per CU, no faster or
    // slower.
    const int cfg128 = (t128 <= kNumCus && K >= 2048) ? kCfg16x128W42Kg2 : kCfg16x128W42;
    const long long kt = (K + 31) / 32;
    // Short k (K <= 256) over at least 128 tiles of 64 x 64: the plain 64 x 64
    // tile, whose k-loop is too short for k-groups, splits or stream-K to pay
    // (1024 x 2048 x 256 TT: 53% of peak vs 47% two k-groups, 33% 128 x 128),
    // unless 128 x 128 tiles spread over the CUs as evenly (each weighed by
    // the cube of its grid's filled fraction): then 128 x 128, 3-6% faster
    // (2048 x 4096 x 256: 5.7%; 1792^3 x 256 TT 5.4%; 46 seeded shapes).
    auto fill3 = [&](int b) {
        const double u = (double)M * N / ((double)tiles(b, b) * b * b);
        return u * u * u;
    };
    if (kt <= 8 && t64 >= 128)
        return cu_balance(t128) * fill3(128) >= cu_balance(t64) * fill3(64) ? cfg128 : kCfg16x64;
    if (t128 >= kNumCus) {
        const bool ta = op_t(transA), tb = op_t(transB);
        // Big tiles (one workgroup per CU) lose to 128 x 128 (two per CU)
        // when K is short and the grid fills the chip only once; with both
        // transposed, 256 x 128 is the one that gains (the register-staged
        // 256 x 256 and 128 x 256 x 16 tiles do not).
        const bool big_ok = !(K < 2048 && t128 < 4 * kNumCus);
        const bool tt = ta && tb;
        const bool wide = !tt && M < N;    // 128 x 256 rather than 256 x 128
        // With A transposed, the 256 x 256 tile with direct-to-LDS loads: for
        // TT the register-staged one spills (960 vs 989 us for 256 x 128 at
        // 4096^3); for TN it is 0.6-1.7% faster than the register-staged one
        // (4096^3 947 vs 960 us, 8192 x 8192 x 2048 1904 vs 1929, 4000^3 1028
        // vs 1035).
        // Its edge tiles run the guarded k-loop (the smaller tiles clamp their
        // edge loads instead), so a 256 x 256 grid that does not divide M and N
        // scores lower (4000^3: 1022 us against 951 for 128 x 256 x 16).
        const double ragged = (M % 256 != 0 || N % 256 != 0) ? 0.92 : 1.0;
        // Edge tiles that cross M or N run whole, so each tile size is also
        // weighed by the cube of the fraction of its grid that holds outputs
        // (1 when the tiles divide M and N). Fitted on 90 seeded shapes with M,
        // N, K multiples of 4 in 512..4096 (mean regret 1.37% -> 1.12%) and
        // checked on 90 others (1.59% -> 1.27%); shapes that the tiles divide
        // pick as before.
        auto filled = [&](int bm, int bn) {
            const double u = (double)M * N / ((double)tiles(bm, bn) * bm * bn);
            return u * u * u;
        };
        const double f_wide = wide ? filled(128, 256) : filled(256, 128);
        const double s_q = big_ok ? (tt ? 1.065 : 1.044) * ragged * cu_balance(tiles(256, 256)) * filled(256, 256)
                                  : -1.0;
        const double s_b4 = big_ok ? (tt ? 1.0 : 1.038) * cu_balance(tiles(128, 256), 2) * filled(128, 256) : -1.0;
        const double s_b8 =
            big_ok ? (tt ? 1.034 : 1.024) * cu_balance(wide ? tiles(128, 256) : tiles(256, 128)) * f_wide : -1.0;
        // The 64 x 64 tile gains on short k (K <= 512), where every larger tile
        // spends a bigger share of its time outside the k-loop.
        const double s_128 = cu_balance(t128) * filled(128, 128);
        const double s_64 = (kt <= 16 ? 0.90 : 0.87) * cu_balance(t64) * filled(64, 64);
        // Stream-K fills every CU slot whatever the tile count: with the
        // 256 x 128 / 128 x 256 tile where big tiles pay, else 128 x 128. Not
        // below K = 1024, where its shares are too short (3584 x 2560 x 512 TT:
        // 65% of peak vs 74% for 64 x 64).
        const bool sk_ok = sk_iters >= 8LL * 2 * kNumCus && kt >= 32;
        const double s_skb = (sk_ok && big_ok) ? 0.955 * f_wide : -1.0;
        const double s_sk = sk_ok ? 0.925 * filled(128, 128) : -1.0;
        // With neither operand transposed, stream-K over 128 x 128 tiles of
        // 16 x 16 blocks, one workgroup per CU, beats the big-tile stream-K
        // (n = 2304: 193 vs 202 us; 3840: 839 vs 854); so it does for TN
        // (3584 x 4096 x 1024: 82% of peak vs 76%; 2048 x 3072 x 2048: 83% vs
        // 75%) and for TT from K = 2048 (1792 x 3584 x 2048: 80% vs 76%), while
        // NT keeps the big-tile stream-K (1792 x 3584 x 4096: 85% vs 83%).
        const double s_sk16 = (sk_ok && (!tb || (ta && kt >= 64))) ? 0.965 * filled(128, 128) : -1.0;
        // The 192 x 192 tile (twelve waves, one workgroup per CU), on grids
        // that fill at least 88% of its waves, also at short K: 3072^3 410 us
        // against 427 for stream-K, 6144^3 3231 against 3273 for 128 x 128,
        // 3072 x 3072 x 512 76.2 against 81.8 for 64 x 64, 3000^3 403 against
        // 427. Weight fitted on 84 seeded shapes near the boundary (mean regret
        // 1.28% -> 0.63%); on 200-220 tiles it loses to 128 x 128 by ~9%.
        const double b_192 = cu_balance(tiles(192, 192));
        const double s_192 = b_192 >= 0.88 ? 1.03 * b_192 * filled(192, 192) : -1.0;
        const double best = fmax(fmax(fmax(s_q, fmax(s_skb, s_sk)), fmax(s_b4, s_b8)),
                                 fmax(fmax(fmax(s_128, s_64), s_sk16), s_192));
        if (best == s_q) return ta ? kCfg256x256Dl : kCfg256x256;
        if (best == s_192) return kCfg16x192W43;
        // With neither operand transposed and at least 400 tiles of 128 x 128,
        // two stream-K workgroups per CU (four waves per SIMD): 3328^3-3840^3
        // 1.5-2.6% faster, 2560^3 0.8%, 30 seeded shapes of 400-1428 tiles
        // +1.2% on average, NN ones +0.3% to +6.1%; with A transposed it was
        // up to 5% slower, and below two waves of tiles (n <= 1792) 4-18%.
        if (best == s_sk16) return (!ta && !tb && t128 >= 400) ? kCfg16StreamK2 : kCfg16StreamK1;
        if (best == s_skb) return wide ? kCfgStreamK128x256 : kCfgStreamK256x128;
        if (best == s_sk) return kCfgStreamK2;
        if (best == s_b4) return kCfg128x256x16;
        if (best == s_b8) return wide ? kCfg128x256 : kCfg256x128;
        return best == s_128 ? cfg128 : kCfg16x64;
    }
    // Stream-K over 128 x 128 tiles, or split-K over 64 x 64 tiles where the
    // timing models put it first. Stream-K's time is fitted on 103 seeded
    // shapes with 64..255 such tiles (15.55 us + 1.967 us per 128 x 128 x 32
    // iteration per CU, mean error 1.4%); the 64 x 64 model runs about 10%
    // long. Scored on 270 seeded random shapes mean regret 1.03% -> 0.73% (on
    // two further scans 0.94% -> 0.89%).
    auto sk_or_split = [&]() {
        const double t_sk = 15.55 + 1.967 * (double)t128 * kt / kNumCus;
        const double t_sp = model_64x64_us(t64, (int)kt, 1, splits_64x64(t64, (int)kt));
        return 0.9 * t_sp < t_sk ? kCfg16x64Split : kCfg16StreamK1;
    };
    // 128..255 tiles of 128 x 128 with enough k-work per workgroup: stream-K,
    // one workgroup per CU (1792 x 1280 x 4096 TN, 140 tiles: 78% of peak vs
    // 58% for 64 x 64; 768 x 3072 x 1024 TN, 144 tiles: 62% vs 56%). At 128
    // tiles it needs 20 k-tiles per workgroup (1024 x 2048 x 1024 with 16:
    // 41.6 vs 38.8 us for 64 x 64).
    // Short k (K < 1024) on up to 229 tiles of 128 x 128 with at least two
    // waves of 64 x 64 tiles: the plain 64 x 64 tile; stream-K shares are too
    // short there and 128 x 128 spreads unevenly (1072 x 2768 x 764 NT: 43.8
    // us against 54.3 for stream-K; 1536 x 2048 x 512: 57% of peak vs 49% for
    // 128 x 128).
    // Below 230 tiles of 128 x 128, where the plain 64 x 64 tile is picked,
    // 128 x 128 instead when its grid spreads nearly as evenly (at least 0.9
    // of the 64 x 64 tile's balance x filled^3): 3-7% faster there (NN
    // 1280 x 2560 x 512 5.1%, 1972 x 1644 x 788 6.8%; nine regret scans, mean
    // regret 0.72% -> 0.67%), where at 0.875 (t128 >= 400, K = 512) 64 x 64
    // still led by 6%.
    auto plain64 = [&]() {
        return cu_balance(t128) * fill3(128) >= 0.9 * cu_balance(t64) * fill3(64) ? cfg128 : kCfg16x64;
    };
    if (t128 < 230 && kt < 32 && t64 >= 2 * kNumCus) return plain64();
    // 461..511 tiles of 64 x 64 fill two k-group workgroups per CU to 90% or
    // more, which beats stream-K (1844 x 1056 x 2032 NN: 73.3 us against 81.6;
    // 828 x 2392 x 3588 NT: 7.9% faster).
    if (t128 < 230 && 10 * t64 >= 9 * 2 * kNumCus && t64 < 2 * kNumCus) return kCfg16x64Kg2;
    // From about 230 tiles the data-parallel 128 x 128 tile fills the CUs well
    // enough (3584 x 1152 x 1024 NT, 252 tiles: 79% of peak vs 69%).
    if (t128 < 230 &&
        ((t128 >= 144 && sk_iters >= 16LL * kNumCus) || (t128 >= 128 && sk_iters >= 20LL * kNumCus)))
        return sk_or_split();
    if (t128 >= 3 * kNumCus / 4) return cfg128;
    // 72..127 tiles with long k (K >= 2048): stream-K again rather than k-groups
    // or split-K over 64 x 64 tiles (1536 x 768 x 4096 TN: 71% of peak vs 63%;
    // 1024 x 1280 x 4096 NT: 73% vs 70%).
    if (t128 >= 72 && kt >= 64) return sk_or_split();
    if (t64 >= 2 * kNumCus) return plain64();
    // 257..511 tiles of 64 x 64 that fill 75-85% of two workgroup slots per
    // CU, with enough k-work and B not transposed: stream-K over 128 x 128
    // tiles keeps every CU busy for the whole k-range (NN 1280^3, beta 0.5:
    // 48.0 vs 49.2 us for two k-groups; 1280 x 1280 x 2560: 78.6 vs 90.9).
    // Fuller grids keep two k-groups (1408^3: 51.4 vs 55.2 us), and so do
    // short k-work (1280 x 1280 x 640: 26.3 vs 29.9 us) and TT (1280^3, beta
    // 0.5: 49.8 vs 53.7 us).
    if (!op_t(transB) && t64 > kNumCus && 4 * t64 >= 3 * 2 * kNumCus && 100 * t64 < 85 * 2 * kNumCus &&
        t128 >= 96 && sk_iters >= 3000)
        return kCfg16StreamK1;
    // 257..511 tiles of 64 x 64: two k-groups unless their workgroups would
    // leave the CU slots badly filled, or the 64 x 64 timing model splits k
    // (two or more splits: 384 tiles at K <= 1024); then split-K over
    // workgroups, whose smaller workgroups spread more evenly (TT 2048 x 768 x
    // 1024: 16.7% faster than two k-groups, NN 1536 x 1024 x 512 11.4%).
    if (t64 > kNumCus)
        return ((double)t64 / (2 * kNumCus) >= 0.75 && splits_64x64(t64, (int)kt) < 2) ? kCfg16x64Kg2
                                                                                       : kCfg16x64Split;
    // Up to 256 tiles of 64 x 64: four k-groups or split-K over workgroups,
    // whichever the timing model puts first.
    const int ktiles = (K + 31) / 32;
    const double t_split = model_64x64_us(t64, ktiles, 1, splits_64x64(t64, ktiles));
    if (t_split < model_64x64_us(t64, ktiles, 4, 1)) return kCfg16x64Split;
    // Four k-groups of two waves (32 x 64 each, a third fewer LDS reads per
    // MFMA) rather than of four, where the grid fills at least 224 of the 256
    // CUs, A is not transposed and K has no tail: 1.0-5% faster on 40 such
    // shapes (NN 1024^3 21.53 -> 20.93 us, NT 21.29 -> 20.93; 1024 x 960 x
    // 512 13.40 -> 12.81); on partly filled grids, with a k tail or with A
    // transposed it is up to 4% slower.
    if (!op_t(transA) && K % 32 == 0 && t64 >= 224) return kCfg16x64W21Kg4;
    return kCfg16x64Kg4;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Whether the tile has a 4-byte straight-line instantiation for this op pair:
// every clamping tile, except the forms whose clamped element addresses do
// not fit the register budget (they spilled: the 128 x 256 x 16 tile, the
// two-workgroup stream-K tiles, the 16 x 16 128 x 128 w4x2 tile other than NT
// and its two-k-group form, and the 32 x 32 128 x 128 w2x4 / w4x2 tiles for
// TN), and the 192 x 192
// tile, whose edge tiles clamp but which has no 4-byte form. mi_sgemm routes
// operands without 16-byte loads away from these tiles (unaligned_substitute);
// when one is forced, it runs the guarded rounds.
template <class CFG, bool TA, bool TB>
constexpr bool kScalarForm =
    kClampEdge<CFG> && !std::is_same_v<CFG, CfgT16> && !std::is_same_v<CFG, CfgL42S2> &&
    !std::is_same_v<CFG, Cfg16Q12> && !std::is_same_v<CFG, Cfg16L42S2> && !std::is_same_v<CFG, Cfg16L42K2> &&
    !(std::is_same_v<CFG, Cfg16L42> && !(!TA && TB)) &&
    !((std::is_same_v<CFG, CfgL24> || std::is_same_v<CFG, CfgL42>) && TA && !TB);

// Operands that cannot be read with 16-byte loads: the pick for aligned ones
// replaced by a tile whose 4-byte straight-line rounds exist. The 256 x 256
// tiles have none (4096 x 4096 x 4095 NN: 1003 us on 256 x 128 against 1245;
// TT on 128 x 256: 1006 against 1253); for the others the replacement was the
// fastest measured (MI355X, pointers one float off 16 bytes):
//   128 x 256 x 16 -> 256 x 128 / 128 x 256   (4000^3 NN: 982 us vs 1046)
//   two-workgroup stream-K (32 x 32 or 16 x 16 blocks), 192 x 192
//                              -> 16 x 16 stream-K (2304 x 2304 x 1024 NT: 97.9
//                                 vs 106.0 us; TT: 106.2 vs 117.4)
//   16 x 16 128 x 128 w4x2 (not NT) -> 256 x 128 on a grid it fills evenly
//                                     (2048 x 4096 x 1024 NN / TN / TT: 136 /
//                                     145 / 139 us vs 153 / 174 / 176), else
//                                     the 16 x 16 stream-K tile (2048^3 NN:
//                                     148.5 vs 151.1 us)
int unaligned_substitute(int config, bool ta, bool tb, int M, int N) {
    const bool wide = M < N;
    // The two-k-group 16 x 16 128 x 128 tile: as the one-group tile.
    if (config == kCfg16x128W42Kg2) config = kCfg16x128W42;
    auto tiles = [&](int bm, int bn) { return (long long)((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    switch (config) {
        case kCfg256x256:
        case kCfg256x256Dl: return (ta && tb) ? kCfg128x256 : kCfg256x128;
        case kCfg128x256x16: return wide && !(ta && tb) ? kCfg128x256 : kCfg256x128;
        case kCfgStreamK2:
        case kCfg16StreamK2:
        case kCfg16x192W43: return kCfg16StreamK1;
        case kCfg16x128W42:
            if (!ta && tb) return config;
            return (tiles(256, 128) >= kNumCus && cu_balance(tiles(256, 128)) >= 0.9) ? kCfg256x128
                                                                                        : kCfg16StreamK1;
        default: return config;
    }
}

template <class CFG, bool TA, bool TB>
hipError_t launch_t(const GemmArgs &g, unsigned workgroups, hipStream_t stream) {
    dim3 grid(workgroups);
    dim3 block(CFG::NT);
    // Operands without 16-byte loads: the 4-byte straight-line instantiation
    // where the tile has one, else the guarded rounds of the usual kernel.
    if constexpr (kScalarForm<CFG, TA, TB>) {
        if (!g.vec_ab) {
            hipLaunchKernelGGL((sgemm_mfma32<CFG, TA, TB, true>), grid, block, 0, stream, g);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((sgemm_mfma32<CFG, TA, TB>), grid, block, 0, stream, g);
    return hipGetLastError();
}

// Workspace for the split-K reduction, one per (device, stream) so that calls
// on different streams never share partials or counters. Allocated on the
// first call that needs it and kept until mi_sgemm_release_workspace or the
// end of the process. mi_sgemm_noalloc uses the device's static scratch of the
// same capacity instead, so both make the same split plans.
constexpr size_t kWsFloats = size_t(16) << 20;  // 64 MiB of partial blocks
constexpr int kWsCounters = 1 << 16;
static_assert(kWsFloats == misgemm_scratch::kPartialFloats && kWsCounters == misgemm_scratch::kCounters,
              "the static scratch has a stream workspace's capacity");

struct Workspace {
    float *partials = nullptr;
    int *counters = nullptr;
    // Handed out while the stream was being captured into a graph: the graph
    // holds its address, so it is never freed.
    bool pinned = false;
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

// Whether work enqueued on `stream` now would be captured into a graph (an
// unknown status counts as capturing).
bool capturing(hipStream_t stream) {
    if (stream == nullptr) return false;
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &capture) != hipSuccess) {
        (void)hipGetLastError();
        return true;
    }
    return capture != hipStreamCaptureStatusNone;
}

const Workspace *get_workspace(hipStream_t stream) {
    int dev = 0;
    if (!stream_device(stream, dev)) return nullptr;
    const bool in_capture = capturing(stream);
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    auto key = std::make_pair(dev, stream);
    auto it = g_ws.find(key);
    if (it != g_ws.end()) {
        if (in_capture) it->second.pinned = true;
        return &it->second;
    }
    // No allocation while the stream is being captured into a graph: the
    // captured call runs unsplit instead.
    if (in_capture) return nullptr;
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

// Where a call's split-K exchange space comes from: the stream's workspace
// (mi_sgemm, allocated on first use) or a fixed one (mi_sgemm_noalloc: the
// device's static scratch, never allocated). With a fixed one, a plan whose
// partial blocks or counters would not fit is refused: `overflow` is set and
// the launcher enqueues nothing.
struct WsSource {
    const Workspace *fixed = nullptr;
    bool overflow = false;
    const Workspace *get(hipStream_t stream, size_t floats, long long counters) {
        if (fixed == nullptr) return get_workspace(stream);
        if (floats > kWsFloats || counters > (long long)kWsCounters) {
            overflow = true;
            return nullptr;
        }
        return fixed;
    }
};

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

hipError_t launch_band(bool ta, bool tb, const GemmArgs &g, hipStream_t stream, WsSource &wsrc) {
    const int mb = g.M <= 16 ? 1 : 2;
    SplitArgs sa;
    sa.g = g;
    sa.ws = nullptr;
    sa.counters = nullptr;
    // Unguarded instantiation: whole bands, whole 16-row chunks, 16-byte loads.
    const bool fast = g.vec_ab && g.N % kBandCols == 0 && g.K % 16 == 0;
    int S = band_splits(g.M, g.N, g.K, mb, fast);
    if (S > 1) {
        const long long tiles = (long long)((g.N + kBandCols - 1) / kBandCols) * ((g.M + 16 * mb - 1) / (16 * mb));
        const Workspace *w = wsrc.get(stream, (size_t)tiles * S * 16 * mb * kBandCols, tiles);
        if (wsrc.overflow) return hipSuccess;
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
hipError_t launch_cfg(bool ta, bool tb, GemmArgs &g, hipStream_t stream, WsSource &wsrc, int split_slots = 0) {
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
            const Workspace *w = wsrc.get(stream, (size_t)tiles * S * CFG::BM * CFG::BN, tiles);
            if (wsrc.overflow) return hipSuccess;
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
            // Partial slots 0 .. 2G-1 and one counter per tile.
            const Workspace *w =
                tiles <= kWsCounters ? wsrc.get(stream, (size_t)2 * G * CFG::BM * CFG::BN, tiles) : nullptr;
            if (wsrc.overflow) return hipSuccess;
            if (w == nullptr) {
                G = tiles;
            } else {
                g.ws = w->partials;
                g.counters = w->counters;
            }
        }
        workgroups = (unsigned)G;
        // Every full wave of tiles goes data-parallel and only the remainder
        // is shared out (see sgemm_mfma32): shares that start at different k
        // offsets share no A or B panels in L2, and over several waves that
        // costs more than the balance gains (5000^3: 113 TFLOP/s all stream-K,
        // 125 with whole waves data-parallel). With only the remainder shared,
        // its tiles split into near-equal k-ranges that co-resident workgroups
        // walk together: 3072^3 moves 487 instead of 1058 MB beyond L2 (L2 hit
        // 74% instead of 45%) at the same speed as sharing the last full wave
        // too.
        // Every share must hold at least one iteration: the exchange counts
        // each workgroup between a tile's first and last owner as one of its
        // segments. When the remainder has fewer iterations than the grid, the
        // last full wave is shared out with it, so that every share spans at
        // least one k-tile.
        const long long waves = tiles / G, rem = tiles - waves * G;
        g.sk_dp_tiles = (int)((rem > 0 && rem * ktiles < G && waves > 0) ? (waves - 1) * G : waves * G);
    }
    if (!ta && !tb) return launch_t<CFG, false, false>(g, workgroups, stream);
    if (!ta && tb) return launch_t<CFG, false, true>(g, workgroups, stream);
    if (ta && !tb) return launch_t<CFG, true, false>(g, workgroups, stream);
    return launch_t<CFG, true, true>(g, workgroups, stream);
}

int run(int config, char transA, char transB, int M, int N, int K, float alpha, const float *A, int lda,
        const float *B, int ldb, float beta, float *C, int ldc, hipStream_t stream, bool noalloc = false) {
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
    if (config < 0) {
        config = select_config(transA, transB, M, N, K);
        if (!g.vec_ab) config = unaligned_substitute(config, ta, tb, M, N);
    }
    if ((config == kCfgSkinny16 || config == kCfgBand) && (M + 2 * 16 - 1) / (2 * 16) > 65535)
        return MISGEMM_TOO_LARGE;
    WsSource wsrc;
    Workspace fixed;
    if (noalloc) {
        // The device's static scratch; on the first call for a device, clear
        // its counters on this stream unless the stream is being captured
        // (the array starts zero-filled, and every split product leaves its
        // counters at zero).
        int dev = 0;
        bool first = false;
        if (!stream_device(stream, dev) ||
            !misgemm_scratch::device_scratch(dev, &fixed.partials, &fixed.counters, &first))
            return MISGEMM_LAUNCH_FAILED;
        if (first && !capturing(stream)) {
            hipLaunchKernelGGL(zero_ints, dim3((kWsCounters + 255) / 256), dim3(256), 0, stream, fixed.counters,
                               kWsCounters);
            if (hipGetLastError() != hipSuccess) return MISGEMM_LAUNCH_FAILED;
        }
        wsrc.fixed = &fixed;
    }
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
        case kCfg128: err = launch_cfg<CfgL>(ta, tb, g, stream, wsrc); break;
        case kCfg64: err = launch_cfg<CfgS>(ta, tb, g, stream, wsrc); break;
        case kCfgSkinny16: err = launch_skinny(ta, tb, g, stream); break;
        case kCfgBand: err = launch_band(ta, tb, g, stream, wsrc); break;
        case kCfg64Kg2: err = launch_cfg<CfgS2>(ta, tb, g, stream, wsrc); break;
        case kCfg64Kg4: err = launch_cfg<CfgS4>(ta, tb, g, stream, wsrc); break;
        case kCfg128Kg2: err = launch_cfg<CfgL2>(ta, tb, g, stream, wsrc); break;
        case kCfg128W24: err = launch_cfg<CfgL24>(ta, tb, g, stream, wsrc); break;
        case kCfg128W42: err = launch_cfg<CfgL42>(ta, tb, g, stream, wsrc); break;
        case kCfg256x128: err = launch_cfg<CfgW>(ta, tb, g, stream, wsrc); break;
        case kCfg128x256: err = launch_cfg<CfgT>(ta, tb, g, stream, wsrc); break;
        case kCfg128W42Split: err = launch_cfg<CfgL42K>(ta, tb, g, stream, wsrc, 1); break;
        case kCfg64Split: err = launch_cfg<CfgSK>(ta, tb, g, stream, wsrc, 2); break;
        case kCfg128Split: err = launch_cfg<CfgLK>(ta, tb, g, stream, wsrc, 1); break;
        case kCfg128x256x16: err = launch_cfg<CfgT16>(ta, tb, g, stream, wsrc); break;
        case kCfg256x256: err = launch_cfg<CfgQ32>(ta, tb, g, stream, wsrc); break;
        case kCfgStreamK1: err = launch_cfg<CfgL42S1>(ta, tb, g, stream, wsrc); break;
        case kCfgStreamK2: err = launch_cfg<CfgL42S2>(ta, tb, g, stream, wsrc); break;
        case kCfgStreamK256x128: err = launch_cfg<CfgWS>(ta, tb, g, stream, wsrc); break;
        case kCfg256x256Dl: err = launch_cfg<CfgQ32D>(ta, tb, g, stream, wsrc); break;
        case kCfg128W42Dl: err = launch_cfg<CfgL42D>(ta, tb, g, stream, wsrc); break;
        case kCfg16x64: err = launch_cfg<Cfg16S>(ta, tb, g, stream, wsrc); break;
        case kCfg16x64Kg2: err = launch_cfg<Cfg16S2>(ta, tb, g, stream, wsrc); break;
        case kCfg16x64Kg4: err = launch_cfg<Cfg16S4>(ta, tb, g, stream, wsrc); break;
        case kCfg16x64Split: err = launch_cfg<Cfg16SK>(ta, tb, g, stream, wsrc, 2); break;
        case kCfg16x128W42: err = launch_cfg<Cfg16L42>(ta, tb, g, stream, wsrc); break;
        case kCfg16StreamK1: err = launch_cfg<Cfg16L42S1>(ta, tb, g, stream, wsrc); break;
        case kCfg16x128: err = launch_cfg<Cfg16L>(ta, tb, g, stream, wsrc); break;
        case kCfg16x256x128: err = launch_cfg<Cfg16W>(ta, tb, g, stream, wsrc); break;
        case kCfg16x128W42Dl: err = launch_cfg<Cfg16L42D>(ta, tb, g, stream, wsrc); break;
        case kCfg16x64Kg4Dl: err = launch_cfg<Cfg16S4D>(ta, tb, g, stream, wsrc); break;
        case kCfg16x192W43: err = launch_cfg<Cfg16Q12>(ta, tb, g, stream, wsrc); break;
        case kCfg16x64W21Kg4: err = launch_cfg<Cfg16S4W>(ta, tb, g, stream, wsrc); break;
        case kCfg16StreamK2: err = launch_cfg<Cfg16L42S2>(ta, tb, g, stream, wsrc); break;
        case kCfg16x128W42Kg2: err = launch_cfg<Cfg16L42K2>(ta, tb, g, stream, wsrc); break;
        default: err = launch_cfg<CfgTS>(ta, tb, g, stream, wsrc); break;   // kCfgStreamK128x256
    }
    if (wsrc.overflow) return MISGEMM_SCRATCH_TOO_SMALL;
    return err == hipSuccess ? MISGEMM_SUCCESS : MISGEMM_LAUNCH_FAILED;
}

}  // namespace

extern "C" int mi_sgemm(char transA, char transB, int M, int N, int K, float alpha, const float *A, int lda,
                        const float *B, int ldb, float beta, float *C, int ldc, hipStream_t stream) {
    return run(-1, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

extern "C" int mi_sgemm_noalloc(char transA, char transB, int M, int N, int K, float alpha, const float *A,
                                int lda, const float *B, int ldb, float beta, float *C, int ldc,
                                hipStream_t stream) {
    return run(-1, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, true);
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
    // A captured graph's kernels hold this workspace's address: keep it.
    if (it->second.pinned) return MISGEMM_WORKSPACE_CAPTURED;
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
        case MISGEMM_SCRATCH_TOO_SMALL: return "split plan needs more than the static scratch of mi_sgemm_noalloc holds";
        case MISGEMM_LAUNCH_FAILED: return "HIP kernel launch failed";
        case MISGEMM_WORKSPACE_CAPTURED: return "workspace is used by a captured HIP graph and stays allocated until the process ends";
        default: return "unknown status";
    }
}
