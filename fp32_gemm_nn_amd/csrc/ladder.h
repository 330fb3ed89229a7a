// Internal interface between the C-ABI dispatcher (misgemm.hip) and the
// vector-ALU technique ladder (ladder.hip). Not part of the public ABI.
#ifndef MISGEMM_LADDER_H
#define MISGEMM_LADDER_H

#include <hip/hip_runtime.h>

namespace misgemm_ladder {

// One SGEMM call, already validated by the dispatcher: M, N, K > 0,
// alpha != 0, leading dimensions legal for the stored shapes.
struct LadderArgs {
    const float *A;
    const float *B;
    float *C;
    int M, N, K;
    int lda, ldb, ldc;
    float alpha, beta;
    int vec_ab;   // A and B: 16-byte aligned base, lda and ldb multiples of 4
    int vec_c;    // C: 16-byte aligned base, ldc multiple of 4
};

// The rungs, in the order the itan.pw RTX 4090 SGEMM page climbs them.
enum Rung : int {
    kNaive = 0,     // one thread per element of C, lanes along n (section 3.1)
    kLds32 = 1,     // 32 x 32 LDS tiles, one element per thread (section 3.2)
    kBlock1d = 2,   // 64 x 64 x 8 tile, 8 elements of a column per thread (section 3.3)
    kBlock2d = 3,   // 128 x 128 x 8 tile, 8 x 8 elements per thread (section 3.4)
    kVec2d = 4,     // + 16-byte loads, transposed A tile, double-buffered LDS,
                    //   conflict-free vector LDS reads (sections 3.5, 3.7, 3.8)
    kNumRungs = 5,
};

// Enqueue one rung on `stream`; returns the launch's error state.
hipError_t launch(int rung, bool ta, bool tb, const LadderArgs &a, hipStream_t stream);

}  // namespace misgemm_ladder

#endif  // MISGEMM_LADDER_H
