// mi_clock_probe: the shader clock the GPU sustains under full FP32 matrix
// load, and the matrix-core rate that clock allows.
//
// Durations mean little without the clock they ran at; the klklkl10086
// SGEMM page ("【CUDA】Sgemm单精度矩阵乘法", 00-朴素实现, the Speed Of Light
// table) prints the SM frequency beside every kernel time for that reason.
// One workgroup per CU (its LDS reservation admits no second one), eight
// waves -- two per SIMD, as the tile kernels run -- each issuing a
// register-only chain of v_mfma_f32_32x32x2_f32 on four independent
// accumulators. Wave 0 of each workgroup stamps the shader-clock counter and
// the constant-rate wall clock before and after the loop; the ratio of the
// two spans is the shader clock, and the FLOPs over the longest wall span the
// matrix rate reached.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "misgemm.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kProbeWaves = 8;
constexpr int kProbeWorkgroups = 256;        // one per CU
constexpr int kProbeLdsFloats = 24 * 1024;   // 96 KiB: one workgroup per CU

__global__ __launch_bounds__(64 * kProbeWaves) void clock_probe(int iters, unsigned long long *out) {
    __shared__ float hold[kProbeLdsFloats];
    const int tid = threadIdx.x;
    // Operand values do not matter; they only have to be opaque.
    const float a = 1.0f + (float)tid * 1e-7f, b = 1.0f - (float)tid * 1e-7f;
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
    hold[tid] = a;
    __syncthreads();
    unsigned long long c0 = 0, w0 = 0;
    if (tid == 0) {
        c0 = clock64();
        w0 = wall_clock64();
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[j], 0, 0, 0);
    }
    float s = hold[(tid + 1) % (64 * kProbeWaves)];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    __syncthreads();
    if (tid == 0) {
        const unsigned long long c1 = clock64(), w1 = wall_clock64();
        unsigned long long *o = out + 4 * blockIdx.x;
        o[0] = c0;
        o[1] = c1;
        o[2] = w0;
        o[3] = w1;
    }
    // Keeps every MFMA's result live; the sum is never this value in practice.
    if (s == -1.0f) out[0] = 0;
}

}  // namespace

extern "C" int mi_clock_probe(int iters, unsigned long long *stamps, int *wall_clock_khz, hipStream_t stream) {
    if (iters < 0) return MISGEMM_BAD_M;
    if (stamps == nullptr) return MISGEMM_NULL_C;
    if (wall_clock_khz != nullptr) {
        int dev = 0;
        if (stream == nullptr) {
            if (hipGetDevice(&dev) != hipSuccess) return MISGEMM_LAUNCH_FAILED;
        } else {
            hipDevice_t d = 0;
            if (hipStreamGetDevice(stream, &d) != hipSuccess) return MISGEMM_LAUNCH_FAILED;
            dev = d;
        }
        if (hipDeviceGetAttribute(wall_clock_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
            return MISGEMM_LAUNCH_FAILED;
    }
    hipLaunchKernelGGL(clock_probe, dim3(kProbeWorkgroups), dim3(64 * kProbeWaves), 0, stream, iters, stamps);
    return hipGetLastError() == hipSuccess ? MISGEMM_SUCCESS : MISGEMM_LAUNCH_FAILED;
}
