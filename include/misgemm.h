/*
 * misgemm -- FP32 SGEMM for AMD Instinct MI355X (gfx950), C ABI.
 *
 * The operation is the BLAS SGEMM C = alpha*op(A)*op(B) + beta*C named in the
 * overview of the itan.pw page on SGEMM optimisation for the RTX 4090, on
 * row-major matrices as in the problem definition (问题定义) of
 * "【CUDA】Sgemm单精度矩阵乘法" (klklkl10086.github.io), where
 * C_ij = sum_k A_ik B_kj and a product costs 2MNK floating-point operations.
 *
 * mi_sgemm computes every product in FP32 on the CDNA4 matrix cores
 * (v_mfma_f32_32x32x2_f32 / v_mfma_f32_16x16x4_f32): FP32 inputs, FP32
 * products and FP32 accumulation, with no reduced-precision emulation.
 * The configurations named valu_* (reachable only through
 * mi_sgemm_with_config) are the itan.pw page's technique ladder (its
 * section 3: naive, LDS tiles, 1-D and 2-D register tiles, 16-byte loads
 * with double-buffered LDS) on the vector ALUs, with FP32 fused
 * multiply-adds in ascending k.
 *
 * Threading: every entry point is thread-safe. The only mutable host state is
 * the set of split-K workspaces (one per device and stream, see mi_sgemm)
 * and the per-device address of mi_sgemm_noalloc's scratch, which locks
 * guard. Concurrent calls of mi_sgemm_noalloc on one GPU share that GPU's
 * scratch and must not overlap (see mi_sgemm_noalloc).
 */
#ifndef MISGEMM_H
#define MISGEMM_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. Every entry point returns one, so that no failure passes
 * silently: the youngju.dev CUDA architecture primer (section
 * よくある落とし穴とチェックリスト, item 6, エラーチェックの省略) warns that
 * unchecked runtime return codes and launch errors yield wrong results
 * without a sign, and advises checking each call and the last launch error.
 * Negative values name the offending argument by its position in mi_sgemm's
 * parameter list (BLAS "info" convention) and are returned before any HIP
 * call; positive values report the HIP runtime. */
#define MISGEMM_SUCCESS          0
#define MISGEMM_BAD_TRANSA      (-1)
#define MISGEMM_BAD_TRANSB      (-2)
#define MISGEMM_BAD_M           (-3)
#define MISGEMM_BAD_N           (-4)
#define MISGEMM_BAD_K           (-5)
#define MISGEMM_NULL_A          (-7)
#define MISGEMM_BAD_LDA         (-8)
#define MISGEMM_NULL_B          (-9)
#define MISGEMM_BAD_LDB         (-10)
#define MISGEMM_NULL_C          (-12)
#define MISGEMM_BAD_LDC         (-13)
#define MISGEMM_BAD_CONFIG      (-20)
#define MISGEMM_TOO_LARGE       (-21)
#define MISGEMM_SCRATCH_TOO_SMALL (-22)
#define MISGEMM_LAUNCH_FAILED     1
#define MISGEMM_WORKSPACE_CAPTURED 2

/*
 * mi_sgemm: C <- alpha * op(A) * op(B) + beta * C   (FP32, row-major)
 *
 *   transA, transB  'N'/'n': op(X) = X;  'T'/'t'/'C'/'c': op(X) = X^T.
 *   M, N, K         op(A) is M x K, op(B) is K x N, C is M x N; each >= 0.
 *   A, lda          device pointer; stored A is M x K (transA 'N') or K x M
 *                   (transA 'T'), row-major with row stride lda elements,
 *                   lda >= max(1, number of stored columns).
 *   B, ldb          likewise: stored B is K x N ('N') or N x K ('T').
 *   C, ldc          device pointer; M x N row-major, ldc >= max(1, N).
 *   alpha, beta     scalars. beta == 0: C is not read (NaN/Inf in C do not
 *                   propagate). alpha == 0 or K == 0: A and B are not read and
 *                   C <- beta*C. M == 0 or N == 0: nothing is done.
 *   stream          HIP stream the work is enqueued on (0: the null stream).
 *
 * Semantics: C(i,j) = alpha * sum_{k<K} opA(i,k)*opB(k,j) + beta*C(i,j) for
 * i < M, j < N, with opA(i,k) = A[i*lda+k] ('N') or A[k*lda+i] ('T') and
 * opB(k,j) = B[k*ldb+j] ('N') or B[j*ldb+k] ('T'). Only those elements of C
 * are written; row padding (columns N..ldc-1) is never touched. The k sum is
 * carried in FP32 in a fixed order, so repeated calls give identical bits.
 *
 * Ownership: all three matrices are device memory owned by the caller. The
 * call does not synchronise and returns once the kernels are enqueued; the
 * caller synchronises `stream` before reading C. C must not overlap A or B.
 * The first call on a stream whose kernel splits the k range over
 * workgroups (split-K or stream-K) allocates that stream's workspace, on the
 * stream's device (the current device for the null stream): 64 MiB
 * of partial blocks and 256 KiB of counters, kept until
 * mi_sgemm_release_workspace or the end of the process. Calls on one stream
 * use its workspace in stream order; calls on different streams never share
 * one. If it cannot be allocated the kernel runs unsplit. No other call
 * allocates or frees memory.
 *
 * Graph capture: a call may be captured into a HIP graph and replayed. It
 * enqueues kernels only (no memset); split-K and stream-K kernels reset
 * their own counters. Make one eager call that splits on the capture stream
 * first, so that its workspace exists before capture (otherwise the captured
 * call runs unsplit). Replays use that stream's workspace: they must not
 * overlap one another or other calls on that stream, and the workspace is
 * then kept until the process ends (see mi_sgemm_release_workspace).
 * mi_sgemm_noalloc captures without any prior call.
 *
 * Alignment: any pointer and leading dimension is accepted. 16-byte aligned
 * pointers with lda, ldb, ldc multiples of 4 take the dwordx4 path.
 *
 * Errors: arguments are checked before any HIP call, in parameter order;
 * the first bad one returns its negative code and nothing is enqueued.
 * Sizes whose element offsets exceed 2^31-1 return MISGEMM_TOO_LARGE.
 * MISGEMM_LAUNCH_FAILED means hipGetLastError reported an error after a
 * launch (the error is left for the caller to inspect with hipGetLastError
 * cleared, i.e. it has been consumed by this check).
 */
int mi_sgemm(char transA, char transB, int M, int N, int K,
             float alpha, const float *A, int lda,
             const float *B, int ldb,
             float beta, float *C, int ldc, hipStream_t stream);

/*
 * mi_sgemm_with_config: as mi_sgemm, but with the kernel configuration chosen
 * by the caller instead of by shape class (config ids 0 .. count-1 from
 * mi_sgemm_config_count). Meant for tests, tuning and baselines: any config
 * computes the same result, to FP32 rounding, for any valid shape (the same
 * bits on integer-valued inputs). Returns MISGEMM_BAD_CONFIG for an unknown
 * id, after the argument checks of mi_sgemm.
 */
int mi_sgemm_with_config(int config, char transA, char transB, int M, int N, int K,
                         float alpha, const float *A, int lda,
                         const float *B, int ldb,
                         float beta, float *C, int ldc, hipStream_t stream);

/*
 * mi_sgemm_select_config: the config id mi_sgemm would use for this shape
 * when A and B allow 16-byte loads (16-byte aligned pointers, lda and ldb
 * multiples of 4); for other operands mi_sgemm replaces the tiles that have
 * no 4-byte straight-line form (the 256 x 256, 192 x 192 and 128 x 256 x 16
 * tiles, the two-workgroup stream-K tiles, and the 16 x 16 128 x 128 w4x2 tile
 * except for NT) by a 256 x 128, 128 x 256 or 16 x 16 stream-K tile. Host-side decision
 * only; no HIP call.
 * Returns a negative status for invalid trans letters or negative sizes.
 */
int mi_sgemm_select_config(char transA, char transB, int M, int N, int K);

/* Number of kernel configurations, and a static name for each (NULL if the id
 * is out of range). The string is owned by the library. */
int mi_sgemm_config_count(void);
const char *mi_sgemm_config_name(int config);

/* Static description of a status code (never NULL; owned by the library),
 * so that a caller can report each checked return code in words (the
 * youngju.dev CUDA architecture primer, section よくある落とし穴とチェックリスト,
 * item 6, エラーチェックの省略). */
const char *mi_sgemm_status_string(int status);

/*
 * mi_sgemm_release_workspace: free the split-K workspace kept for `stream`
 * (on the stream's device; for the null stream, the current device), if any, after waiting for the work already enqueued on
 * that stream (hipStreamSynchronize). Meant for callers that destroy streams
 * which ran split products: call it before hipStreamDestroy to return the
 * memory. A later split call on the stream allocates a fresh workspace.
 * Returns MISGEMM_SUCCESS (also when there was none), or
 * MISGEMM_LAUNCH_FAILED if waiting for the stream or freeing failed. A
 * workspace that a call captured into a HIP graph uses is never freed (the
 * graph's kernels hold its address): release then returns
 * MISGEMM_WORKSPACE_CAPTURED and the workspace stays until the process ends.
 * It must not run while another thread enqueues an mi_sgemm call on the same
 * stream.
 */
int mi_sgemm_release_workspace(hipStream_t stream);

/*
 * mi_sgemm_noalloc: mi_sgemm for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops that forbid allocation). Same
 * arguments, kernels, results and errors as mi_sgemm, but it never calls
 * hipMalloc or hipFree: the split-K, stream-K and skinny-band kernels keep
 * their partial blocks and tile counters in a static device array of the
 * library (scratch) instead of a per-stream workspace.
 *
 * Scratch: 64 MiB of partial blocks and 65,536 tile counters (256 KiB), the
 * same capacity as a stream's workspace, so the same split plan and the same
 * bits as mi_sgemm. Each GPU the library runs this entry point on holds its
 * own copy until the process ends (the device memory is reserved when the
 * library's code object is loaded on that GPU). The split plans are bounded
 * by this capacity; a plan that would exceed it is refused with
 * MISGEMM_SCRATCH_TOO_SMALL and nothing is enqueued.
 *
 * The first call on a device looks up that device's copy of the array
 * (hipGetSymbolAddress) and, unless the stream is being captured, clears its
 * counters with a kernel on `stream`; the loader hands the array over
 * zero-filled, and every split product leaves its counters at zero.
 *
 * Concurrency: every call on one GPU shares that GPU's scratch. Calls that
 * may overlap on one GPU -- on different streams, from different threads, or
 * replays of graphs that captured this call -- race on the partial blocks
 * and counters and give wrong results; order them (one stream, or events).
 * The scratch keeps the last call's contents; nothing is read before this
 * call has written it.
 */
int mi_sgemm_noalloc(char transA, char transB, int M, int N, int K,
                     float alpha, const float *A, int lda,
                     const float *B, int ldb,
                     float beta, float *C, int ldc, hipStream_t stream);

/*
 * mi_clock_probe: measurement aid, not part of the product path. Reads the
 * shader clock the GPU sustains under full FP32 matrix load, so that a
 * kernel time can be stated beside the clock it ran at (the klklkl10086
 * SGEMM page, "【CUDA】Sgemm单精度矩阵乘法", 00-朴素实现, prints the SM
 * frequency in its Speed Of Light table beside each duration).
 *
 * Enqueues one kernel on `stream`: 256 workgroups (one per CU) of eight
 * waves, each wave issuing `iters` rounds of four independent
 * v_mfma_f32_32x32x2_f32 (4096 FLOP each) on registers only. Wave 0 of
 * workgroup w writes four values to stamps[4w .. 4w+3]: the shader-clock
 * counter before and after the loop, then the constant-rate wall clock
 * before and after. `stamps` is a device buffer of at least 1024 unsigned
 * 64-bit integers owned by the caller. If `wall_clock_khz` is not NULL it
 * receives the wall clock's rate (kHz) for the stream's device (the current
 * device for the null stream). Shader clock = (c1 - c0) / (w1 - w0) * rate;
 * the matrix rate reached is 256 * 8 * iters * 4 * 4096 FLOP over the
 * longest wall span. Returns MISGEMM_BAD_M for iters < 0, MISGEMM_NULL_C for
 * a null `stamps`, MISGEMM_LAUNCH_FAILED if a HIP call fails.
 */
int mi_clock_probe(int iters, unsigned long long *stamps, int *wall_clock_khz, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MISGEMM_H */
