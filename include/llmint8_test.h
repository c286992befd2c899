/*
 * llmint8_test.h -- test and benchmark hooks of libllmint8.so.
 *
 * Not part of the method's interface (include/llmint8.h): these entry points
 * force the kernel choice of a matmul, bracket its main kernel with timing
 * events, size the workspace of a forced choice, and expose the int8 product
 * on its own, so that tests can check each kernel against the CPU oracle and
 * the benchmark can time the main kernel on its stream.  Conventions (device
 * pointers, alignment, status codes, stream semantics) are those of
 * llmint8.h.
 */
#ifndef LLMINT8_TEST_H
#define LLMINT8_TEST_H

#include "llmint8.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel choice of the *_path entry points: 0 = automatic (as the plain entry
 * point), 1 = tiled GEMM, 2 = weight-streaming kernel (T <= 16). */
enum { LLMINT8_PATH_AUTO = 0, LLMINT8_PATH_GEMM = 1, LLMINT8_PATH_DECODE = 2 };

/* Workspace bytes of a call with the kernel choice `path` (llmint8_workspace_bytes
 * is path 0); 0 for invalid sizes or path. */
LLMINT8_API size_t llmint8_workspace_bytes_path(int64_t T, int64_t K, int64_t N, int path);

/*
 * llmint8_matmul (the decomposition of llmint8.h) with the kernel choice
 * forced and optional timing events: path as above (path 2 requires
 * T <= 16, else LLMINT8_ERR_UNSUPPORTED_SHAPE); the workspace must hold
 * llmint8_workspace_bytes_path(T, K, N, path) bytes.  When main_start / main_stop are non-NULL
 * they are recorded on `stream` immediately before and after the launch of
 * the main kernel (the GEMM or weight-streaming kernel), so their elapsed
 * time is that kernel's duration.  The events are created and owned by the
 * caller.  An event record is the one piece of work that is not a kernel
 * launch, so a timed call is not meant for graph capture.
 */
LLMINT8_API llmint8_status_t llmint8_matmul_path(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                                     const int8_t *CB, const float *SCB, const uint16_t *bias,
                                     float threshold, uint16_t *out, void *ws, size_t ws_bytes,
                                     int path, hipEvent_t main_start, hipEvent_t main_stop,
                                     hipStream_t stream);

/* llmint8_matmul_zp with the path choice and timing events of llmint8_matmul_path. */
LLMINT8_API llmint8_status_t llmint8_matmul_zp_path(const uint16_t *X, int64_t T, int64_t K,
                                                    int64_t N, const int8_t *CB, const float *ND,
                                                    const int32_t *ZP, const int32_t *RS,
                                                    const uint16_t *bias, float threshold,
                                                    uint16_t *out, void *ws, size_t ws_bytes,
                                                    int path, hipEvent_t main_start,
                                                    hipEvent_t main_stop, hipStream_t stream);

/* llmint8_matmul_f8 with the path choice and timing events of llmint8_matmul_path. */
LLMINT8_API llmint8_status_t llmint8_matmul_f8_path(const uint16_t *X, int64_t T, int64_t K,
                                                    int64_t N, const uint8_t *CB8,
                                                    const float *SC8, const uint16_t *bias,
                                                    float threshold, uint16_t *out, void *ws,
                                                    size_t ws_bytes, int path,
                                                    hipEvent_t main_start, hipEvent_t main_stop,
                                                    hipStream_t stream);

/* llmint8_matmul_e4m3 with the path choice and timing events of llmint8_matmul_path. */
LLMINT8_API llmint8_status_t llmint8_matmul_e4m3_path(const uint16_t *X, int64_t T, int64_t K,
                                                      int64_t N, const uint8_t *CB8,
                                                      const float *SC8, const uint16_t *bias,
                                                      float threshold, uint16_t *out, void *ws,
                                                      size_t ws_bytes, int path,
                                                      hipEvent_t main_start, hipEvent_t main_stop,
                                                      hipStream_t stream);

/*
 * The int8 product alone, C[t,n] = sum_k Xq[t,k] * CB[n,k] in int32 (LLM.int8()
 * summary, section "Int8 Matrix Multiplication with 16-bit Float Inputs and
 * Outputs"), through the same main loops as llmint8_matmul with the epilogue
 * storing the raw accumulators.  For exact checks of the accumulators.
 *
 *   Xq in: int8 [T,K];  CB in: int8 [N,K];  C out: int32 [T,N]
 *   path: 0 = automatic, 1 = tiled GEMM, 2 = weight-streaming (T <= 16)
 */
LLMINT8_API llmint8_status_t llmint8_igemm_i32(const int8_t *Xq, int64_t T, int64_t K, int64_t N,
                                   const int8_t *CB, int32_t *C, int path, hipStream_t stream);

/*
 * The MFMA ceiling on given operands: `blocks` workgroups of 4 wavefronts,
 * each wavefront loading 4 + 4 16-byte fragments of two 32-byte k-steps from
 * A and B (rows of a 128 x 128 tile at a position that differs per
 * wavefront) and issuing iters * 32 MFMAs on them from registers, nothing
 * else: v_mfma_i32_32x32x32_i8 (kind 0; A, B int8 [T,K], [N,K]; 65536 ops
 * each) or v_mfma_f32_32x32x16_f16 (kind 1; A, B fp16 [T,K], [N,K]; 32768
 * flops each).  The dense MFMA peaks hold at the top clock; under a
 * sustained MFMA load the clock is power-managed, and this measures the rate
 * that is left on the workload's own operand bits.  out: int32
 * [blocks * 256], a value per lane (the products' checksum, so none is
 * dropped).  start / stop as for llmint8_matmul_path, around the one launch.
 * Requires T, N >= 128 and row bytes (K, or 2K for kind 1) a multiple of 64.
 */
LLMINT8_API llmint8_status_t llmint8_mfma_ceiling(const void *A, int64_t T, const void *B,
                                                  int64_t N, int64_t K, int kind, int blocks,
                                                  int iters, int32_t *out, hipEvent_t start,
                                                  hipEvent_t stop, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LLMINT8_TEST_H */
