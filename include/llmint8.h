/*
 * llmint8.h -- C ABI of the MI355X (gfx950) LLM.int8() mixed-precision
 * decomposition matmul.
 *
 * The operation (kurtkim.github.io, "LLM.int8()" paper summary, section
 * "The Core of LLM.int8(): Mixed-precision Decomposition", equation for
 * C_f16; agentlenshq.com, "Hugging Face, LLM.int8() 8-bit matrix
 * multiplication integrated into Transformers and Accelerate", section "Core
 * idea", steps 1-3):
 *
 *   out[t,n] = fp16( sum_{k in O} X[t,k] * Wdq[n,k]
 *                    + C[t,n] * a[t] * SCB[n] / 127^2  [+ bias[n]] )
 *   O        = { k : max_t |X[t,k]| > threshold }            (outlier columns)
 *   a[t]     = max_{k not in O} |X[t,k]|                      (row absmax)
 *   Xq[t,k]  = k in O ? 0 : round(127 * X[t,k] / a[t])        (int8)
 *   C[t,n]   = sum_k Xq[t,k] * CB[n,k]                        (exact int32)
 *   Wdq[n,k] = fp16(CB[n,k] * SCB[n] / 127)
 *
 * "round" is to nearest with ties to even, of the exact quotient; the int8
 * values lie in [-127, 127].
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers on the current HIP device,
 *    row-major and contiguous, owned by the caller, 16-byte aligned (the
 *    optional bias: 8-byte aligned; row_zp: 8-byte aligned).  Outputs must
 *    not alias inputs.  fp16 data is passed as raw IEEE binary16 bit
 *    patterns (uint16_t).
 *  - Shapes: T >= 1 (any value; a ragged last tile is handled), K and N
 *    multiples of 64, K <= 133144 (so K * 127^2 fits in int32).
 *  - Every call only enqueues work on `stream` (NULL = the default stream)
 *    and returns; it never allocates, frees or synchronizes.  The library
 *    keeps no mutable state, so concurrent calls on different streams with
 *    separate outputs and workspaces are safe.  The work is kernel launches
 *    only (no memset, copy or event; the workspace needs no clearing), so a
 *    call made during stream capture can be replayed from a HIP graph.
 *  - Status codes: arguments are checked on the host before anything is
 *    enqueued, in this order: null pointers, non-positive sizes or a NaN /
 *    negative threshold -> LLMINT8_ERR_INVALID_ARG; K or N not a multiple of
 *    64 or K > 133144 -> LLMINT8_ERR_UNSUPPORTED_SHAPE; workspace smaller than
 *    the query -> LLMINT8_ERR_WORKSPACE.  A failed launch -> LLMINT8_ERR_HIP.
 *    On an error status nothing has been enqueued (for LLMINT8_ERR_HIP, the
 *    launches before the failing one may have been).  Faults inside kernels
 *    surface at the caller's next synchronization, as for any HIP work.
 *  - Inputs must be finite (not checked).
 */
#ifndef LLMINT8_H
#define LLMINT8_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifndef LLMINT8_API
#define LLMINT8_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LLMINT8_OK = 0,
    LLMINT8_ERR_INVALID_ARG = 1,
    LLMINT8_ERR_UNSUPPORTED_SHAPE = 2,
    LLMINT8_ERR_WORKSPACE = 3,
    LLMINT8_ERR_HIP = 4,
    LLMINT8_ERR_SCRATCH = 5
} llmint8_status_t;

/* Static, NUL-terminated description of a status code (never NULL). */
LLMINT8_API const char *llmint8_status_string(int status);

/* Bytes of workspace llmint8_matmul (and its _act, _zp and _f8 forms) needs
 * for a [T,K] x [K,N] call, the worst case over all outlier counts.  Besides
 * the int8 activations (max(T,16) * K bytes) it holds at most
 * (2*T + N)*min(K,1024) bytes of gathered outlier operands for T > 16
 * (more outlier columns than fit are read in place), and 2*T*K for T <= 16
 * (no weight operand); for T >= 512 and K <= 65536 also
 * N*min(K/4 rounded down to 128, 4096) bytes for the weight codes of the
 * non-outlier columns, which the int8 product runs over alone when at least
 * three quarters of the columns are outliers.  Pure host function; returns 0
 * for invalid sizes. */
LLMINT8_API size_t llmint8_workspace_bytes(int64_t T, int64_t K, int64_t N);

/* Bytes of workspace llmint8_quantize_act needs for K columns. */
LLMINT8_API size_t llmint8_quantize_act_workspace_bytes(int64_t K);

/*
 * Weight quantization (agentlenshq.com write-up, section "Integration into
 * transformers": the weight is quantized once, when it is moved to the GPU,
 * into int8 CB in [-127, 127] plus SCB, with W ~= CB * SCB / 127; vector-wise,
 * one scale per output column -- LLM.int8() summary, section "Vector-wise
 * Quantization").
 *
 *   W_t  in : fp16 [N,K]  -- W transposed (row n = output column n), the
 *                            nn.Linear weight layout
 *   CB   out: int8 [N,K]  -- CB[n,k] = round(127 * W_t[n,k] / SCB[n]), 0 if SCB[n] = 0
 *   SCB  out: f32  [N]    -- SCB[n] = max_k |W_t[n,k]| (an fp16 value)
 *
 * Call it once per weight; quantizing an already dequantized weight again is
 * not an identity in general.
 */
LLMINT8_API llmint8_status_t llmint8_quantize_weight(const uint16_t *W_t, int64_t K, int64_t N,
                                         int8_t *CB, float *SCB, hipStream_t stream);

/*
 * Activation quantization: outlier-column detection and row-wise absmax
 * quantization of the remaining columns (agentlenshq.com write-up, "Core
 * idea" steps 1-2; LLM.int8() summary, sections "8-bit Data Types and
 * Quantization" and "The Core of LLM.int8()").
 *
 *   X            in : fp16 [T,K]
 *   threshold    in : outliers are columns with some |x| > threshold
 *                     (strict; 6.0 is the pages' value; +inf = no outliers,
 *                     0 = every column holding a nonzero)
 *   Xq           out: int8 [T,K], outlier columns stored as 0
 *   row_absmax   out: f32  [T], a[t] over the non-outlier columns (0 if none)
 *   outlier_idx  out: int32 [K] capacity; entries [0, n) are O ascending,
 *                     later entries are unspecified
 *   n_outliers   out: int32 [1] (device), n = |O|
 *   ws, ws_bytes    : scratch of at least
 *                     llmint8_quantize_act_workspace_bytes(K) bytes
 */
LLMINT8_API llmint8_status_t llmint8_quantize_act(const uint16_t *X, int64_t T, int64_t K, float threshold,
                                      int8_t *Xq, float *row_absmax, int32_t *outlier_idx,
                                      int32_t *n_outliers, void *ws, size_t ws_bytes,
                                      hipStream_t stream);

/*
 * The decomposition matmul (LLM.int8() summary, section "The Core of
 * LLM.int8(): Mixed-precision Decomposition"; agentlenshq.com write-up,
 * "Core idea" step 3: dequantize the int8 result and add the fp16 outlier
 * result).  Runs activation quantization, the int8 product with int32
 * accumulation, vector-wise dequantization by a[t] * SCB[n] / 127^2, the
 * fp16 product of the outlier columns with the dequantized weight rows, and
 * the optional bias, with a single rounding to fp16 at the end.
 *
 *   X          in : fp16 [T,K]
 *   CB, SCB    in : from llmint8_quantize_weight, [N,K] int8 and [N] f32
 *                   (SCB 16-byte aligned: the epilogue reads 4 scales at once)
 *   bias       in : fp16 [N] or NULL (8-byte aligned)
 *   threshold  in : as for llmint8_quantize_act
 *   out        out: fp16 [T,N] (overflow rounds to +-inf)
 *   ws, ws_bytes  : scratch of at least llmint8_workspace_bytes(T, K, N)
 *
 * T <= 16 runs a weight-streaming kernel (the decode regime), larger T a
 * tiled MFMA GEMM; both give results that meet the same tolerance.
 * (include/llmint8_test.h has hooks that force either and time it.)
 */
LLMINT8_API llmint8_status_t llmint8_matmul(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                                const int8_t *CB, const float *SCB, const uint16_t *bias,
                                float threshold, uint16_t *out, void *ws, size_t ws_bytes,
                                hipStream_t stream);

/* Bytes of the static device scratch of llmint8_matmul_noalloc (64 MiB):
 * a call fits when llmint8_workspace_bytes(T, K, N), less the optional
 * segment for the non-outlier weight codes (N*min(K/4 rounded down to 128,
 * 4096) bytes for T >= 512, K <= 65536), is at most this, e.g. every
 * T <= 16 call, T = 4096 x K = 4096 x N = 16384 (42 MB, 59 MB with the
 * optional segment), or T = 2048 x K = 16384 x N = 4096 (40 MB). */
#define LLMINT8_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * llmint8_matmul without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same operation, arguments (less ws and
 * ws_bytes), kernels and results as llmint8_matmul.
 *
 * The workspace is a static device array of LLMINT8_NOALLOC_SCRATCH_BYTES
 * that the library holds on every device it runs on until the process ends.
 * Its device address is resolved on the first call on each device (call it
 * once outside stream capture); the call itself allocates nothing.  The
 * kernels need no cleared workspace, so what an earlier call left in it
 * does not matter.  All calls on one device share the array: calls that
 * may overlap on one device (different streams, or host threads without an
 * ordering) race and must be serialized by the caller.
 *
 * When the array holds the workspace but not its optional segment for the
 * non-outlier weight codes, the call runs without it: the int8 product then
 * runs over all of K, with the same result.
 *
 * Errors: as llmint8_matmul (argument and shape checks in the same order),
 * then LLMINT8_ERR_SCRATCH when the workspace less that optional segment
 * exceeds LLMINT8_NOALLOC_SCRATCH_BYTES (nothing enqueued), LLMINT8_ERR_HIP
 * when the array's address cannot be resolved or a launch fails.
 */
LLMINT8_API llmint8_status_t llmint8_matmul_noalloc(const uint16_t *X, int64_t T, int64_t K,
                                                    int64_t N, const int8_t *CB, const float *SCB,
                                                    const uint16_t *bias, float threshold,
                                                    uint16_t *out, hipStream_t stream);

/* Output activations of llmint8_matmul_act. */
enum { LLMINT8_ACT_NONE = 0, LLMINT8_ACT_RELU = 1 };

/*
 * llmint8_matmul followed by the layer's activation, fused into the output
 * rounding: out = fp16(act(v)) for the unrounded output v above (with
 * LLMINT8_ACT_RELU, act(v) = max(v, 0); rounding to nearest commutes with
 * it, so this equals max(fp16(v), 0)).  For the feed-forward layers the
 * method targets (LLM.int8() summary, "Introduction": the feed-forward and
 * attention projection layers), whose expansion is followed by a ReLU (the
 * summary's "8-bit Data Types and Quantization" names ReLU outputs as the
 * activations that feed the next layer), so that the next llmint8_matmul
 * reads the activated values without a separate pass.  Arguments as for
 * llmint8_matmul; an activation other than the two above ->
 * LLMINT8_ERR_INVALID_ARG.
 */
LLMINT8_API llmint8_status_t llmint8_matmul_act(const uint16_t *X, int64_t T, int64_t K,
                                                int64_t N, const int8_t *CB, const float *SCB,
                                                const uint16_t *bias, float threshold,
                                                int activation, uint16_t *out, void *ws,
                                                size_t ws_bytes, hipStream_t stream);

/*
 * Zero-point (asymmetric) variant of the decomposition.  The LLM.int8()
 * summary (kurtkim.github.io, "LLM.int8()", section "8-bit Data Types and
 * Quantization", zeropoint quantization; and "Int8 Matrix Multiplication with
 * 16-bit Float Inputs and Outputs") maps a vector's range onto [-127, 127]
 * with the normalized dynamic range nd = 2*127/(max - min) and an integer
 * zero point zp, multiplies the shifted values (A + zp_a)(B + zp_b) in
 * integers and dequantizes by dividing by nd_a*nd_b.  Here, per vector (a row
 * of X over its non-outlier columns; a row of W_t, i.e. an output column of
 * W, over all K):
 *
 *   min' = min(min, 0), max' = max(max, 0)     (0 joins every range)
 *   d    = max' - min',  nd = 254 / d              (exact; d = 0: nd = 0, zp = 0)
 *   zp   = RNE(nd * min') + 127                     (in [-127, 127])
 *   code = RNE(nd * x) - zp                         (in [-127, 127])
 *
 * RNE rounds the exact rational nd*x = 254x/d to the nearest integer, ties
 * to even (the page fixes no precision, so nothing is rounded before the
 * codes, as in the absmax variant); code + zp = RNE(nd*x) is the page's
 * shifted value and x ~= (code + zp)/nd.  What ND[n] and the activation
 * rows' nd[t] store is the fp32 value nearest to the exact nd; the
 * dequantization below uses those stored values.
 * Outlier columns of X (as for llmint8_matmul) hold the code of 0, -zp, so
 * they add nothing to the integer sum, and
 *
 *   out[t,n] = fp16( sum_k (Xq[t,k] + zp_a[t]) * (CB[n,k] + ZP[n]) / (nd_a[t] * ND[n])
 *                    + sum_{k in O} X[t,k] * fp16(fp32(CB[n,k] + ZP[n]) / ND[n])  [+ bias[n]] )
 *
 * (the integer term is 0 when either nd is 0).  The integer sum is formed
 * unrolled, as the page writes it when no 16-bit multiply exists:
 * C + ZP[n]*(rs_a[t] + K*zp_a[t]) + zp_a[t]*RS[n] with C the int8 product and
 * rs, RS the code sums; |code + zp| <= 254 keeps it exact in int32 for
 * K <= 33286, the limit of these entry points (larger K ->
 * LLMINT8_ERR_UNSUPPORTED_SHAPE).  Other conventions as above.
 */

/*
 * Zero-point weight quantization, once per weight.
 *   W_t in: fp16 [N,K];  CB out: int8 [N,K] codes;  ND out: fp32 [N] nd;
 *   ZP out: int32 [N] zero points;  RS out: int32 [N], RS[n] = sum_k CB[n,k].
 */
LLMINT8_API llmint8_status_t llmint8_quantize_weight_zp(const uint16_t *W_t, int64_t K, int64_t N,
                                                        int8_t *CB, float *ND, int32_t *ZP,
                                                        int32_t *RS, hipStream_t stream);

/*
 * Zero-point activation quantization with outlier detection (as
 * llmint8_quantize_act, same workspace query llmint8_quantize_act_workspace_bytes).
 *   X in: fp16 [T,K];  Xq out: int8 [T,K];  nd out: fp32 [T];
 *   row_zp out: int32 [T][2] (8-byte aligned), row_zp[t] = {zp_a[t], sum_k Xq[t,k]};
 *   outlier_idx / n_outliers out: as llmint8_quantize_act.
 */
LLMINT8_API llmint8_status_t llmint8_quantize_act_zp(const uint16_t *X, int64_t T, int64_t K,
                                                     float threshold, int8_t *Xq, float *nd,
                                                     int32_t *row_zp, int32_t *outlier_idx,
                                                     int32_t *n_outliers, void *ws,
                                                     size_t ws_bytes, hipStream_t stream);

/*
 * The zero-point decomposition: out [T,N] fp16 from X [T,K] fp16 and the
 * output of llmint8_quantize_weight_zp (CB, ND, ZP, RS; ND, ZP and RS
 * 16-byte aligned), with optional bias and the threshold as llmint8_matmul.
 * Workspace: llmint8_workspace_bytes(T, K, N).
 */
LLMINT8_API llmint8_status_t llmint8_matmul_zp(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                                               const int8_t *CB, const float *ND,
                                               const int32_t *ZP, const int32_t *RS,
                                               const uint16_t *bias, float threshold,
                                               uint16_t *out, void *ws, size_t ws_bytes,
                                               hipStream_t stream);

/*
 * FP8 variant of the decomposition.  The LLM.int8() summary
 * (kurtkim.github.io, "LLM.int8()", section "Related work", 8-bit data types)
 * names floating-point 8-bit formats with a 5-bit exponent and a 2-bit
 * fraction as the common kind, and its "Discussion and Limitations" expects
 * the Int8 findings to carry over to FP8.  Here the non-outlier part is held
 * in E5M2 (binary16's layout with a 2-bit fraction; largest finite 57344)
 * with vector-wise power-of-two scales:
 *
 *   e        = largest integer with absmax * 2^e <= 57344   (0 for absmax 0)
 *   code     = E5M2 nearest to x * 2^e, ties to even        (the scaling is exact)
 *   scale    = 2^-e                                          (stored)
 *   out[t,n] = fp16( sum_k e5m2(Xq8[t,k]) * e5m2(CB8[n,k]) * sc[t] * SC8[n]
 *                    + sum_{k in O} X[t,k] * fp16(e5m2(CB8[n,k]) * SC8[n])  [+ bias[n]] )
 *
 * with the row absmax over the non-outlier columns (outlier columns are +0
 * in Xq8) and the weight's over all K.  The E5M2 products are summed in fp32
 * by the matrix cores (v_mfma_f32_32x32x64_f8f6f4; its sums of 64 products
 * are not rounded like sequential fp32 additions), so the output is not
 * unique to the last bit.  Shapes and conventions as llmint8_matmul.
 */

/*
 * FP8 weight quantization, once per weight.
 *   W_t in: fp16 [N,K];  CB8 out: E5M2 codes [N,K] (one byte each);  SC8 out: fp32 [N] scales.
 */
LLMINT8_API llmint8_status_t llmint8_quantize_weight_f8(const uint16_t *W_t, int64_t K, int64_t N,
                                                        uint8_t *CB8, float *SC8,
                                                        hipStream_t stream);

/*
 * FP8 activation quantization with outlier detection (as llmint8_quantize_act,
 * same workspace query).  Xq8 out: E5M2 codes [T,K], outlier columns +0;
 * row_scale out: fp32 [T] scales 2^-e.
 */
LLMINT8_API llmint8_status_t llmint8_quantize_act_f8(const uint16_t *X, int64_t T, int64_t K,
                                                     float threshold, uint8_t *Xq8,
                                                     float *row_scale, int32_t *outlier_idx,
                                                     int32_t *n_outliers, void *ws,
                                                     size_t ws_bytes, hipStream_t stream);

/*
 * The FP8 decomposition: out [T,N] fp16 from X [T,K] fp16 and the output of
 * llmint8_quantize_weight_f8 (SC8 16-byte aligned).  Workspace:
 * llmint8_workspace_bytes(T, K, N).
 */
LLMINT8_API llmint8_status_t llmint8_matmul_f8(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                                               const uint8_t *CB8, const float *SC8,
                                               const uint16_t *bias, float threshold,
                                               uint16_t *out, void *ws, size_t ws_bytes,
                                               hipStream_t stream);

/*
 * The same FP8 variant in E4M3, the other 8-bit float format of the matrix
 * cores (4 exponent bits with bias 7, 3 fraction bits, no infinities; largest
 * finite 448, smallest subnormal 2^-9).  The page names only the 5-bit
 * exponent kind; this form keeps every convention of the E5M2 one above with
 * E4M3 in its place: e is the largest integer with absmax * 2^e <= 448,
 * codes are the E4M3 values nearest to x * 2^e (ties to even), scales 2^-e,
 * outlier columns +0, and the products are summed in fp32 by
 * v_mfma_f32_32x32x64_f8f6f4 (format E4M3 for both operands).  Arguments,
 * alignment, workspace and errors exactly as the _f8 functions; CB8 and Xq8
 * hold E4M3 codes.
 */
LLMINT8_API llmint8_status_t llmint8_quantize_weight_e4m3(const uint16_t *W_t, int64_t K,
                                                          int64_t N, uint8_t *CB8, float *SC8,
                                                          hipStream_t stream);
LLMINT8_API llmint8_status_t llmint8_quantize_act_e4m3(const uint16_t *X, int64_t T, int64_t K,
                                                       float threshold, uint8_t *Xq8,
                                                       float *row_scale, int32_t *outlier_idx,
                                                       int32_t *n_outliers, void *ws,
                                                       size_t ws_bytes, hipStream_t stream);
LLMINT8_API llmint8_status_t llmint8_matmul_e4m3(const uint16_t *X, int64_t T, int64_t K,
                                                 int64_t N, const uint8_t *CB8, const float *SC8,
                                                 const uint16_t *bias, float threshold,
                                                 uint16_t *out, void *ws, size_t ws_bytes,
                                                 hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LLMINT8_H */
