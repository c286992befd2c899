// internal.h -- device helpers and launcher declarations shared by the
// library's translation units (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llmint8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kOutlierPad = 32;   // outlier rows of up to 32 columns are padded to this length

// Row stride, in halves, of the gathered outlier operands x_out [T, ld] and
// w_out [N, ld]; the rows are zero-padded up to it.  Up to 32 outliers: 32
// (the GEMM epilogue's two 16-deep fp16 MFMA steps); more: a multiple of 64
// halves, the 128-byte stages of the fp16 GEMM pass.  Rows stay short and
// dense, and every reader derives ld from n.
__host__ __device__ __forceinline__ int64_t outlier_ld(int n)
{
    return n == 0 ? 0 : n <= kOutlierPad ? kOutlierPad : (int64_t)(n + 63) / 64 * 64;
}

__device__ __forceinline__ float h2f(uint16_t u) { return (float)__builtin_bit_cast(_Float16, u); }
// fp32 -> fp16, round to nearest even (v_cvt_f16_f32 in the default mode); overflow -> inf.
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// The layer's activation applied to the output before its one rounding to
// fp16 (kRelu: max(v, 0); round-to-nearest commutes with it).
template <bool kRelu>
__device__ __forceinline__ uint16_t f2h_act(float v)
{
    return f2h(kRelu ? __builtin_fmaxf(v, 0.0f) : v);
}

// round(127 * x / a) to nearest, ties to even, for fp16 values x and a with
// |x| <= a and a > 0.  127*x is exact in fp32 (7 + 11 bits) and the quotient
// is one IEEE-correct fp32 division (the library is built with
// -fhip-fp32-correctly-rounded-divide-sqrt): such a quotient of binary16
// values never lands on the wrong side of, or onto, a half-integer, so this
// is the exact-rational rounding.
__device__ __forceinline__ int quant127(float x, float a)
{
    return (int)__builtin_rintf((127.0f * x) / a);
}

// fp16 nearest to cb * scb / 127: the product is exact in fp32 and the fp32
// quotient of a rational with odd denominator 127 cannot sit on or across a
// binary16 midpoint, so the two roundings give the singly rounded value.
__device__ __forceinline__ uint16_t dequant_w(int cb, float scb)
{
    return f2h(((float)cb * scb) / 127.0f);
}

// Zero-point variant: the fp16 weight fp16(fp32(cb + zp) / nd) of code cb
// in a column with parameters (nd, zp); 0 when nd = 0 (an all-zero column).
// cb + zp is an integer of at most 9 bits, exact in fp32; one correctly
// rounded division, then the rounding to fp16.
__device__ __forceinline__ uint16_t dequant_w_zp(int cb, int zp, float nd)
{
    return nd > 0.0f ? f2h((float)(cb + zp) / nd) : (uint16_t)0;
}

// FP8 (E5M2) variant.  An E5M2 code is the high byte of the binary16 with
// the same value (same sign, exponent field and bias; 2 of the 10 fraction
// bits), so decoding is a shift.
__device__ __forceinline__ float e5m2_to_f(unsigned c) { return h2f((uint16_t)(c << 8)); }

// The power of two 2^e that scales a vector with absmax a (an fp16 value, as
// fp32) into E5M2's range: e is the largest integer with a * 2^e <= 57344 =
// 1.75 * 2^15 (e = 0 for a = 0).  With a = f * 2^E, f in [1, 2): e = 15 - E
// for f <= 1.75, else 14 - E.
__device__ __forceinline__ int f8_scale_exp(float a)
{
    if (!(a > 0.0f))
        return 0;
    int ex;
    const float fr = __builtin_frexpf(a, &ex);   // a = fr * 2^ex, fr in [0.5, 1)
    return (2.0f * fr <= 1.75f ? 15 : 14) - (ex - 1);
}

// fp16 weight of E5M2 code c in a column with scale sc (a power of two): the
// exact product rounded once.
__device__ __forceinline__ uint16_t dequant_w_f8(unsigned c, float sc)
{
    return f2h(e5m2_to_f(c) * sc);
}

// 1/nd for the zero-point dequantization (0 when nd = 0).  v_rcp_f32 is
// within 1 ulp: the dequantized value, an fp32 product rounded to fp16 at
// the end, moves by a few fp32 ulps at most.
__device__ __forceinline__ float zp_inv(float nd)
{
    return nd > 0.0f ? __builtin_amdgcn_rcpf(nd) : 0.0f;
}

__device__ __forceinline__ unsigned wave_max_u32(unsigned v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        unsigned o = __shfl_xor(v, off, kWave);
        v = o > v ? o : v;
    }
    return v;
}

// Workspace segments of one llmint8_matmul call (byte offsets from the base).
struct MatmulWorkspace {
    size_t partial, mask, chunk_pre, outlier_idx, n_outliers, row_absmax, row_zp, xq, x_out, w_out,
        total;
};
MatmulWorkspace matmul_workspace_layout(int64_t T, int64_t K, int64_t N);
size_t act_workspace_bytes(int64_t K);

// ---- launchers (each enqueues on `s`; return hipGetLastError()) ----
hipError_t launch_quantize_weight(const uint16_t *W_t, int64_t K, int64_t N, int8_t *CB,
                                  float *SCB, hipStream_t s);

// What the row-quantization launch needs to also produce the dequantized
// outlier weight rows for the GEMM: w_out[n, j] = fp16(CB[n,O[j]]*SCB[n]/127),
// zero for n_outliers <= j < outlier_ld(n_outliers), which is also the row
// stride.  w_out == null skips it.
struct GatherArgs {
    const int8_t *CB;
    const float *SCB;   // zero-point variant: nd of each column; FP8: scale 2^-e
    int64_t N;
    uint16_t *w_out;
    const int32_t *zp = nullptr;   // zero-point variant: zp of each column (else null)
    bool f8 = false;               // FP8 variant: CB holds E5M2 codes
};

// Row ranges of the outlier detection: the partial-flag buffer holds
// kDetectSplits bytes per 8-column chunk (kDetectSplits * K/8 bytes).
constexpr int kDetectSplits = 16;
// The row quantization takes a wavefront per row from kRowQuantWaveMinT rows
// on when the rows are at most kRowQuantWaveMaxK long (measured on MI355X:
// 15 vs 20 us at 2048 x 2048, equal at 4096 x 4096); otherwise a block of
// 256 threads per row, which keeps more loads in flight per row for long
// rows (49 vs 53 us at 4096 x 12288).
constexpr int64_t kRowQuantWaveMinT = 256;
constexpr int64_t kRowQuantWaveMaxK = 4096;

// Outlier detection + compaction + row quantization (+ the optional outlier
// weight gather).  x_out (fp16 [T, outlier_ld(n)]) receives the gathered
// outlier columns, zero-padded, when non-null.  xq_packed (T <= 16 only) writes Xq in the decode kernel's
// fragment order [K/64][4][16][16] (16*K bytes; rows >= T are left as they
// are) instead of row-major [T, K].
hipError_t launch_quantize_act(const uint16_t *X, int64_t T, int64_t K, float threshold,
                               int8_t *Xq, float *a, int32_t *O, int32_t *n_out,
                               uint8_t *partial, uint8_t *mask, int32_t *chunk_pre,
                               uint16_t *x_out, const GatherArgs &g, bool xq_packed,
                               hipStream_t s);

// The same quantization for few rows in one launch of T blocks and without
// workspace (each block derives the outlier set from all rows itself): one
// row with K <= kQuantRowsMaxK1, or up to kQuantRowsMaxT rows with
// K <= kQuantRowsMaxK.  Results are identical to launch_quantize_act's.
constexpr int64_t kQuantRowsMaxT = 16;
constexpr int64_t kQuantRowsMaxK = 16384;
constexpr int64_t kQuantRowsMaxK1 = 65536;
bool quantize_act_fits_rows(int64_t T, int64_t K);
hipError_t launch_quantize_act_rows(const uint16_t *X, int64_t T, int64_t K, float threshold,
                                    int8_t *Xq, float *a, int32_t *O, int32_t *n_out,
                                    uint16_t *x_out, bool xq_packed, hipStream_t s);

struct EpilogueArgs {
    const float *a;          // [T] row absmax (zero-point variant: nd of each row)
    const float *scb;        // [N] (zero-point variant: nd of each column)
    const uint16_t *x_out;   // [T, outlier_ld(n)] gathered outlier activations (fp16)
    const uint16_t *w_out;   // [N, outlier_ld(n)] dequantized outlier weights (fp16), GEMM path
    const int32_t *O;        // [n] outlier column indices (weight-streaming path)
    const int32_t *n_out;    // device scalar n
    const uint16_t *bias;    // [N] or null
    uint16_t *out;           // [T, N] fp16
    int32_t *c_i32;          // [T, N] raw accumulators (debug epilogue) or null
    int act;                 // output activation: 0 none, 1 ReLU
    // Zero-point variant (all null otherwise): per row {zp, sum of the row's
    // codes}, per column zp and sum of the column's codes.  The integer part
    // is then sum_k (A + zp_a)(B + zp_b) = C + zp_b*(rs_a + K*zp_a) + zp_a*rs_b.
    const int2 *row_zp = nullptr;
    const int32_t *zp_b = nullptr;
    const int32_t *rs_b = nullptr;
    // FP8 variant: Xq and CB hold E5M2 codes, a and scb the scales 2^-e of
    // the rows and columns; the products are summed in fp32 by fp8 MFMAs.
    bool f8 = false;
};

// Zero-point variant (the asymmetric quantizer of the LLM.int8() summary,
// "8-bit Data Types and Quantization"): per vector, range [min(min,0),
// max(max,0)], d = fp32(max' - min'), nd = fp32(254/d), zp = RNE(nd*min') +
// 127, code = min(RNE(nd*x) - zp, 127) (roundings of the exact product);
// d = 0 gives nd = 0, zp = 0, codes 0.  Weight: per row of W_t over all K,
// with RS[n] the sum of the row's codes.  K <= kMaxKZp keeps the shifted
// product sum_k (A+zp_a)(B+zp_b), |A+zp| <= 254, inside int32.
constexpr int64_t kMaxKZp = 33286;
hipError_t launch_quantize_weight_zp(const uint16_t *W_t, int64_t K, int64_t N, int8_t *CB,
                                     float *ND, int32_t *ZP, int32_t *RS, hipStream_t s);
// Activations: as launch_quantize_act, but the non-outlier part of each row
// zero-point quantized (nd[t]; row_zp[t] = {zp, sum of the row's K codes});
// outlier columns hold the code of 0, -zp.  g.zp must be set when g.w_out
// is (the outlier weight rows are then dequantized as fp16((cb+zp)/nd)).
// Without w_out and for the shapes of quantize_act_fits_rows it is one
// launch (the few-rows kernel), else detection, compaction and a block per
// row.
hipError_t launch_quantize_act_zp(const uint16_t *X, int64_t T, int64_t K, float threshold,
                                  int8_t *Xq, float *nd, int2 *row_zp, int32_t *O,
                                  int32_t *n_out, uint8_t *partial, uint8_t *mask,
                                  int32_t *chunk_pre, uint16_t *x_out, const GatherArgs &g,
                                  bool xq_packed, hipStream_t s);

// FP8 variant (E5M2, the 5-bit-exponent, 2-bit-fraction format the
// LLM.int8() summary names under "Related work"): per vector a power-of-two
// scale 2^e (f8_scale_exp of the absmax; the row absmax over the
// non-outlier columns), codes = E5M2 nearest to x * 2^e (ties to even),
// stored scale 2^-e; outlier columns are +0.  Weight: per row of W_t.
hipError_t launch_quantize_weight_f8(const uint16_t *W_t, int64_t K, int64_t N, uint8_t *CB8,
                                     float *SC8, hipStream_t s);
// Activations: as launch_quantize_act (same kernels with the E5M2 codes;
// sc receives the row scales 2^-e); g.f8 must be set when g.w_out is.
hipError_t launch_quantize_act_f8(const uint16_t *X, int64_t T, int64_t K, float threshold,
                                  uint8_t *Xq8, float *sc, int32_t *O, int32_t *n_out,
                                  uint8_t *partial, uint8_t *mask, int32_t *chunk_pre,
                                  uint16_t *x_out, const GatherArgs &g, bool xq_packed,
                                  hipStream_t s);

// ev0/ev1 (optional) are recorded on s right before and after the main kernel.
hipError_t launch_gemm(const int8_t *Xq, const int8_t *CB, int64_t T, int64_t K, int64_t N,
                       const EpilogueArgs &ep, hipStream_t s, hipEvent_t ev0 = nullptr,
                       hipEvent_t ev1 = nullptr);
// Activation rows from which the decode path takes Xq in fragment order
// (one contiguous KB per k-step, shared by a block's wavefronts through L1);
// a single row stays row-major (one 64-byte piece per k-step).
constexpr int64_t kDecodePackedMinT = 2;
// xq_packed: Xq is in the fragment order written by launch_quantize_act.
hipError_t launch_decode(const int8_t *Xq, const int8_t *CB, int64_t T, int64_t K, int64_t N,
                         const EpilogueArgs &ep, bool xq_packed, hipStream_t s,
                         hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

}  // namespace llmint8
