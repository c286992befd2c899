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

// How the GEMM path forms the fp16 product over the outlier columns O, chosen
// on the device from n = |O| and the number of 64-column groups of K that hold
// an outlier (ng), identically by every kernel that needs it:
//   kOutFew      n <= 32: compact fp16 operands x_out [T,32] and w_out [N,32]
//                (dequantized weights), two fp16 MFMAs per tile in k_gemm;
//   kOutCompact  more, at most kCompactMaxLd after padding, and scattered:
//                compact operands x_out [T,ld] (fp16) and the weight codes of
//                the outlier columns [N,ld] (int8), dequantized by k_gemm_many
//                as it stages them;
//   kOutDense    otherwise (e.g. every column an outlier): k_gemm_many walks
//                the non-empty 64-column groups of X and CB themselves, with
//                the weight codes of non-outlier columns masked to zero, so no
//                operand is gathered.
// The workspace therefore holds gathered operands of at most kCompactMaxLd
// columns: it grows with T and N, not with T*K or N*K.
enum { kOutFew = 0, kOutCompact = 1, kOutDense = 2 };
constexpr int64_t kCompactMaxLd = 1024;
// The outlier-set summary in the workspace: int32 info[kInfoWords] =
// {n, ng, mode, kc} (kc: see kept_ld).
constexpr int kInfoWords = 4;

// Kept-column mode of the GEMM path's 8-bit part (absmax and FP8 variants;
// the zero-point variant's unrolled sum runs over all K): when most
// columns are outliers, the int8 product runs over the kept (non-outlier)
// columns alone, compacted in column order.  The row quantization writes
// each row's kept codes to the start of its Xq row (row stride K),
// zero-padded to kc = the kept count rounded up to 128 bytes, and its row
// blocks write the kept codes of every weight row to cb_kept [N, kc] (both
// through one list of the kept columns per block); every product of an
// outlier column is 0 in the int8 sum, so the sum is unchanged.
// Chosen on the device when kc <= kept_cap(K) (a quarter of K, at most
// kKeptMaxLd: the int8 work falls at least fourfold, and the workspace
// segment stays at most N * min(K/4, 4096) bytes), for launches of at least
// kKeptMinT rows (with fewer rows the int8 work saved does not repay reading
// CB once more) and K <= kKeptMaxK (the list's 16-bit column indices).
constexpr int64_t kKeptMaxLd = 4096;
constexpr int64_t kKeptMinT = 512;
constexpr int64_t kKeptMaxK = 65536;
__host__ __device__ __forceinline__ int64_t kept_cap(int64_t K)
{
    const int64_t h = K / 4 / 128 * 128;
    return h < kKeptMaxLd ? h : kKeptMaxLd;
}
// kc for n outlier columns out of K; 0: the int8 part runs over all of K
// (few outliers), or not at all (n = K).
__host__ __device__ __forceinline__ int64_t kept_ld(int64_t K, int n)
{
    if (n <= kOutlierPad || n >= K)
        return 0;
    const int64_t kc = (K - n + 127) / 128 * 128;
    return kc <= kept_cap(K) ? kc : 0;
}

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

// The same value through r = fp32(scb / 127), computed once per column:
// fp32(cb * r) is within 2^-23 (two roundings) of cb * scb / 127 relative to
// it, while that value -- cb * m * 2^e / 127 for the binary16 scb = m * 2^e,
// never a binary16 midpoint since 127 is prime -- lies at least about 2^-18
// relative from every binary16 midpoint; so both round to the same fp16.
// (Exhaustive check over every code and binary16 scale on the CPU.)
__device__ __forceinline__ uint16_t dequant_w_r(int cb, float r)
{
    return f2h((float)cb * r);
}

// Zero-point variant: the fp16 weight fp16(fp32(cb + zp) / nd) of code cb
// in a column with parameters (nd, zp); 0 when nd = 0 (an all-zero column).
// cb + zp is an integer of at most 9 bits, exact in fp32; one correctly
// rounded division, then the rounding to fp16.
__device__ __forceinline__ uint16_t dequant_w_zp(int cb, int zp, float nd)
{
    return nd > 0.0f ? f2h((float)(cb + zp) / nd) : (uint16_t)0;
}

// The same value through rinv = fp32(1 / nd), computed once per column.
// q = fp32((cb + zp) * rinv) is within 3 fp32 ulps of fp32((cb + zp) / nd)
// (three roundings of at most 2^-24 each, relative); both round to the same
// fp16 unless a binary16 midpoint -- an fp32 value whose low 13 bits are
// 0x1000 in the normal binary16 range -- lies within that distance of q, or q
// is below the normal binary16 range.  Only then is the correctly rounded
// division taken.
__device__ __forceinline__ uint16_t dequant_w_zp_r(int cb, int zp, float nd, float rinv)
{
    if (!(nd > 0.0f))
        return 0;
    const float m = (float)(cb + zp);
    const float q = m * rinv;
    const unsigned b = __builtin_bit_cast(unsigned, q) & 0x7fffffffu;
    const bool near = b < 0x38800000u ? b != 0u : ((b & 0x1fffu) - 0x0ffbu) <= 10u;
    return f2h(near ? m / nd : q);
}

// FP8 variant.  Formats: E5M2 (5 exponent bits with bias 15, 2 fraction
// bits, largest finite 57344) and E4M3 (4 exponent bits with bias 7, 3
// fraction bits, no infinities, largest finite 448, subnormal step 2^-9);
// kF8None selects the int8 path wherever a format parameter appears.
enum { kF8None = 0, kF8E5M2 = 1, kF8E4M3 = 2 };

// Value of an FP8 code.  An E5M2 code is the high byte of the binary16 with
// the same value (same sign, exponent field and bias; 2 of the 10 fraction
// bits), so decoding is a shift.  E4M3: a normal code (exponent field e > 0)
// is the fp32 with exponent field e + 120 and the 3 fraction bits on top of
// its fraction; a subnormal one is f * 2^-9, exact in fp32.
template <int kFmt>
__device__ __forceinline__ float f8_to_f(unsigned c)
{
    if constexpr (kFmt == kF8E4M3) {
        const unsigned e = (c >> 3) & 15u, f = c & 7u;
        const float mag = e ? __builtin_bit_cast(float, ((e + 120u) << 23) | (f << 20))
                            : (float)f * 0.001953125f;
        return (c & 0x80u) ? -mag : mag;
    } else {
        return h2f((uint16_t)(c << 8));
    }
}

// The power of two 2^e that scales a vector with absmax a (an fp16 value, as
// fp32) into the format's range: e is the largest integer with a * 2^e <=
// 1.75 * 2^M, M = 15 (E5M2, 57344) or 8 (E4M3, 448); e = 0 for a = 0.  With
// a = f * 2^E, f in [1, 2): e = M - E for f <= 1.75, else M - 1 - E.
template <int kFmt>
__device__ __forceinline__ int f8_scale_exp(float a)
{
    constexpr int M = kFmt == kF8E4M3 ? 8 : 15;
    if (!(a > 0.0f))
        return 0;
    int ex;
    const float fr = __builtin_frexpf(a, &ex);   // a = fr * 2^ex, fr in [0.5, 1)
    return (2.0f * fr <= 1.75f ? M : M - 1) - (ex - 1);
}

// fp16 weight of FP8 code c in a column with scale sc (a power of two): the
// exact product rounded once.
template <int kFmt>
__device__ __forceinline__ uint16_t dequant_w_f8(unsigned c, float sc)
{
    return f2h(f8_to_f<kFmt>(c) * sc);
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

// Workspace segments of one llmint8_matmul call (byte offsets from the base);
// decode: the weight-streaming path's layout (no gathered weight operand,
// x_out for any outlier count).
struct MatmulWorkspace {
    size_t mask, groups, outlier_idx, info, row_absmax, row_zp, xq, x_out, w_out, kept, total;
};
MatmulWorkspace matmul_workspace_layout(int64_t T, int64_t K, int64_t N, bool decode);
size_t act_workspace_bytes(int64_t K);

// ---- launchers (each enqueues on `s`; return hipGetLastError()) ----
hipError_t launch_quantize_weight(const uint16_t *W_t, int64_t K, int64_t N, int8_t *CB,
                                  float *SCB, hipStream_t s);

// What the row-quantization launch needs for the GEMM path's outlier weight
// operand (w_out == null: not the GEMM path).  kOutFew: w_out[n, j] =
// fp16(CB[n,O[j]]*SCB[n]/127) for j < n_outliers, zero up to 32, row stride
// 32 halves; kOutCompact: w_out[n, j] = the code CB[n,O[j]] (int8), zero up
// to outlier_ld(n_outliers), which is the row stride; kOutDense: nothing.
struct GatherArgs {
    const int8_t *CB;
    const float *SCB;   // zero-point variant: nd of each column; FP8: scale 2^-e
    int64_t N;
    void *w_out;
    const int32_t *zp = nullptr;   // zero-point variant: zp of each column (else null)
    int f8 = kF8None;              // FP8 variant: the format of CB's codes
    int8_t *cb_kept = nullptr;     // kept-column mode's weight operand [N, kc] (null: off)
};

// Where the row quantization puts the outlier-set summary: info (n, ng,
// mode; info[0] is n_out) and the ascending list of non-empty 64-column
// groups (groups, K/64 entries).  groups null: only n and the outlier list
// are written.
struct OutlierInfoOut {
    int32_t *info;
    int32_t *groups = nullptr;
    uint8_t *mask = nullptr;   // GEMM path: the combined flags (dense mode only)
};

// The detection area `mask` of a call (detect_area_bytes(K)): the combined
// flags of every 8-column chunk (K/8 bytes, written by the row quantization
// for the GEMM kernel when it reads X in place), then nr flag sets (one per
// row range, `pitch` bytes apart) that k_detect writes and every
// row-quantization block ORs.  nr (a power of two, at most
// kDetectMaxRanges, each range of at least 256 rows) is the first that
// minimizes the busiest compute unit's share of the launch's K/64 * nr
// blocks, each over 1/nr of a 64-column slice's rows: a block streams its
// rows at the rate its compute unit's outstanding misses allow, so the
// launch runs at the pace of the CU with the most rows (K = 4096: 4 ranges;
// 2048: 8; 12288: 4, where one range left a quarter of the CUs idle; 16384:
// 1).
struct DetectFlags {
    const uint8_t *parts;
    int nr, pitch;
};
constexpr int kDetectMaxRanges = 8;
__host__ __device__ inline int64_t detect_pitch(int64_t K) { return (K / 8 + 15) / 16 * 16; }
inline size_t detect_area_bytes(int64_t K)
{
    const size_t a = ((size_t)K / 8 + 255) & ~(size_t)255;
    return a + (((size_t)kDetectMaxRanges * detect_pitch(K) + 255) & ~(size_t)255);
}
inline DetectFlags detect_flags(uint8_t *mask, int64_t T, int64_t K)
{
    constexpr int64_t kCUs = 256;
    const int64_t slices = K / 64;
    int nr = 1;
    int64_t best_num = (slices + kCUs - 1) / kCUs, best_den = 1;   // busiest CU: num/den slices
    for (int c = 2; c <= kDetectMaxRanges && T >= 256 * (int64_t)c; c *= 2) {
        const int64_t num = (slices * c + kCUs - 1) / kCUs;
        if (num * best_den < best_num * c) {
            best_num = num;
            best_den = c;
            nr = c;
        }
    }
    const size_t a = ((size_t)K / 8 + 255) & ~(size_t)255;
    return DetectFlags{mask + a, nr, (int)detect_pitch(K)};
}

// The row quantization takes a wavefront per row from kRowQuantWaveMinT rows
// on when the rows are at most kRowQuantWaveMaxK long (measured on MI355X:
// 15 vs 20 us at 2048 x 2048, equal at 4096 x 4096); otherwise a block of
// 256 threads per row, which keeps more loads in flight per row for long
// rows (49 vs 53 us at 4096 x 12288).
constexpr int64_t kRowQuantWaveMinT = 256;
constexpr int64_t kRowQuantWaveMaxK = 4096;

// Outlier detection (k_detect: the flags of every 8-column chunk into the
// detection area `mask`, see DetectFlags), then one launch that quantizes the rows and, in every block,
// derives the outlier set from those flags itself (block 0 writes the outlier list and the
// summary `io`), plus the GEMM path's outlier weight gather (g.w_out).
// x_out (fp16 [T, outlier_ld(n)]) receives the gathered outlier columns,
// zero-padded, when non-null: on the decode path (xq_packed or
// !g.w_out) for every outlier count, on the GEMM path unless the mode is
// kOutDense.  On the GEMM path nothing is written for a row when every
// column is an outlier (the int8 part is then zero).  xq_packed (T <= 16
// only) writes Xq in the decode kernel's fragment order [K/64][4][16][16]
// (16*K bytes; rows >= T are left as they are) instead of row-major [T, K].
hipError_t launch_quantize_act(const uint16_t *X, int64_t T, int64_t K, float threshold,
                               int8_t *Xq, float *a, int32_t *O, const OutlierInfoOut &io,
                               uint8_t *mask, uint16_t *x_out, const GatherArgs &g,
                               bool xq_packed, hipStream_t s);

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
    const void *w_out;       // GEMM path: kOutFew fp16 [N,32], kOutCompact int8 codes [N,ld]
    const int32_t *O;        // [n] outlier column indices (weight-streaming path)
    const int32_t *n_out;    // outlier-set summary {n, ng, mode} (weight-streaming path: n)
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
    // FP8 variant (f8 = kF8E5M2 or kF8E4M3): Xq and CB hold codes of that
    // format, a and scb the scales 2^-e of the rows and columns; the
    // products are summed in fp32 by fp8 MFMAs.
    int f8 = kF8None;
    // GEMM path, kOutDense: the activations, the chunk flags and the
    // non-empty 64-column groups
    const uint16_t *X = nullptr;
    const uint8_t *mask = nullptr;
    const int32_t *groups = nullptr;
    // kept-column mode (info[3] = kc > 0): the weight rows' kept codes [N, kc]
    const int8_t *cb_kept = nullptr;
};

// Zero-point variant (the asymmetric quantizer of the LLM.int8() summary,
// "8-bit Data Types and Quantization"): per vector, range [min(min,0),
// max(max,0)], d = max' - min', nd = 254/d (exact), zp = RNE(nd*min') + 127,
// code = RNE(nd*x) - zp (roundings of the exact rationals, ties to even); the
// stored nd is the fp32 value nearest to it; d = 0 gives nd = 0, zp = 0,
// codes 0.  Weight: per row of W_t over all K,
// with RS[n] the sum of the row's codes.  K <= kMaxKZp keeps the shifted
// product sum_k (A+zp_a)(B+zp_b), |A+zp| <= 254, inside int32.
constexpr int64_t kMaxKZp = 33286;
hipError_t launch_quantize_weight_zp(const uint16_t *W_t, int64_t K, int64_t N, int8_t *CB,
                                     float *ND, int32_t *ZP, int32_t *RS, hipStream_t s);
// Activations: as launch_quantize_act, but the non-outlier part of each row
// zero-point quantized (nd[t]; row_zp[t] = {zp, sum of the row's K codes});
// outlier columns hold the code of 0, -zp.  g.zp must be set when g.w_out
// is (the kOutFew outlier weight rows are then dequantized as
// fp16((cb+zp)/nd)).  Without w_out and for the shapes of
// quantize_act_fits_rows it is one launch (the few-rows kernel), else
// detection and a block per row.
hipError_t launch_quantize_act_zp(const uint16_t *X, int64_t T, int64_t K, float threshold,
                                  int8_t *Xq, float *nd, int2 *row_zp, int32_t *O,
                                  const OutlierInfoOut &io, uint8_t *mask, uint16_t *x_out,
                                  const GatherArgs &g, bool xq_packed, hipStream_t s);

// FP8 variant (fmt kF8E5M2: the 5-bit-exponent, 2-bit-fraction format the
// LLM.int8() summary names under "Related work"; kF8E4M3: the 4-bit-exponent
// one): per vector a power-of-two scale 2^e (f8_scale_exp of the absmax; the
// row absmax over the non-outlier columns), codes = the format's value
// nearest to x * 2^e (ties to even), stored scale 2^-e; outlier columns are
// +0.  Weight: per row of W_t.
hipError_t launch_quantize_weight_f8(const uint16_t *W_t, int64_t K, int64_t N, uint8_t *CB8,
                                     float *SC8, int fmt, hipStream_t s);
// Activations: as launch_quantize_act (same kernels with the FP8 codes;
// sc receives the row scales 2^-e); g.f8 must equal fmt when g.w_out is set.
hipError_t launch_quantize_act_f8(const uint16_t *X, int64_t T, int64_t K, float threshold,
                                  uint8_t *Xq8, float *sc, int32_t *O, const OutlierInfoOut &io,
                                  uint8_t *mask, uint16_t *x_out, const GatherArgs &g,
                                  bool xq_packed, int fmt, hipStream_t s);

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
