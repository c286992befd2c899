/*
 * llmint8_oracle.c -- plain CPU oracle of the LLM.int8() mixed-precision
 * decomposition matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no source, header, table or helper with the
 * HIP library.
 *
 * Every function is the definition written out, one output element at a
 * time, with no blocking, fusion or reordering.  Sources (the web pages this
 * follows):
 *   [HF]   agentlenshq.com, "Hugging Face, LLM.int8() 8-bit matrix
 *          multiplication integrated into Transformers and Accelerate":
 *          the three-step method, the absmax example, the Int8Params note
 *          that the fp16 weight is recovered as CB*SCB/127.
 *   [SUM]  kurtkim.github.io, "LLM.int8()" paper summary: the absmax
 *          equation (section "8-bit Data Types and Quantization"), the int32
 *          accumulation (section "Int8 Matrix Multiplication with 16-bit Float
 *          Inputs and Outputs"), vector-wise quantization (section
 *          "Vector-wise Quantization"), and the decomposition over the outlier
 *          set O with alpha = 6.0 (section "The Core of LLM.int8():
 *          Mixed-precision Decomposition").
 *   [QB]   techblog.paldyn.com, quantization basics: the binary16 layout
 *          (1 sign, 5 exponent, 10 fraction bits; largest finite 65504).
 *
 * Readings where the pages leave a step open (each one is listed, with its
 * reason, in the design notes):
 *   - rounding is to nearest with ties to even, of the exact rational value;
 *   - a column is an outlier when its largest |x| is strictly greater than
 *     the threshold;
 *   - the row absmax runs over the non-outlier columns only, and the int8
 *     matrix keeps outlier columns as zeros;
 *   - the weight absmax runs over all of K;
 *   - the outlier product uses the weight dequantized to fp16 from CB and
 *     SCB, because only CB and SCB exist once the weight is quantized;
 *   - the output is one rounding to fp16 of the exact-as-possible (fp64)
 *     sum of the dequantized int8 part, the outlier part and the bias.
 * The zero-point (asymmetric) and FP8 variants near the end of this file
 * have their own lists of readings there.
 *
 * fp16 values cross this interface as raw IEEE binary16 bit patterns
 * (uint16_t); the codec below is written from the bit layout.
 * Build: gcc -O2 -fopenmp -fno-fast-math -ffp-contract=off -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* binary16 codec ([QB] floating-point formats: 1 sign bit, 5 exponent bits  */
/* with bias 15, 10 fraction bits).                                          */
/* ------------------------------------------------------------------------ */

/* Exact value of a binary16 bit pattern. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);              /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);  /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Round a double to the nearest binary16 value, ties to even, in one step.
 * Magnitudes from 65520 (halfway between 65504 and 2^16) upward become inf. */
uint16_t oracle_double_to_half(double v)
{
    if (isnan(v))
        return 0x7e00;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return sign | 0x7c00;
    int e2;
    frexp(a, &e2);          /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;         /* binade exponent of a */
    if (E < -14)
        E = -14;            /* subnormals share the spacing of the lowest binade */
    if (E > 15)
        return sign | 0x7c00;
    double ulp = ldexp(1.0, E - 10);    /* spacing of binary16 values in [2^E, 2^(E+1)) */
    double q = a / ulp;                 /* exact: scaling by a power of two */
    double r = floor(q);
    double frac = q - r;                /* exact */
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0))
        r += 1.0;
    if (r >= 2048.0) {                  /* rounded up into the next binade */
        r = 1024.0;
        E += 1;
    }
    if (E > 15)
        return sign | 0x7c00;
    if (r < 1024.0)                     /* only possible for E == -14: subnormal */
        return sign | (uint16_t)r;
    return sign | (uint16_t)(((E + 15) << 10) | ((int)r - 1024));
}

/* |x| of a binary16 bit pattern, as a bit pattern (clear the sign bit).  For
 * finite values the unsigned order of these patterns is the order of the
 * magnitudes, so the max of patterns is the pattern of the max. */
static uint16_t half_abs_bits(uint16_t h) { return (uint16_t)(h & 0x7fff); }

/* Split a finite non-negative binary16 value into integer mantissa m and
 * exponent p with value = m * 2^p. */
static void half_split(uint16_t h, int64_t *m, int *p)
{
    int e = (h >> 10) & 31;
    int f = h & 1023;
    if (e == 0) {
        *m = f;
        *p = -24;
    } else {
        *m = 1024 + f;
        *p = e - 25;
    }
}

/* ------------------------------------------------------------------------ */
/* Absmax quantization ([SUM] "8-bit Data Types and Quantization": the int8   */
/* value is 127*x / max|X| rounded to the nearest integer).                  */
/* ------------------------------------------------------------------------ */

/* Nearest integer to the exact rational 127*x/a, ties to even, for binary16
 * values x and a with 0 < a and |x| <= a.  Written with integers so that no
 * floating-point rounding enters: 127*x/a = 127*mx*2^px / (ma*2^pa). */
int oracle_round_127x_over_a(uint16_t xh, uint16_t ah)
{
    uint16_t xa = half_abs_bits(xh);
    int64_t mx, ma;
    int px, pa;
    half_split(xa, &mx, &px);
    half_split(half_abs_bits(ah), &ma, &pa);
    if (ma == 0 || mx == 0)
        return 0;
    int d = px - pa;
    int64_t num, den;
    if (d >= 0) {            /* |x| <= a bounds num by 127*ma, so no overflow */
        num = (127 * mx) << d;
        den = ma;
    } else {                 /* -d <= 29 and ma < 2^11: den < 2^40 */
        num = 127 * mx;
        den = ma << (-d);
    }
    int64_t q = num / den;
    int64_t rem = num - q * den;
    if (2 * rem > den || (2 * rem == den && (q & 1)))
        q += 1;
    return (xh & 0x8000) ? (int)-q : (int)q;
}

/* Dequantized fp16 weight: the binary16 value nearest to CB*SCB/127 ([HF]
 * Int8Params note).  The product is exact in fp64 and the quotient is
 * correctly rounded in fp64; a rational with odd denominator 127 and
 * numerator on a grid no finer than SCB's lies at least 2^-18 of its binade
 * away from any binary16 midpoint, far more than the fp64 rounding error, so
 * this single conversion equals rounding the exact rational once. */
uint16_t oracle_dequant_weight(int8_t cb, float scb)
{
    return oracle_double_to_half(((double)cb * (double)scb) / 127.0);
}

/* ------------------------------------------------------------------------ */
/* Step: weight quantization ([HF] Int8Params: CB int8 in [-127,127] plus     */
/* SCB with W ~= CB*SCB/127; vector-wise means one scale per output column   */
/* of W, i.e. per row of the stored [N,K] weight).                           */
/* ------------------------------------------------------------------------ */

/* W_t: [N,K] binary16, row n holds output column n of W.  CB: [N,K] int8,
 * SCB: [N] float (the absmax, an fp16 value widened exactly). */
void oracle_quantize_weight(const uint16_t *W_t, int64_t K, int64_t N,
                            int8_t *CB, float *SCB)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const uint16_t *row = W_t + n * K;
        uint16_t amax = 0;
        for (int64_t k = 0; k < K; ++k)
            if (half_abs_bits(row[k]) > amax)
                amax = half_abs_bits(row[k]);
        SCB[n] = (float)oracle_half_to_double(amax);
        for (int64_t k = 0; k < K; ++k)
            CB[n * K + k] = (int8_t)oracle_round_127x_over_a(row[k], amax);
    }
}

/* ------------------------------------------------------------------------ */
/* Step: outlier feature columns ([HF] step 1; [SUM] mixed-precision          */
/* decomposition: O holds the hidden dimensions h with a value above alpha). */
/* ------------------------------------------------------------------------ */

/* colmax[k] = max_t |X[t,k]|; O = { k : colmax[k] > threshold } in ascending
 * order.  Returns n = |O|.  O needs room for K entries. */
int64_t oracle_outlier_columns(const uint16_t *X, int64_t T, int64_t K,
                               float threshold, int32_t *O)
{
    int64_t n = 0;
    for (int64_t k = 0; k < K; ++k) {
        uint16_t cmax = 0;
        for (int64_t t = 0; t < T; ++t)
            if (half_abs_bits(X[t * K + k]) > cmax)
                cmax = half_abs_bits(X[t * K + k]);
        if (oracle_half_to_double(cmax) > (double)threshold)
            O[n++] = (int32_t)k;
    }
    return n;
}

/* Membership table of O over 0..K-1 (1 = outlier column). */
static unsigned char *outlier_mask(const int32_t *O, int64_t n, int64_t K)
{
    unsigned char *m = (unsigned char *)calloc((size_t)K, 1);
    for (int64_t j = 0; j < n; ++j)
        m[O[j]] = 1;
    return m;
}

/* ------------------------------------------------------------------------ */
/* Step: row-wise absmax quantization of the non-outlier part ([HF] step 2:  */
/* activations row-wise; [SUM] the int8 sum runs over h not in O).           */
/* ------------------------------------------------------------------------ */

/* For each listed row t: a[t] = max_{k not in O} |X[t,k]| (0 if none);
 * Xq[t,k] = 0 for k in O, else nearest integer to 127*X[t,k]/a[t] (0 when
 * a[t] = 0).  rows == NULL means all T rows; Xq/a are indexed by position i
 * in the row list (Xq: [nrows,K], a: [nrows]). */
void oracle_quantize_rows(const uint16_t *X, int64_t T, int64_t K,
                          const int32_t *O, int64_t n,
                          const int64_t *rows, int64_t nrows,
                          int8_t *Xq, float *a)
{
    unsigned char *isout = outlier_mask(O, n, K);
    if (rows == NULL)
        nrows = T;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t t = rows ? rows[i] : i;
        const uint16_t *xr = X + t * K;
        uint16_t amax = 0;
        for (int64_t k = 0; k < K; ++k)
            if (!isout[k] && half_abs_bits(xr[k]) > amax)
                amax = half_abs_bits(xr[k]);
        a[i] = (float)oracle_half_to_double(amax);
        for (int64_t k = 0; k < K; ++k)
            Xq[i * K + k] = isout[k] ? 0 : (int8_t)oracle_round_127x_over_a(xr[k], amax);
    }
    free(isout);
}

/* ------------------------------------------------------------------------ */
/* Step: int8 matrix product with 32-bit integer result ([SUM] "Int8 Matrix  */
/* Multiplication with 16-bit Float Inputs and Outputs": C_i32 = A_i8 B_i8). */
/* ------------------------------------------------------------------------ */

/* C[i,n] = sum_k Xq[i,k] * CB[n,k], summed in int64.  Xq: [M,K], CB: [N,K],
 * C: [M,N].  Returns the number of sums that do not fit in int32 (those are
 * stored clamped); 0 is the expected result for K <= 133144. */
int64_t oracle_int_gemm(const int8_t *Xq, const int8_t *CB, int64_t M,
                        int64_t K, int64_t N, int32_t *C)
{
    int64_t bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)Xq[i * K + k] * (int64_t)CB[n * K + k];
            if (s > INT32_MAX) {
                s = INT32_MAX;
                ++bad;
            } else if (s < INT32_MIN) {
                s = INT32_MIN;
                ++bad;
            }
            C[i * N + n] = (int32_t)s;
        }
    }
    return bad;
}

/* ------------------------------------------------------------------------ */
/* The whole decomposition for a list of output rows ([SUM] mixed-precision  */
/* decomposition: C ~= sum_{h in O} X^h W^h + S * sum_{h not in O} Xi8 Wi8,   */
/* with S the outer product of the row and column scales over 127^2; [HF]    */
/* step 3: dequantize the int8 result and add the fp16 outlier result).      */
/* ------------------------------------------------------------------------ */

/* out[i,c] = fp16( C[t,c]*a[t]*SCB[c]/127^2
 *                  + sum_{k in O} X[t,k] * Wdq(CB[c,k], SCB[c])  [+ bias[c]] )
 * for t = rows[i] (all rows when rows == NULL) and c = cols[j] (all N
 * columns when cols == NULL).  O is found from all T rows of X.
 * out: [nrows, ncols]; bias: [N] binary16 or NULL.  If O_out / n_out are
 * given they receive O and n; a_out ([nrows]) receives the row scales.
 * Returns the number of int32 overflows in C (0 expected). */
int64_t oracle_matmul(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                      const int8_t *CB, const float *SCB, const uint16_t *bias,
                      float threshold, const int64_t *rows, int64_t nrows,
                      const int64_t *cols, int64_t ncols, uint16_t *out,
                      int32_t *O_out, int64_t *n_out, float *a_out)
{
    if (rows == NULL)
        nrows = T;
    if (cols == NULL)
        ncols = N;
    int32_t *O = (int32_t *)malloc(sizeof(int32_t) * (size_t)(K > 0 ? K : 1));
    int64_t n = oracle_outlier_columns(X, T, K, threshold, O);
    int8_t *Xq = (int8_t *)malloc((size_t)(nrows * K > 0 ? nrows * K : 1));
    float *a = (float *)malloc(sizeof(float) * (size_t)(nrows > 0 ? nrows : 1));
    oracle_quantize_rows(X, T, K, O, n, rows, nrows, Xq, a);
    int64_t bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t t = rows ? rows[i] : i;
        for (int64_t j = 0; j < ncols; ++j) {
            int64_t c = cols ? cols[j] : j;
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)Xq[i * K + k] * (int64_t)CB[c * K + k];
            if (s > INT32_MAX || s < INT32_MIN)
                ++bad;
            /* dequantized int8 part: C * a[t] * SCB[c] / 127^2 */
            double acc = (double)s * (double)a[i] * (double)SCB[c] / 16129.0;
            /* fp16 outlier part, over O in ascending order */
            for (int64_t jj = 0; jj < n; ++jj) {
                int64_t k = O[jj];
                acc += oracle_half_to_double(X[t * K + k]) *
                       oracle_half_to_double(oracle_dequant_weight(CB[c * K + k], SCB[c]));
            }
            if (bias)
                acc += oracle_half_to_double(bias[c]);
            out[i * ncols + j] = oracle_double_to_half(acc);
        }
    }
    if (O_out)
        memcpy(O_out, O, sizeof(int32_t) * (size_t)n);
    if (n_out)
        *n_out = n;
    if (a_out)
        memcpy(a_out, a, sizeof(float) * (size_t)nrows);
    free(O);
    free(Xq);
    free(a);
    return bad;
}

/* ------------------------------------------------------------------------ */
/* Zero-point (asymmetric) vector-wise variant ([SUM] "8-bit Data Types and  */
/* Quantization", zeropoint quantization: scale by the normalized dynamic    */
/* range nd = 2*127/(max - min), shift by an integer zero point zp so that   */
/* the values fill [-127, 127]; the product of two such numbers is           */
/* (A_i8 + zp_a)(B_i8 + zp_b), accumulated in int32 and dequantized by       */
/* dividing by nd_a*nd_b; [SUM] "Int8 Matrix Multiplication with 16-bit      */
/* Float Inputs and Outputs" names nd_x, nd_w as the zeropoint constants).   */
/*                                                                            */
/* Readings (the page's zero-point formulas are garbled; these are the       */
/* plainest consistent ones, each listed in the design notes):               */
/*   - one (nd, zp) per vector: per row of X over its non-outlier columns,   */
/*     per output column of W over all of K (vector-wise, like the absmax    */
/*     variant);                                                             */
/*   - the range always contains 0: min' = min(min, 0), max' = max(max, 0),  */
/*     so zp fits the page's int16 (it lies in [-127, 127]), the value 0 has */
/*     an exact code (-zp), and every |A_i8 + zp| <= 254;                    */
/*   - nd = 254 / (max' - min') is the exact rational, as round(127 x / a)   */
/*     is in the absmax variant: the page fixes no precision, so nothing is  */
/*     rounded before the codes; d = max' - min' = 0 (an all-zero vector)    */
/*     gives nd = 0, zp = 0 and codes 0;                                     */
/*   - zp = RNE(nd * min') + 127 and A_i8 = RNE(nd * x) - zp, roundings of   */
/*     the exact rationals to the nearest integer, ties to even; then        */
/*     A_i8 + zp runs from RNE(nd * min') to RNE(nd * min' + 254) =          */
/*     RNE(nd * min') + 254, so every code lies in [-127, 127] with no clamp; */
/*   - what is stored for dequantization (ND of a weight column, nd of an    */
/*     activation row) is the fp32 value nearest to the exact nd;            */
/*   - outlier columns hold the code of 0, -zp, so that A_i8 + zp_a = 0      */
/*     there and they add nothing to the integer product;                    */
/*   - the fp16 outlier product uses the weight dequantized from the stored  */
/*     values as fp16(fp32(CB + zp) / ND) (one fp32 division, then one       */
/*     rounding to fp16; 0 when ND = 0).                                     */
/* fp16 values are integer multiples of 2^-24, so with X = x * 2^24 and      */
/* D = d * 2^24 (integers, |X| < 2^40, D < 2^41) every rational here is a    */
/* quotient of integers: nd * x = 254 X / D.                                 */
/* ------------------------------------------------------------------------ */

/* x * 2^24 as an integer (exact for every binary16 value). */
static int64_t fixed24(double x)
{
    return (int64_t)ldexp(x, 24);
}

/* num / den rounded to the nearest integer, ties to even (den > 0). */
static int64_t rne_ratio(int64_t num, int64_t den)
{
    int64_t q = num / den, r = num % den;     /* C division truncates toward 0 */
    if (r < 0) {                              /* make it floor: 0 <= r < den */
        q -= 1;
        r += den;
    }
    if (2 * r > den || (2 * r == den && (q & 1)))
        q += 1;
    return q;
}

/* The fp32 value nearest to 254 * 2^24 / D (ties to even), D > 0: the
 * quotient scaled by a power of two into [2^23, 2^24), rounded as an
 * integer. */
static float nearest_f32_nd(int64_t D)
{
    unsigned __int128 num = (unsigned __int128)254 << 24, den = (unsigned __int128)D;
    int e = 0;                                 /* value = (num / den) * 2^-e */
    while (num / den >= ((unsigned __int128)1 << 24)) {
        den <<= 1;                             /* halves the quotient */
        --e;
    }
    while (num / den < ((unsigned __int128)1 << 23)) {
        num <<= 1;                             /* doubles the quotient */
        ++e;
    }
    unsigned __int128 q = num / den, r = num % den;
    if (2 * r > den || (2 * r == den && (q & 1)))
        q += 1;
    return (float)ldexp((double)(uint64_t)q, -e);
}

/* The zero-point parameters of one vector from its smallest and largest
 * value (binary16, already widened to double) with 0 added to the range:
 * D = (max' - min') * 2^24, the stored nd and zp. */
static void zp_params(double vmin, double vmax, int64_t *D, float *nd, int32_t *zp)
{
    if (vmin > 0.0)
        vmin = 0.0;
    if (vmax < 0.0)
        vmax = 0.0;
    *D = fixed24(vmax) - fixed24(vmin);
    if (*D == 0) {
        *nd = 0.0f;
        *zp = 0;
        return;
    }
    *nd = nearest_f32_nd(*D);
    *zp = (int32_t)(rne_ratio(254 * fixed24(vmin), *D) + 127);
}

/* Code of value x in a vector with parameters (D, zp). */
static int8_t zp_code(int64_t D, int32_t zp, double x)
{
    if (D == 0)
        return 0;
    return (int8_t)(rne_ratio(254 * fixed24(x), D) - zp);
}

/* Dequantized fp16 weight of code cb in a column with parameters (nd, zp). */
uint16_t oracle_dequant_weight_zp(int8_t cb, int32_t zp, float nd)
{
    if (nd == 0.0f)
        return 0;
    float w = (float)(cb + zp) / nd;          /* exact numerator, one division */
    return oracle_double_to_half((double)w);  /* fp32 -> fp16, one rounding */
}

/* W_t: [N,K] binary16.  CB: [N,K] int8 codes, ND: [N] nd, ZP: [N] zp. */
void oracle_quantize_weight_zp(const uint16_t *W_t, int64_t K, int64_t N,
                               int8_t *CB, float *ND, int32_t *ZP)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const uint16_t *row = W_t + n * K;
        double vmin = 0.0, vmax = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double v = oracle_half_to_double(row[k]);
            if (v < vmin)
                vmin = v;
            if (v > vmax)
                vmax = v;
        }
        int64_t D;
        zp_params(vmin, vmax, &D, &ND[n], &ZP[n]);
        for (int64_t k = 0; k < K; ++k)
            CB[n * K + k] = zp_code(D, ZP[n], oracle_half_to_double(row[k]));
    }
}

/* For each listed row t (all T when rows == NULL): (nd, zp) over the
 * non-outlier columns, Xq[i,k] = the code of X[t,k] for k not in O and -zp
 * (the code of 0) for k in O. */
void oracle_quantize_rows_zp(const uint16_t *X, int64_t T, int64_t K,
                             const int32_t *O, int64_t n,
                             const int64_t *rows, int64_t nrows,
                             int8_t *Xq, float *nd, int32_t *zp)
{
    unsigned char *isout = outlier_mask(O, n, K);
    if (rows == NULL)
        nrows = T;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t t = rows ? rows[i] : i;
        const uint16_t *xr = X + t * K;
        double vmin = 0.0, vmax = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            if (isout[k])
                continue;
            double v = oracle_half_to_double(xr[k]);
            if (v < vmin)
                vmin = v;
            if (v > vmax)
                vmax = v;
        }
        int64_t D;
        zp_params(vmin, vmax, &D, &nd[i], &zp[i]);
        for (int64_t k = 0; k < K; ++k)
            Xq[i * K + k] = isout[k] ? (int8_t)(-zp[i])
                                     : zp_code(D, zp[i], oracle_half_to_double(xr[k]));
    }
    free(isout);
}

/* out[i,c] = fp16( sum_k (Xq[t,k] + zp_a[t]) * (CB[c,k] + ZP[c]) / (nd_a[t] * ND[c])
 *                  + sum_{k in O} X[t,k] * Wdq_zp(CB[c,k], ZP[c], ND[c])  [+ bias[c]] )
 * with the shifted products summed directly in int64 (the page's 16-bit
 * multiply form, no unrolling) and the rest in fp64, rounded once.  A zero
 * nd on either side makes the integer term 0.  Arguments as oracle_matmul;
 * nd_out / zp_out ([nrows]) receive the row parameters.  Returns the number
 * of integer sums outside int32 (0 expected for K <= 33286). */
int64_t oracle_matmul_zp(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                         const int8_t *CB, const float *ND, const int32_t *ZP,
                         const uint16_t *bias, float threshold,
                         const int64_t *rows, int64_t nrows,
                         const int64_t *cols, int64_t ncols, uint16_t *out,
                         int32_t *O_out, int64_t *n_out, float *nd_out, int32_t *zp_out)
{
    if (rows == NULL)
        nrows = T;
    if (cols == NULL)
        ncols = N;
    int32_t *O = (int32_t *)malloc(sizeof(int32_t) * (size_t)(K > 0 ? K : 1));
    int64_t n = oracle_outlier_columns(X, T, K, threshold, O);
    int8_t *Xq = (int8_t *)malloc((size_t)(nrows * K > 0 ? nrows * K : 1));
    float *nd = (float *)malloc(sizeof(float) * (size_t)(nrows > 0 ? nrows : 1));
    int32_t *zp = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nrows > 0 ? nrows : 1));
    oracle_quantize_rows_zp(X, T, K, O, n, rows, nrows, Xq, nd, zp);
    int64_t bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t t = rows ? rows[i] : i;
        for (int64_t j = 0; j < ncols; ++j) {
            int64_t c = cols ? cols[j] : j;
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += ((int64_t)Xq[i * K + k] + zp[i]) * ((int64_t)CB[c * K + k] + ZP[c]);
            if (s > INT32_MAX || s < INT32_MIN)
                ++bad;
            double acc = 0.0;
            if (nd[i] != 0.0f && ND[c] != 0.0f)
                acc = (double)s / ((double)nd[i] * (double)ND[c]);
            for (int64_t jj = 0; jj < n; ++jj) {
                int64_t k = O[jj];
                acc += oracle_half_to_double(X[t * K + k]) *
                       oracle_half_to_double(oracle_dequant_weight_zp(CB[c * K + k], ZP[c], ND[c]));
            }
            if (bias)
                acc += oracle_half_to_double(bias[c]);
            out[i * ncols + j] = oracle_double_to_half(acc);
        }
    }
    if (O_out)
        memcpy(O_out, O, sizeof(int32_t) * (size_t)n);
    if (n_out)
        *n_out = n;
    if (nd_out)
        memcpy(nd_out, nd, sizeof(float) * (size_t)nrows);
    if (zp_out)
        memcpy(zp_out, zp, sizeof(int32_t) * (size_t)nrows);
    free(O);
    free(Xq);
    free(nd);
    free(zp);
    return bad;
}

/* Element-wise form of oracle_dequant_weight_zp (for the tests). */
void oracle_dequant_weight_zp_n(const int8_t *cb, const int32_t *zp, const float *nd,
                                int64_t len, uint16_t *out)
{
    for (int64_t i = 0; i < len; ++i)
        out[i] = oracle_dequant_weight_zp(cb[i], zp[i], nd[i]);
}

/* ------------------------------------------------------------------------ */
/* FP8 variant ([SUM] "Related work", 8-bit data types: floating-point 8-bit */
/* formats with a 5-bit exponent and a 2-bit fraction are the common kind;   */
/* "Discussion and Limitations": the Int8 findings are expected to carry     */
/* over to FP8).  The same decomposition with the non-outlier part in E5M2.  */
/*                                                                            */
/* Readings (the pages give no FP8 procedure; each is listed in the design   */
/* notes):                                                                   */
/*   - E5M2 is the binary16 layout with a 2-bit fraction: sign, 5 exponent   */
/*     bits with bias 15, 2 fraction bits; subnormals step 2^-16; largest    */
/*     finite 57344;                                                         */
/*   - vector-wise scaling as in the int8 method, by a power of two: each    */
/*     vector is multiplied by 2^e, e the largest integer with               */
/*     absmax * 2^e <= 57344 (e = 0 for an all-zero vector), so the scaling  */
/*     is exact and the only rounding is to E5M2 (nearest, ties to even);    */
/*     the stored scale is 2^-e, the factor that undoes it;                  */
/*   - the row scale runs over the non-outlier columns, outlier columns are  */
/*     +0 in the FP8 matrix, and the weight scale over all of K;             */
/*   - the FP8 products are summed in fp64 here (the kernels accumulate in   */
/*     fp32; the sum's rounding order is not fixed by the method);           */
/*   - the outlier product uses the weight dequantized to fp16: the E5M2     */
/*     value times its scale, rounded once to binary16.                      */
/* ------------------------------------------------------------------------ */

/* Exact value of an E5M2 code. */
double oracle_e5m2_to_double(uint8_t c)
{
    int sign = (c >> 7) & 1;
    int e = (c >> 2) & 31;
    int f = c & 3;
    double v;
    if (e == 0)
        v = ldexp((double)f, -16);              /* subnormal: f/4 * 2^-14 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(4 + f), e - 17);     /* (1 + f/4) * 2^(e-15) */
    return sign ? -v : v;
}

/* Nearest E5M2 code to v, ties to even; |v| beyond 61440 (halfway between
 * 57344 and 2^16) gives infinity. */
uint8_t oracle_double_to_e5m2(double v)
{
    if (isnan(v))
        return 0x7f;
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return sign | 0x7c;
    int e2;
    frexp(a, &e2);
    int E = e2 - 1;                     /* a in [2^E, 2^(E+1)) */
    if (E < -14)
        E = -14;                        /* subnormals share the lowest binade's spacing */
    if (E > 15)
        return sign | 0x7c;
    double ulp = ldexp(1.0, E - 2);
    double q = a / ulp;                 /* exact */
    double r = floor(q);
    double frac = q - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0))
        r += 1.0;
    if (r >= 8.0) {                     /* carried into the next binade */
        r = 4.0;
        E += 1;
    }
    if (E > 15)
        return sign | 0x7c;
    if (r < 4.0)                        /* only for E == -14: subnormal */
        return sign | (uint8_t)r;
    return sign | (uint8_t)(((E + 15) << 2) | ((int)r - 4));
}

/* The scaling exponent of a vector with absmax amax (a binary16 value):
 * the largest e with amax * 2^e <= 57344; 0 when amax is 0. */
int oracle_f8_scale_exp(double amax)
{
    if (amax == 0.0)
        return 0;
    int e = 0;
    while (ldexp(amax, e) > 57344.0)
        --e;
    while (ldexp(amax, e + 1) <= 57344.0)
        ++e;
    return e;
}

/* ------------------------------------------------------------------------ */
/* E4M3, the other common 8-bit floating-point format (4 exponent bits with  */
/* bias 7, 3 fraction bits, the "fn" layout: no infinities, S.1111.111 is    */
/* NaN, largest finite 1.75 * 2^8 = 448, subnormals step 2^-9).  The pages   */
/* name only the 5-bit-exponent kind; the E4M3 form of the variant takes     */
/* every reading of the E5M2 one with this format in its place (the scale    */
/* targets 448).                                                             */
/* ------------------------------------------------------------------------ */

/* Exact value of an E4M3 code. */
double oracle_e4m3_to_double(uint8_t c)
{
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 15;
    int f = c & 7;
    double v;
    if (e == 0)
        v = ldexp((double)f, -9);               /* subnormal: f/8 * 2^-6 */
    else if (e == 15 && f == 7)
        v = NAN;
    else
        v = ldexp((double)(8 + f), e - 10);     /* (1 + f/8) * 2^(e-7) */
    return sign ? -v : v;
}

/* Nearest E4M3 code to v, ties to even; a value that rounds above 448
 * (|v| > 464, past the tie with the next step, which goes to the even 448)
 * has no code and gives NaN. */
uint8_t oracle_double_to_e4m3(double v)
{
    if (isnan(v))
        return 0x7f;
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return sign | 0x7f;
    int e2;
    frexp(a, &e2);
    int E = e2 - 1;                     /* a in [2^E, 2^(E+1)) */
    if (E < -6)
        E = -6;                         /* subnormals share the lowest binade's spacing */
    if (E > 8)
        return sign | 0x7f;
    double ulp = ldexp(1.0, E - 3);
    double q = a / ulp;                 /* exact */
    double r = floor(q);
    double frac = q - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0))
        r += 1.0;
    if (r >= 16.0) {                    /* carried into the next binade */
        r = 8.0;
        E += 1;
    }
    if (E > 8 || (E == 8 && r > 14.0))  /* beyond 448 */
        return sign | 0x7f;
    if (r < 8.0)                        /* only for E == -6: subnormal */
        return sign | (uint8_t)r;
    return sign | (uint8_t)(((E + 7) << 3) | ((int)r - 8));
}

/* Format codes of the FP8 functions below: 1 = E5M2, 2 = E4M3. */
static double f8_value(uint8_t c, int fmt)
{
    return fmt == 2 ? oracle_e4m3_to_double(c) : oracle_e5m2_to_double(c);
}

static uint8_t f8_code(double v, int fmt)
{
    return fmt == 2 ? oracle_double_to_e4m3(v) : oracle_double_to_e5m2(v);
}

/* The scaling exponent in format fmt: the largest e with amax * 2^e at most
 * the format's largest finite value (57344 or 448); 0 when amax is 0. */
int oracle_f8_scale_exp_fmt(double amax, int fmt)
{
    if (fmt != 2)
        return oracle_f8_scale_exp(amax);
    if (amax == 0.0)
        return 0;
    int e = 0;
    while (ldexp(amax, e) > 448.0)
        --e;
    while (ldexp(amax, e + 1) <= 448.0)
        ++e;
    return e;
}

/* W_t: [N,K] binary16.  CB8: [N,K] E5M2 codes, SC8: [N] scale 2^-e. */
void oracle_quantize_weight_f8_fmt(const uint16_t *W_t, int64_t K, int64_t N,
                                   uint8_t *CB8, float *SC8, int fmt);
void oracle_quantize_weight_f8(const uint16_t *W_t, int64_t K, int64_t N,
                               uint8_t *CB8, float *SC8)
{
    oracle_quantize_weight_f8_fmt(W_t, K, N, CB8, SC8, 1);
}

/* The same in format fmt (codes of that format, scale 2^-e for its e). */
void oracle_quantize_weight_f8_fmt(const uint16_t *W_t, int64_t K, int64_t N,
                                   uint8_t *CB8, float *SC8, int fmt)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const uint16_t *row = W_t + n * K;
        uint16_t amax = 0;
        for (int64_t k = 0; k < K; ++k)
            if (half_abs_bits(row[k]) > amax)
                amax = half_abs_bits(row[k]);
        int e = oracle_f8_scale_exp_fmt(oracle_half_to_double(amax), fmt);
        SC8[n] = (float)ldexp(1.0, -e);
        for (int64_t k = 0; k < K; ++k)
            CB8[n * K + k] = f8_code(ldexp(oracle_half_to_double(row[k]), e), fmt);
    }
}

/* For each listed row t: the scale over the non-outlier columns, Xq8[i,k] =
 * +0 for k in O, else the code (format fmt) of X[t,k] * 2^e. */
void oracle_quantize_rows_f8_fmt(const uint16_t *X, int64_t T, int64_t K,
                                 const int32_t *O, int64_t n,
                                 const int64_t *rows, int64_t nrows,
                                 uint8_t *Xq8, float *sc8, int fmt)
{
    unsigned char *isout = outlier_mask(O, n, K);
    if (rows == NULL)
        nrows = T;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t t = rows ? rows[i] : i;
        const uint16_t *xr = X + t * K;
        uint16_t amax = 0;
        for (int64_t k = 0; k < K; ++k)
            if (!isout[k] && half_abs_bits(xr[k]) > amax)
                amax = half_abs_bits(xr[k]);
        int e = oracle_f8_scale_exp_fmt(oracle_half_to_double(amax), fmt);
        sc8[i] = (float)ldexp(1.0, -e);
        for (int64_t k = 0; k < K; ++k)
            Xq8[i * K + k] = isout[k] ? 0 : f8_code(ldexp(oracle_half_to_double(xr[k]), e), fmt);
    }
    free(isout);
}

/* E5M2 rows (the original form). */
void oracle_quantize_rows_f8(const uint16_t *X, int64_t T, int64_t K,
                             const int32_t *O, int64_t n,
                             const int64_t *rows, int64_t nrows,
                             uint8_t *Xq8, float *sc8)
{
    oracle_quantize_rows_f8_fmt(X, T, K, O, n, rows, nrows, Xq8, sc8, 1);
}

/* Dequantized fp16 weight of an E5M2 code with scale sc (a power of two):
 * the exact product rounded once to binary16. */
uint16_t oracle_dequant_weight_f8(uint8_t c, float sc)
{
    return oracle_double_to_half(oracle_e5m2_to_double(c) * (double)sc);
}

/* The same for a code of format fmt. */
uint16_t oracle_dequant_weight_f8_fmt(uint8_t c, float sc, int fmt)
{
    return oracle_double_to_half(f8_value(c, fmt) * (double)sc);
}

/* out[i,c] = fp16( sum_k e5m2(Xq8[t,k]) * e5m2(CB8[c,k]) * sc8[t] * SC8[c]
 *                  + sum_{k in O} X[t,k] * Wdq8(CB8[c,k], SC8[c])  [+ bias[c]] ),
 * the sum in fp64, rounded once.  Arguments as oracle_matmul; sc_out
 * ([nrows]) receives the row scales. */
void oracle_matmul_f8_fmt(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                          const uint8_t *CB8, const float *SC8, const uint16_t *bias,
                          float threshold, const int64_t *rows, int64_t nrows,
                          const int64_t *cols, int64_t ncols, uint16_t *out,
                          int32_t *O_out, int64_t *n_out, float *sc_out, int fmt);
void oracle_matmul_f8(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                      const uint8_t *CB8, const float *SC8, const uint16_t *bias,
                      float threshold, const int64_t *rows, int64_t nrows,
                      const int64_t *cols, int64_t ncols, uint16_t *out,
                      int32_t *O_out, int64_t *n_out, float *sc_out)
{
    oracle_matmul_f8_fmt(X, T, K, N, CB8, SC8, bias, threshold, rows, nrows, cols, ncols, out,
                         O_out, n_out, sc_out, 1);
}

/* The same in format fmt (1 = E5M2, 2 = E4M3): codes and the dequantized
 * outlier weights of that format. */
void oracle_matmul_f8_fmt(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                          const uint8_t *CB8, const float *SC8, const uint16_t *bias,
                          float threshold, const int64_t *rows, int64_t nrows,
                          const int64_t *cols, int64_t ncols, uint16_t *out,
                          int32_t *O_out, int64_t *n_out, float *sc_out, int fmt)
{
    if (rows == NULL)
        nrows = T;
    if (cols == NULL)
        ncols = N;
    int32_t *O = (int32_t *)malloc(sizeof(int32_t) * (size_t)(K > 0 ? K : 1));
    int64_t n = oracle_outlier_columns(X, T, K, threshold, O);
    uint8_t *Xq8 = (uint8_t *)malloc((size_t)(nrows * K > 0 ? nrows * K : 1));
    float *sc = (float *)malloc(sizeof(float) * (size_t)(nrows > 0 ? nrows : 1));
    oracle_quantize_rows_f8_fmt(X, T, K, O, n, rows, nrows, Xq8, sc, fmt);
    double lut[256];
    for (int v = 0; v < 256; ++v)
        lut[v] = f8_value((uint8_t)v, fmt);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t t = rows ? rows[i] : i;
        for (int64_t j = 0; j < ncols; ++j) {
            int64_t c = cols ? cols[j] : j;
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s += lut[Xq8[i * K + k]] * lut[CB8[c * K + k]];
            double acc = s * (double)sc[i] * (double)SC8[c];
            for (int64_t jj = 0; jj < n; ++jj) {
                int64_t k = O[jj];
                acc += oracle_half_to_double(X[t * K + k]) *
                       oracle_half_to_double(oracle_dequant_weight_f8_fmt(CB8[c * K + k], SC8[c], fmt));
            }
            if (bias)
                acc += oracle_half_to_double(bias[c]);
            out[i * ncols + j] = oracle_double_to_half(acc);
        }
    }
    if (O_out)
        memcpy(O_out, O, sizeof(int32_t) * (size_t)n);
    if (n_out)
        *n_out = n;
    if (sc_out)
        memcpy(sc_out, sc, sizeof(float) * (size_t)nrows);
    free(O);
    free(Xq8);
    free(sc);
}

void oracle_e5m2_to_double_n(const uint8_t *c, int64_t len, double *out)
{
    for (int64_t i = 0; i < len; ++i)
        out[i] = oracle_e5m2_to_double(c[i]);
}

void oracle_double_to_e5m2_n(const double *v, int64_t len, uint8_t *out)
{
    for (int64_t i = 0; i < len; ++i)
        out[i] = oracle_double_to_e5m2(v[i]);
}

void oracle_f8_scale_exp_n(const double *a, int64_t len, int32_t *out)
{
    for (int64_t i = 0; i < len; ++i)
        out[i] = oracle_f8_scale_exp(a[i]);
}

void oracle_e4m3_to_double_n(const uint8_t *c, int64_t len, double *out)
{
    for (int64_t i = 0; i < len; ++i)
        out[i] = oracle_e4m3_to_double(c[i]);
}

void oracle_double_to_e4m3_n(const double *v, int64_t len, uint8_t *out)
{
    for (int64_t i = 0; i < len; ++i)
        out[i] = oracle_double_to_e4m3(v[i]);
}

void oracle_f8_scale_exp_fmt_n(const double *a, int64_t len, int32_t *out, int fmt)
{
    for (int64_t i = 0; i < len; ++i)
        out[i] = oracle_f8_scale_exp_fmt(a[i], fmt);
}

/* Number of threads the parallel loops use (for reporting the CPU baseline). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Element-wise array forms of the scalar helpers above (for the tests).     */
/* ------------------------------------------------------------------------ */

void oracle_half_to_double_n(const uint16_t *h, int64_t len, double *out)
{
    for (int64_t i = 0; i < len; ++i)
        out[i] = oracle_half_to_double(h[i]);
}

void oracle_double_to_half_n(const double *v, int64_t len, uint16_t *out)
{
    for (int64_t i = 0; i < len; ++i)
        out[i] = oracle_double_to_half(v[i]);
}

void oracle_round_127x_over_a_n(const uint16_t *x, const uint16_t *a,
                                int64_t len, int32_t *out)
{
    for (int64_t i = 0; i < len; ++i)
        out[i] = oracle_round_127x_over_a(x[i], a[i]);
}

void oracle_dequant_weight_n(const int8_t *cb, const float *scb, int64_t len,
                             uint16_t *out)
{
    for (int64_t i = 0; i < len; ++i)
        out[i] = oracle_dequant_weight(cb[i], scb[i]);
}
