// quant.hip -- weight quantization and activation quantization kernels.
//
// Weight quantization follows the Int8Params note of the Hugging Face
// LLM.int8() write-up (agentlenshq.com, section "Integration into
// transformers": int8 CB in [-127,127] plus SCB, W ~= CB*SCB/127), per output
// column (LLM.int8() summary, kurtkim.github.io, "Vector-wise Quantization").
// Activation quantization follows steps 1-2 of the write-up's "Core idea" and
// the summary's "The Core of LLM.int8(): Mixed-precision Decomposition": the
// outlier set O is every column with some |x| > threshold, and the remaining
// columns are absmax-quantized per row ("8-bit Data Types and Quantization").
//
// All of these kernels are HBM-bound streams over X or W: 16-byte loads per
// lane (8 fp16 values), whole rows per wavefront, reductions with cross-lane
// shuffles, no LDS.

#include "internal.h"

namespace llmint8 {
namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;

__device__ __forceinline__ unsigned abs_lo(unsigned w) { return w & 0x7fffu; }
__device__ __forceinline__ unsigned abs_hi(unsigned w) { return (w >> 16) & 0x7fffu; }
__device__ __forceinline__ unsigned umax(unsigned a, unsigned b) { return a > b ? a : b; }

// Max of |x| over the 8 fp16 values of a 16-byte chunk.  |x| bit patterns of
// finite values order like the magnitudes, so integer max is magnitude max.
__device__ __forceinline__ unsigned chunk_absmax(uint4 v)
{
    unsigned m = umax(abs_lo(v.x), abs_hi(v.x));
    m = umax(m, umax(abs_lo(v.y), abs_hi(v.y)));
    m = umax(m, umax(abs_lo(v.z), abs_hi(v.z)));
    m = umax(m, umax(abs_lo(v.w), abs_hi(v.w)));
    return m;
}

// Running per-column maximum of |x| over rows, two binary16 columns per
// 32-bit word (packed 16-bit integer max on the magnitude bit patterns, which
// order like the magnitudes); a column is an outlier iff its maximum is above
// the threshold, so the flags are derived once from the maxima.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned pk_max_abs(unsigned m, unsigned v)
{
    const u16x2 a = __builtin_bit_cast(u16x2, m), b = __builtin_bit_cast(u16x2, v & 0x7fff7fffu);
    return __builtin_bit_cast(unsigned, __builtin_elementwise_max(a, b));
}

__device__ __forceinline__ uint4 colmax8(uint4 m, uint4 v)
{
    return make_uint4(pk_max_abs(m.x, v.x), pk_max_abs(m.y, v.y), pk_max_abs(m.z, v.z),
                      pk_max_abs(m.w, v.w));
}

// Bit i: column i of the chunk has a magnitude above the threshold.
__device__ __forceinline__ unsigned flags8(uint4 m, unsigned thr_bits)
{
    const unsigned w[4] = {m.x, m.y, m.z, m.w};
    unsigned fl = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        fl |= (abs_lo(w[i]) > thr_bits ? 1u : 0u) << (2 * i);
        fl |= (abs_hi(w[i]) > thr_bits ? 1u : 0u) << (2 * i + 1);
    }
    return fl;
}

__device__ __forceinline__ uint16_t half_at(uint4 v, int i)
{
    unsigned w = i < 2 ? v.x : i < 4 ? v.y : i < 6 ? v.z : v.w;
    return (uint16_t)((i & 1) ? (w >> 16) : (w & 0xffffu));
}

// 1.5 * 2^23: for |y| <= 2^22, y + kRoundMagic lands in [2^23, 2^24), where
// the fp32 spacing is 1, so the addition rounds y to an integer (ties to even,
// kRoundMagic being even) held in the low mantissa bits:
// bits(y + kRoundMagic) = bits(kRoundMagic) + rint(y), and its low byte is
// rint(y) as an int8 in two's complement.
constexpr float kRoundMagic = 12582912.0f;

// The 8 integers held as kRoundMagic + q in s[] (|q| <= 127), as int8 bytes.
__device__ __forceinline__ uint2 pack_low_bytes(const float (&s)[8])
{
    unsigned b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        b[i] = __builtin_bit_cast(unsigned, s[i]);
    // low bytes: perm selector 0..3 picks a byte of the second operand, 4..7
    // of the first, 0x0c gives 0
    const unsigned lo0 = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);
    const unsigned hi0 = __builtin_amdgcn_perm(b[3], b[2], 0x04000c0cu);
    const unsigned lo1 = __builtin_amdgcn_perm(b[5], b[4], 0x0c0c0400u);
    const unsigned hi1 = __builtin_amdgcn_perm(b[7], b[6], 0x04000c0cu);
    return make_uint2(lo0 | hi0, lo1 | hi1);
}

__device__ __forceinline__ uint2 quant8(uint4 v, float amax, float r)
{
    // r = 127/amax (0 when amax = 0, and then every value here is 0); |x| <=
    // amax for every value.  The reciprocal route settles nearly every chunk:
    // r is one correctly rounded division, so y = x*r is within 2^-22 |z| <
    // 2^-16 of the exact quotient z = 127x/amax (two roundings of relative
    // size 2^-24, |z| <= 127), and rint(y) is the rounding of z unless y lies
    // within 2^-15 of a half-integer (y - rint(y) is exact).  The largest
    // |y - rint(y)| of the chunk tells; at or above 0.5 - 2^-15 the chunk is
    // redone with correctly rounded divisions, which such values need rarely.
    float s[8];
    float dmax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float y = h2f(half_at(v, i)) * r;
        s[i] = y + kRoundMagic;
        dmax = __builtin_fmaxf(dmax, __builtin_fabsf(y - (s[i] - kRoundMagic)));
    }
    if (!(dmax < 0.499969482421875f)) {   // 0.5 - 2^-15
#pragma unroll
        for (int i = 0; i < 8; ++i)
            s[i] = (float)quant127(h2f(half_at(v, i)), amax) + kRoundMagic;
    }
    return pack_low_bytes(s);
}

// FP8 variant: codes of 8 values scaled by sc = 2^e (the product is exact:
// a power of two, and |x * 2^e| is at most the format's largest finite
// value), each rounded to the nearest value of the format with ties to even
// by v_cvt_pk_bf8_f32 (E5M2) or v_cvt_pk_fp8_f32 (E4M3), two per
// instruction, into the low or high half of a dword.
template <int kFmt, bool kHi>
__device__ __forceinline__ int cvt_pk_f8(float a, float b, int old)
{
    if constexpr (kFmt == kF8E4M3)
        return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, kHi);
    else
        return __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, kHi);
}

template <int kFmt>
__device__ __forceinline__ uint2 quant8_f8(uint4 v, float sc)
{
    unsigned w[2];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        int x = 0;
        x = cvt_pk_f8<kFmt, false>(h2f(half_at(v, 4 * d)) * sc, h2f(half_at(v, 4 * d + 1)) * sc,
                                   x);
        x = cvt_pk_f8<kFmt, true>(h2f(half_at(v, 4 * d + 2)) * sc,
                                  h2f(half_at(v, 4 * d + 3)) * sc, x);
        w[d] = (unsigned)x;
    }
    return make_uint2(w[0], w[1]);
}

// The row quantization of an absmax-type kernel: int8 codes from (amax, r =
// 127/amax), or (kF8, a format) FP8 codes from sc = 2^e.
template <int kF8>
__device__ __forceinline__ uint2 quant8_mode(uint4 v, float amax, float r, float sc)
{
    if constexpr (kF8 != kF8None)
        return quant8_f8<kF8>(v, sc);
    else
        return quant8(v, amax, r);
}

// v with the halves whose flag bit is set replaced by +0.
__device__ __forceinline__ uint4 drop_flagged(uint4 v, unsigned fl)
{
    unsigned k[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        k[i] = (((fl >> (2 * i)) & 1u) ? 0u : 0x0000ffffu) |
               (((fl >> (2 * i + 1)) & 1u) ? 0u : 0xffff0000u);
    return make_uint4(v.x & k[0], v.y & k[1], v.z & k[2], v.w & k[3]);
}

// ---------------------------------------------------------------------------
// Weight quantization: one wavefront per output column n (row n of W_t).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_quantize_weight(const uint16_t *__restrict__ W_t,
                                                            int64_t K, int64_t N,
                                                            int8_t *__restrict__ CB,
                                                            float *__restrict__ SCB)
{
    const int lane = threadIdx.x % kWave;
    const int64_t n = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    if (n >= N)
        return;
    const uint4 *row = reinterpret_cast<const uint4 *>(W_t + n * K);
    const int64_t nchunk = K / 8;
    unsigned m = 0;
    for (int64_t c = lane; c < nchunk; c += kWave)
        m = umax(m, chunk_absmax(row[c]));
    m = wave_max_u32(m);
    const float amax = h2f((uint16_t)m);
    uint2 *dst = reinterpret_cast<uint2 *>(CB + n * K);
    if (amax > 0.0f) {
        const float r = 127.0f / amax;
        for (int64_t c = lane; c < nchunk; c += kWave)
            dst[c] = quant8(row[c], amax, r);
    } else {
        for (int64_t c = lane; c < nchunk; c += kWave)
            dst[c] = make_uint2(0u, 0u);
    }
    if (lane == 0)
        SCB[n] = amax;
}

// FP8 variant: one wavefront per output column, the power-of-two scale of
// the row's absmax, codes of format kFmt, and the stored scale 2^-e.
template <int kFmt>
__global__ __launch_bounds__(kBlock) void k_quantize_weight_f8(const uint16_t *__restrict__ W_t,
                                                               int64_t K, int64_t N,
                                                               uint8_t *__restrict__ CB8,
                                                               float *__restrict__ SC8)
{
    const int lane = threadIdx.x % kWave;
    const int64_t n = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    if (n >= N)
        return;
    const uint4 *row = reinterpret_cast<const uint4 *>(W_t + n * K);
    const int64_t nchunk = K / 8;
    unsigned m = 0;
    for (int64_t c = lane; c < nchunk; c += kWave)
        m = umax(m, chunk_absmax(row[c]));
    m = wave_max_u32(m);
    const int e = f8_scale_exp<kFmt>(h2f((uint16_t)m));
    const float sc = __builtin_ldexpf(1.0f, e);
    uint2 *dst = reinterpret_cast<uint2 *>(CB8 + n * K);
    for (int64_t c = lane; c < nchunk; c += kWave)
        dst[c] = quant8_f8<kFmt>(row[c], sc);
    if (lane == 0)
        SC8[n] = __builtin_ldexpf(1.0f, -e);
}

// ---------------------------------------------------------------------------
// Outlier-column detection in one launch, without atomics or a clearing
// pass.  A block takes one 64-column slice (a 128-byte line of every row: 8
// lanes per row, a lane owns one 8-column chunk) over one of nr row ranges;
// each lane keeps the running maxima of |x| of its chunk over every 128th
// row of the range (8 rows' loads in flight), and the flags "maximum above
// the threshold" are ORed over the block into the 8 chunk bytes of the
// slice in the range's flag set (parts + r * pitch).  The consumers OR the nr
// sets (nr > 1 only when K is narrow: more blocks to fill the chip).  The
// comparison |x| > threshold is done on binary16 bit patterns against the
// largest binary16 value not above the threshold (computed on the host),
// which is the same test as comparing the exact values.
// ---------------------------------------------------------------------------
constexpr int kDetectThreads = 1024;
constexpr int kDetectRowsPerPass = kDetectThreads / 8;   // 8 lanes (one line) per row

__global__ __launch_bounds__(kDetectThreads) void k_detect(const uint16_t *__restrict__ X,
                                                           int64_t T, int64_t K, int nr,
                                                           int pitch, unsigned thr_bits,
                                                           uint8_t *__restrict__ parts)
{
    __shared__ uint2 s_or[kDetectThreads / kWave];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int64_t nslice = K / 64;
    const int64_t slice = blockIdx.x % nslice;
    const int r = (int)(blockIdx.x / nslice);
    const int64_t rows = (T + nr - 1) / nr;
    const int64_t t_begin = r * rows, t_end = t_begin + rows < T ? t_begin + rows : T;
    const uint16_t *col = X + slice * 64 + 8 * (tid % 8);
    constexpr int kRowsInFlight = 8;
    uint4 cm = make_uint4(0u, 0u, 0u, 0u);
    for (int64_t t0 = t_begin + tid / 8; t0 < t_end; t0 += kRowsInFlight * kDetectRowsPerPass) {
        uint4 v[kRowsInFlight];
        // a row past the range re-reads row t0, which leaves the maximum as
        // it is; the loads are unconditional, so all of them are in flight
        // at once (a load under a condition is waited for inside it)
#pragma unroll
        for (int u = 0; u < kRowsInFlight; ++u) {
            const int64_t t = t0 + (int64_t)u * kDetectRowsPerPass;
            v[u] = *reinterpret_cast<const uint4 *>(col + (t < t_end ? t : t0) * K);
        }
#pragma unroll
        for (int u = 0; u < kRowsInFlight; ++u)
            cm = colmax8(cm, v[u]);
    }
    unsigned bits = flags8(cm, thr_bits);
    // OR over the lanes of one chunk (equal lane % 8) in the wavefront; chunk
    // c's byte then sits in lane c, and is shifted into place
    bits |= __shfl_xor(bits, 8, kWave);
    bits |= __shfl_xor(bits, 16, kWave);
    bits |= __shfl_xor(bits, 32, kWave);
    const int c = lane & 7;
    unsigned lo = c < 4 ? bits << (8 * c) : 0u, hi = c < 4 ? 0u : bits << (8 * (c - 4));
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
        lo |= __shfl_xor(lo, off, kWave);
        hi |= __shfl_xor(hi, off, kWave);
    }
    if (lane == 0)
        s_or[wave] = make_uint2(lo, hi);
    __syncthreads();
    if (tid == 0) {
        uint2 o = make_uint2(0u, 0u);
#pragma unroll
        for (int w = 0; w < kDetectThreads / kWave; ++w) {
            o.x |= s_or[w].x;
            o.y |= s_or[w].y;
        }
        *reinterpret_cast<uint2 *>(parts + (int64_t)r * pitch + slice * 8) = o;
    }
}

// ---------------------------------------------------------------------------
// The outlier set from the detection flags, derived by every block of the
// row-quantization launch itself (no compaction launch): a block copies the
// K/8 flag bytes (from L2) into LDS and reduces them to n; the positions of
// the outlier columns follow from a block scan of the flags' population
// counts in column order.  Every block computes the same values; block 0 also
// writes the outlier list and the summary for the kernels after it.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int wave_sum(int v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    return v;
}

// Sum over the block's kBlock threads; s_red: kWavesPerBlock ints of LDS not
// in use by another reduction that may still be read.
__device__ __forceinline__ int block_sum(int v, int *s_red)
{
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    v = wave_sum(v);
    if (lane == 0)
        s_red[wave] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w)
        t += s_red[w];
    return t;
}

// Exclusive prefix sum in thread order over the block; s_red as block_sum.
__device__ __forceinline__ int block_excl_scan(int v, int *s_red)
{
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    int inc = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(inc, off, kWave);
        if (lane >= off)
            inc += o;
    }
    if (lane == kWave - 1)
        s_red[wave] = inc;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w)
        before += w < wave ? s_red[w] : 0;
    return before + inc - v;
}

struct OutlierSet {
    int n;      // |O|
    int ng;     // non-empty 64-column groups (only computed when n > kOutlierPad)
    int mode;   // kOutFew / kOutCompact / kOutDense
    int kc;     // kept-column mode's int8 width (0: off; see kept_ld)
};

// The GEMM path's way of forming the outlier product (see internal.h):
// compact while the padded outlier rows are short and not much shorter than
// the groups that hold them would be.
__device__ __forceinline__ int outlier_mode(int n, int ng)
{
    if (n <= kOutlierPad)
        return kOutFew;
    const int64_t ld = outlier_ld(n);
    return (ld > kCompactMaxLd || (int64_t)ng * 64 <= ld + ld / 4) ? kOutDense : kOutCompact;
}

// All threads: s_fl[c] = the outlier flags of chunk c (bit i: column 8c+i),
// for every chunk, the OR of the detection's flag sets (16 chunks per load);
// returns the block-uniform summary.  s_red: 2 * kWavesPerBlock ints.  Ends
// with the flags visible to the whole block.
// between(): the caller's own loads (its rows), issued after the flag loads
// and before their use, so that the two latencies overlap (memory loads
// complete in issue order, so waiting for the flags does not wait for the
// rows).  First pass: thread i loads 16-byte pieces i / nr and
// i / nr + kBlock / nr of set i % nr (nr is a power of two, so a piece's nr
// loads sit in adjacent lanes of one wavefront and are ORed by lane
// exchanges), pieces 0 .. 2 kBlock/nr - 1; a loop takes the pieces past
// those, a thread per piece ORing the nr sets itself (at the shapes measured
// it runs only for nr = 1 and K > 65536).  The first pass's loads are
// unconditional (threads past the flags re-read piece 0 of set 0), so they
// are in flight with the caller's loads.
struct NoLoads {
    __device__ void operator()() const {}
};
template <class Between = NoLoads>
__device__ __forceinline__ OutlierSet derive_outliers(const DetectFlags &df, int nchunk,
                                                      uint8_t *s_fl, int *s_red,
                                                      Between &&between = Between{})
{
    int cnt = 0;
    constexpr int kFirst = 2;   // pieces per thread in the first pass
    {
        const int nr = df.nr, r = (int)threadIdx.x % nr;
        uint4 f[kFirst];
        int c[kFirst];
#pragma unroll
        for (int k = 0; k < kFirst; ++k) {
            c[k] = 16 * ((int)threadIdx.x / nr + k * (kBlock / nr));
            const bool act = c[k] < nchunk;
            f[k] = *reinterpret_cast<const uint4 *>(df.parts +
                                                    (act ? (int64_t)r * df.pitch + c[k] : 0));
        }
        __builtin_amdgcn_sched_barrier(0);
        between();
        __builtin_amdgcn_sched_barrier(0);
        for (int off = 1; off < nr; off <<= 1) {
#pragma unroll
            for (int k = 0; k < kFirst; ++k) {
                f[k].x |= __shfl_xor(f[k].x, off, kWave);
                f[k].y |= __shfl_xor(f[k].y, off, kWave);
                f[k].z |= __shfl_xor(f[k].z, off, kWave);
                f[k].w |= __shfl_xor(f[k].w, off, kWave);
            }
        }
#pragma unroll
        for (int k = 0; k < kFirst; ++k) {
            if (c[k] < nchunk && r == 0) {
                if (c[k] + 16 > nchunk) {   // K % 64 == 0: an 8-byte tail
                    f[k].z = 0u;
                    f[k].w = 0u;
                    *reinterpret_cast<uint2 *>(s_fl + c[k]) = make_uint2(f[k].x, f[k].y);
                } else {
                    *reinterpret_cast<uint4 *>(s_fl + c[k]) = f[k];
                }
                cnt += __builtin_popcount(f[k].x) + __builtin_popcount(f[k].y) +
                       __builtin_popcount(f[k].z) + __builtin_popcount(f[k].w);
            }
        }
    }
    // K % 64 == 0: nchunk is a multiple of 8; whole 16-byte pieces, then a tail
    // (the pitch is a multiple of 16)
    for (int c = 16 * ((int)threadIdx.x + kFirst * kBlock / df.nr); c < nchunk; c += 16 * kBlock) {
        const uint8_t *p = df.parts + c;
        if (c + 16 <= nchunk) {
            uint4 f = *reinterpret_cast<const uint4 *>(p);
            for (int r = 1; r < df.nr; ++r) {
                const uint4 g = *reinterpret_cast<const uint4 *>(p + (int64_t)r * df.pitch);
                f = make_uint4(f.x | g.x, f.y | g.y, f.z | g.z, f.w | g.w);
            }
            *reinterpret_cast<uint4 *>(s_fl + c) = f;
            cnt += __builtin_popcount(f.x) + __builtin_popcount(f.y) + __builtin_popcount(f.z) +
                   __builtin_popcount(f.w);
        } else {
            uint2 f = *reinterpret_cast<const uint2 *>(p);
            for (int r = 1; r < df.nr; ++r) {
                const uint2 g = *reinterpret_cast<const uint2 *>(p + (int64_t)r * df.pitch);
                f = make_uint2(f.x | g.x, f.y | g.y);
            }
            *reinterpret_cast<uint2 *>(s_fl + c) = f;
            cnt += __builtin_popcount(f.x) + __builtin_popcount(f.y);
        }
    }
    OutlierSet o;
    o.n = block_sum(cnt, s_red);   // its barrier publishes s_fl
    o.ng = 0;
    if (o.n > kOutlierPad) {
        int g = 0;
        for (int q = threadIdx.x; q < nchunk / 8; q += kBlock)
            g += *reinterpret_cast<const uint2 *>(s_fl + 8 * q) != make_uint2(0u, 0u) ? 1 : 0;
        o.ng = block_sum(g, s_red + kWavesPerBlock);
    }
    o.mode = outlier_mode(o.n, o.ng);
    o.kc = 0;   // the row kernels that support the kept-column mode set it
    return o;
}

// All threads: from the flags, s_pre8[q] = the number of outlier columns
// before 64-column group q (chunks 8q .. 8q+7; when s_pre8 is non-null) and
// O[j] = the j-th outlier column for j < cap (when O is non-null; global
// memory or LDS).  Each thread walks a contiguous run of chunks.  s_red:
// kWavesPerBlock ints.
__device__ __forceinline__ void outlier_positions(const uint8_t *s_fl, int nchunk, int *s_pre8,
                                                  int32_t *O, int cap, int *s_red)
{
    const int per = (nchunk + kBlock - 1) / kBlock;
    const int b0 = min((int)threadIdx.x * per, nchunk), b1 = min(b0 + per, nchunk);
    int cnt = 0;
    for (int b = b0; b < b1; ++b)
        cnt += __builtin_popcount(s_fl[b]);
    int j = block_excl_scan(cnt, s_red);
    for (int b = b0; b < b1; ++b) {
        const unsigned m = s_fl[b];
        if (s_pre8 && (b & 7) == 0)
            s_pre8[b >> 3] = j;
        if (O) {
            for (int i = 0; i < 8; ++i)
                if ((m >> i) & 1u) {
                    if (j < cap)
                        O[j] = 8 * b + i;
                    ++j;
                }
        } else {
            j += __builtin_popcount(m);
        }
    }
}

// The position of chunk c's first outlier column in the compact row: the
// group's prefix plus the flags of the group's chunks before c.
__device__ __forceinline__ int chunk_pos(const uint8_t *s_fl, const int *s_pre8, int c)
{
    const int q = c >> 3;
    const unsigned long long g = *reinterpret_cast<const unsigned long long *>(s_fl + 8 * q);
    const unsigned long long below = (c & 7) ? (1ull << (8 * (c & 7))) - 1ull : 0ull;
    return s_pre8[q] + __popcll(g & below);
}

// Block 0's part: the summary {n, ng, mode} and (when requested, in dense
// mode) the combined flags and the ascending list of non-empty 64-column
// groups.
__device__ __forceinline__ void write_outlier_info(const uint8_t *s_fl, int nchunk,
                                                   const OutlierSet &os, const OutlierInfoOut &io,
                                                   int *s_red)
{
    const int tid = threadIdx.x;
    if (tid == 0) {
        io.info[0] = os.n;
        if (io.groups) {
            io.info[1] = os.ng;
            io.info[2] = os.mode;
            io.info[3] = os.kc;
        }
    }
    if (io.mask && os.mode == kOutDense) {
        // the OR of the flag sets, for the GEMM kernel's dense mode
        for (int c = 16 * tid; c < nchunk; c += 16 * kBlock) {
            if (c + 16 <= nchunk)
                *reinterpret_cast<uint4 *>(io.mask + c) = *reinterpret_cast<const uint4 *>(s_fl + c);
            else
                *reinterpret_cast<uint2 *>(io.mask + c) = *reinterpret_cast<const uint2 *>(s_fl + c);
        }
    }
    if (io.groups && os.mode == kOutDense) {
        const int ngrp = nchunk / 8;
        const int per = (ngrp + kBlock - 1) / kBlock;
        const int q0 = min(tid * per, ngrp), q1 = min(q0 + per, ngrp);
        int cnt = 0;
        for (int q = q0; q < q1; ++q)
            cnt += *reinterpret_cast<const uint2 *>(s_fl + 8 * q) != make_uint2(0u, 0u) ? 1 : 0;
        int j = block_excl_scan(cnt, s_red);
        for (int q = q0; q < q1; ++q)
            if (*reinterpret_cast<const uint2 *>(s_fl + 8 * q) != make_uint2(0u, 0u))
                io.groups[j++] = q;
    }
}

// Dynamic LDS of the row-quantization kernels: the chunk flags, then either
// the 64-column group prefix counts (a row's gathered outlier positions) or a
// gather block's outlier list (at most kCompactMaxLd entries): at most
// 16.7 + 8.3 KB at the largest K.  Launches that may take the kept-column
// mode add the list of kept columns: kept_cap(K) 16-bit entries.
__host__ __device__ __forceinline__ int64_t flags_lds_bytes(int64_t nchunk)
{
    return (nchunk + 15) / 16 * 16;
}
__host__ __device__ __forceinline__ int64_t aux_lds_bytes(int64_t nchunk)
{
    return 4 * (nchunk / 8 > kCompactMaxLd ? nchunk / 8 : kCompactMaxLd);
}
__host__ __forceinline__ size_t rowquant_lds_bytes(int64_t K, bool kept = false)
{
    const int64_t nchunk = K / 8;
    return (size_t)(flags_lds_bytes(nchunk) + aux_lds_bytes(nchunk) + (kept ? 2 * kept_cap(K) : 0));
}

// What a row-quantization launch is for: the public activation quantizer (no
// gathered outlier operands), the weight-streaming path (x_out for every
// outlier count) or the GEMM path (x_out unless kOutDense; nothing at all
// for a row when every column is an outlier).
enum { kForAct = 0, kForDecode = 1, kForGemm = 2 };

// ---------------------------------------------------------------------------
// Row quantization: one 256-thread block per row t (so that even a handful of
// rows keeps many lanes busy).  The block first derives the outlier set (see
// derive_outliers), then reads its row once into registers (NC 16-byte
// chunks per thread; NC = 0 re-reads it from cache for very long rows),
// reduces its absmax over the non-outlier columns with shuffles and LDS,
// packs the int8 row with outlier columns as 0, and gathers the outlier
// values into the compact fp16 row x_out[t, .] (row stride outlier_ld(n),
// zero-padded): the outlier columns of chunk c start at the chunk's prefix
// count.  Chunks without outlier columns (nearly all of them) take a
// branch-free path.
// ---------------------------------------------------------------------------
// The 8 values of a chunk whose columns are all outliers: they sit at
// consecutive positions p0 .. p0+7 of the compact row.
__device__ __forceinline__ void copy8(uint16_t *__restrict__ dst, uint4 v)
{
    if ((reinterpret_cast<uintptr_t>(dst) & 15u) == 0u) {
        *reinterpret_cast<uint4 *>(dst) = v;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            dst[i] = half_at(v, i);
    }
}

// The outlier values of one chunk (flags fl != 0) into the compact row xrow,
// from position pre on in column order.
__device__ __forceinline__ void scatter_outliers(uint4 v, unsigned fl, int pre,
                                                 uint16_t *__restrict__ xrow)
{
    if (fl == 0xffu) {
        copy8(xrow + pre, v);
        return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if ((fl >> i) & 1u)
            xrow[pre + __builtin_popcount(fl & ((1u << i) - 1u))] = half_at(v, i);
}

// One chunk of a row: outlier columns (flags fl) are 0 in the int8 row and go
// to the compact row xrow (null: not gathered) from position pre on; the
// others are quantized (r = 127/amax, or 0 when amax = 0).
template <int kF8 = kF8None>
__device__ __forceinline__ uint2 quant_chunk(uint4 v, unsigned fl, float amax, float r, int pre,
                                            uint16_t *__restrict__ xrow, float sc = 0.0f)
{
    if (fl) {
        if (xrow)
            scatter_outliers(v, fl, pre, xrow);
        v = drop_flagged(v, fl);
    }
    return quant8_mode<kF8>(v, amax, r, sc);
}

__device__ __forceinline__ unsigned chunk_absmax_masked(uint4 v, unsigned fl)
{
    return chunk_absmax(fl ? drop_flagged(v, fl) : v);
}

// Destination of the 8 int8 values k = 8c .. 8c+7 of row t.  Row-major
// [T, K], or (decode path, T <= 16) the MFMA fragment order
// [K/64][4][16][16]: 64-byte k-step, 16-byte chunk, row, byte.
__device__ __forceinline__ uint2 *xq_chunk(int8_t *Xq, int64_t t, int64_t K, int64_t c,
                                           bool packed)
{
    const int64_t off =
        packed ? (c / 8) * 1024 + ((c % 8) / 2) * 256 + t * 16 + (c % 2) * 8 : t * K + 8 * c;
    return reinterpret_cast<uint2 *>(Xq + off);
}

// The GEMM path's outlier weight operand, built by the blocks gb = 0 .. nb-1
// past the row blocks of a row-quantization launch, which share the N weight
// rows (see GatherArgs).  s_O holds the first min(n, kCompactMaxLd) outlier
// columns (LDS).  kOutFew: a lane takes one 8-column group of one row, 16
// rows per wavefront, and dequantizes its at most 8 values.  kOutCompact: a
// wavefront per row, a lane gathers the codes of 8 consecutive outlier
// columns (one 8-byte load when they are 8 aligned consecutive columns) and
// stores them at once; past n the row holds zeros.  kOutDense: nothing.
// kMode 0: absmax.  1, zero-point variant: SCB holds each row's nd, ZP its
// zp, and the kOutFew values are fp16((cb + zp) / nd).  2 and 3, FP8
// variant: the bytes are E5M2 (2) or E4M3 (3) codes and SCB the scales 2^-e.
constexpr int kModeAbsmax = 0, kModeZp = 1, kModeF8 = 2, kModeF8E4 = 3;
// The FP8 format of a mode (kF8None for the int8 modes), and back.
constexpr int mode_f8(int mode)
{
    return mode == kModeF8 ? kF8E5M2 : mode == kModeF8E4 ? kF8E4M3 : kF8None;
}
constexpr int f8_mode(int fmt)
{
    return fmt == kF8E5M2 ? kModeF8 : fmt == kF8E4M3 ? kModeF8E4 : kModeAbsmax;
}
template <int kMode>
__device__ __forceinline__ uint16_t dequant_row(int cb, float sc, int zp)
{
    if constexpr (mode_f8(kMode) != kF8None)
        return dequant_w_f8<mode_f8(kMode)>((unsigned)cb & 0xffu, sc);
    else if constexpr (kMode == kModeZp)
        return dequant_w_zp(cb, zp, sc);
    else
        return dequant_w(cb, sc);
}

template <int kMode = kModeAbsmax>
__device__ __forceinline__ void gather_w_out(int64_t gb, int64_t nb, int64_t K,
                                             const OutlierSet &os, const int *s_O,
                                             const int8_t *__restrict__ CB,
                                             const float *__restrict__ SCB, int64_t N,
                                             void *__restrict__ w_out,
                                             const int32_t *__restrict__ ZP = nullptr)
{
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int n = os.n;
    if (os.mode == kOutFew) {
        uint16_t *wo = static_cast<uint16_t *>(w_out);
        constexpr int kGroups = kOutlierPad / 8, kRowsPerWave = kWave / kGroups;
        const int g = lane % kGroups;
        int o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int j = 8 * g + e;
            o[e] = j < n ? s_O[j] : 0;
        }
        for (int64_t r = (gb * kWavesPerBlock + wave) * kRowsPerWave + lane / kGroups; r < N;
             r += nb * kWavesPerBlock * kRowsPerWave) {
            const float sc = SCB[r];
            const int zr = kMode == kModeZp ? ZP[r] : 0;
            const int8_t *cbr = CB + r * K;
            unsigned h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const unsigned v = dequant_row<kMode>(cbr[o[e]], sc, zr);
                h[e] = 8 * g + e < n ? v : 0u;
            }
            *reinterpret_cast<uint4 *>(wo + r * kOutlierPad + 8 * g) =
                make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                           h[6] | (h[7] << 16));
        }
        return;
    }
    if (os.mode != kOutCompact)
        return;
    int8_t *wo = static_cast<int8_t *>(w_out);
    const int64_t ldo = outlier_ld(n);   // <= kCompactMaxLd
    for (int64_t r = gb * kWavesPerBlock + wave; r < N; r += nb * kWavesPerBlock) {
        const int8_t *cbr = CB + r * K;
        for (int j0 = 8 * lane; j0 < ldo; j0 += 8 * kWave) {
            unsigned b[8];
            if (j0 + 8 <= n && s_O[j0 + 7] == s_O[j0] + 7 && (s_O[j0] & 7) == 0) {
                const uint2 raw = *reinterpret_cast<const uint2 *>(cbr + s_O[j0]);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    b[e] = ((e < 4 ? raw.x : raw.y) >> (8 * (e & 3))) & 0xffu;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    b[e] = j0 + e < n ? (unsigned)(uint8_t)cbr[s_O[j0 + e]] : 0u;
            }
            *reinterpret_cast<uint2 *>(wo + r * ldo + j0) =
                make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                           b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
        }
    }
}

// Kept-column mode: the kept (non-outlier) columns of the row set, in column
// order, into the LDS list s_list (16-bit column indices; K <= kKeptMaxK):
// chunk c's kept columns start at position 8c - (outlier columns before c),
// and a lane walks the clear bits of each of its chunks' flags.  The list
// serves the block's activation row and its weight rows alike, so each of
// them is compacted by gathering 8 listed columns per thread (a per-byte
// placement of every kept code cost ~2200 instructions per wavefront at
// 4096 x 16384).  The m kept columns are followed by column 0 up to kc, so
// that the gathers below load unconditionally (a load under a condition is
// waited for inside it) and zero those entries after the load.  s_pre8: the
// 64-column group prefix counts.
__device__ __forceinline__ void kept_list(const uint8_t *s_fl, const int *s_pre8, int nchunk,
                                          int m, int kc, uint16_t *s_list)
{
    for (int c = threadIdx.x; c < nchunk; c += kBlock) {
        unsigned km = ~(unsigned)s_fl[c] & 0xffu;
        if (km == 0u)
            continue;
        int p = 8 * c - chunk_pos(s_fl, s_pre8, c);
        while (km) {
            s_list[p++] = (uint16_t)(8 * c + __builtin_ctz(km));
            km &= km - 1u;
        }
    }
    for (int j = m + (int)threadIdx.x; j < kc; j += kBlock)
        s_list[j] = 0;
}

// 8 consecutive entries j0 .. j0+7 of a compacted row: the listed columns of
// row src (fp16 values or int8 codes), 0 past the m kept columns.
__device__ __forceinline__ uint4 kept_gather_h(const uint16_t *__restrict__ src,
                                               const uint16_t *s_list, int j0, int m)
{
    unsigned h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        h[e] = src[s_list[j0 + e]];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        h[e] = j0 + e < m ? h[e] : 0u;
    return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                      h[6] | (h[7] << 16));
}

__device__ __forceinline__ uint2 kept_gather_b(const int8_t *__restrict__ src,
                                               const uint16_t *s_list, int j0, int m)
{
    const uint8_t *u = reinterpret_cast<const uint8_t *>(src);
    unsigned b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        b[e] = u[s_list[j0 + e]];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        b[e] = j0 + e < m ? b[e] : 0u;
    return make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                      b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
}

// The gather blocks' part of a row-quantization launch: the first outlier
// columns into LDS, then the weight operand.  s_O: kCompactMaxLd ints.
template <int kMode>
__device__ __forceinline__ void gather_block(int64_t gb, int64_t nb, int64_t K, int nchunk,
                                             const OutlierSet &os, const uint8_t *s_fl, int *s_O,
                                             int *s_red, const int8_t *CB, const float *SCB,
                                             int64_t N, void *w_out, const int32_t *ZP = nullptr)
{
    if (os.mode == kOutDense || os.n == 0)
        return;
    outlier_positions(s_fl, nchunk, nullptr, s_O, (int)kCompactMaxLd, s_red);
    __syncthreads();
    gather_w_out<kMode>(gb, nb, K, os, s_O, CB, SCB, N, w_out, ZP);
}

// The start of every row-quantization kernel: the outlier set from the
// detection flags; block 0 writes the summary (and the outlier list, except on
// the GEMM path, whose kernels do not read it); then, when the row's
// outlier values are gathered, the chunk prefix counts into s_pre.  Returns
// whether this block has a row to quantize (false on the GEMM path when
// every column is an outlier: the int8 part is then zero and unused).
// s_red: 4 * kWavesPerBlock ints.
__device__ __forceinline__ bool row_prologue(const OutlierSet &os, const uint8_t *s_fl,
                                             int nchunk, int64_t K, int use, bool gather_x,
                                             int *s_pre8, int32_t *O, const OutlierInfoOut &io,
                                             int *s_red, bool first)
{
    if (use == kForGemm && os.n == K) {
        if (first)
            write_outlier_info(s_fl, nchunk, os, io, s_red + 3 * kWavesPerBlock);
        return false;
    }
    const bool list = first && use != kForGemm;
    if (gather_x || list)
        outlier_positions(s_fl, nchunk, gather_x ? s_pre8 : nullptr, list ? O : nullptr, (int)K,
                          s_red + 2 * kWavesPerBlock);
    if (first)
        write_outlier_info(s_fl, nchunk, os, io, s_red + 3 * kWavesPerBlock);
    __syncthreads();   // s_pre8 complete
    return true;
}

// Whether a row-quantization launch gathers the rows' outlier values.
__device__ __forceinline__ bool gathers_x(const uint16_t *x_out, int use, const OutlierSet &os)
{
    return x_out && (use == kForDecode || (use == kForGemm && os.mode != kOutDense));
}

template <int NC, int kF8 = kF8None>
__global__ __launch_bounds__(kBlock) void k_rowquant(const uint16_t *__restrict__ X, int64_t T,
                                                     int64_t K, const DetectFlags df,
                                                     int use, int32_t *__restrict__ O,
                                                     OutlierInfoOut io, int8_t *__restrict__ Xq,
                                                     float *__restrict__ a,
                                                     uint16_t *__restrict__ x_out,
                                                     const int8_t *__restrict__ CB,
                                                     const float *__restrict__ SCB, int64_t N,
                                                     void *__restrict__ w_out, bool packed,
                                                     int8_t *__restrict__ cb_kept, bool early)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t s_dyn[];
    __shared__ unsigned s_max[kWavesPerBlock];
    __shared__ int s_red[4 * kWavesPerBlock];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int nchunk = (int)(K / 8);
    uint8_t *s_fl = s_dyn;
    int *s_aux = reinterpret_cast<int *>(s_dyn + flags_lds_bytes(nchunk));
    // kept-column mode (cb_kept non-null only for launches with its LDS
    // region): the list of kept columns
    uint16_t *s_list =
        reinterpret_cast<uint16_t *>(s_dyn + flags_lds_bytes(nchunk) + aux_lds_bytes(nchunk));
    // the gather blocks come first
    const int64_t gb = (int64_t)gridDim.x - T;
    if ((int64_t)blockIdx.x < gb) {
        OutlierSet os = derive_outliers(df, nchunk, s_fl, s_red);
        gather_block<f8_mode(kF8)>(blockIdx.x, gb, K, nchunk, os, s_fl, s_aux,
                                   s_red + 2 * kWavesPerBlock, CB, SCB, N, w_out);
        return;
    }
    const int64_t t = (int64_t)blockIdx.x - gb;
    const uint4 *xr = reinterpret_cast<const uint4 *>(X + t * K);
    // Row t's loads go out before the prologue's scans and barriers, so that
    // their latency runs under them.  With `early` (the host's guess that the
    // row has an int8 part: threshold > 0) they go out with the flag loads,
    // unconditionally (chunks past the row re-read chunk 0, zeroed after), so
    // that the flags' wait leaves them in flight; otherwise after the flags,
    // and not at all when every column is an outlier on the GEMM path.
    uint4 v[NC > 0 ? NC : 1];
    auto load_row = [&]() {
        if constexpr (NC > 0) {
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                const int c = tid + i * kBlock;
                v[i] = xr[c < nchunk ? c : 0];
            }
        }
    };
    OutlierSet os = early ? derive_outliers(df, nchunk, s_fl, s_red, load_row)
                          : derive_outliers(df, nchunk, s_fl, s_red);
    if (!early && !(use == kForGemm && os.n == K))
        load_row();
    if constexpr (NC > 0) {
#pragma unroll
        for (int i = 0; i < NC; ++i)
            if (tid + i * kBlock >= nchunk)
                v[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    if (cb_kept)
        os.kc = (int)kept_ld(K, os.n);
    const bool gx = gathers_x(x_out, use, os);
    const bool kept = os.kc > 0;
    if (!row_prologue(os, s_fl, nchunk, K, use, gx || kept, s_aux, O, io, s_red, t == 0))
        return;
    if (kept)   // the list is complete at the absmax's barrier
        kept_list(s_fl, s_aux, nchunk, (int)K - os.n, os.kc, s_list);
    const int nout = os.n;
    const int64_t ldo = outlier_ld(nout);
    uint16_t *xrow = gx ? x_out + t * ldo : nullptr;
    unsigned m = 0;
    unsigned fl[NC > 0 ? NC : 1];
    if constexpr (NC > 0) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int c = tid + i * kBlock;
            fl[i] = c < nchunk ? s_fl[c] : 0u;
        }
#pragma unroll
        for (int i = 0; i < NC; ++i)
            m = umax(m, chunk_absmax_masked(v[i], fl[i]));
    } else {
        for (int c = tid; c < nchunk; c += kBlock)
            m = umax(m, chunk_absmax_masked(xr[c], s_fl[c]));
    }
    m = wave_max_u32(m);
    if (lane == 0)
        s_max[wave] = m;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w)
        m = umax(m, s_max[w]);
    const float amax = h2f((uint16_t)m);
    const float r = kF8 ? 0.0f : amax > 0.0f ? 127.0f / amax : 0.0f;
    const int e8 = kF8 ? f8_scale_exp<kF8>(amax) : 0;
    const float sc = kF8 ? __builtin_ldexpf(1.0f, e8) : 0.0f;
    if (kept) {
        // the row's outlier values (compact mode with few kept columns, small K)
        if (xrow) {
            if constexpr (NC > 0) {
#pragma unroll
                for (int i = 0; i < NC; ++i) {
                    const int c = tid + i * kBlock;
                    if (c < nchunk && fl[i])
                        scatter_outliers(v[i], fl[i], chunk_pos(s_fl, s_aux, c), xrow);
                }
            } else {
                for (int c = tid; c < nchunk; c += kBlock)
                    if (s_fl[c])
                        scatter_outliers(xr[c], s_fl[c], chunk_pos(s_fl, s_aux, c), xrow);
            }
        }
        // the kept codes, zero-padded to kc, at the start of Xq's row t; then
        // the kept weight operand: row block t builds weight rows t, t + T,
        // t + 2T, ... (the row blocks share the N rows evenly, and no extra
        // blocks sit idle when the mode is not taken); both gather through
        // the list (the rows are in cache: row t was just read)
        const int mk = (int)K - nout;
        const uint16_t *xt = X + t * K;
        for (int j0 = 8 * tid; j0 < os.kc; j0 += 8 * kBlock)
            *reinterpret_cast<uint2 *>(Xq + t * K + j0) =
                quant8_mode<kF8>(kept_gather_h(xt, s_list, j0, mk), amax, r, sc);
        for (int64_t rr = t; rr < N; rr += T)
            for (int j0 = 8 * tid; j0 < os.kc; j0 += 8 * kBlock)
                *reinterpret_cast<uint2 *>(cb_kept + rr * os.kc + j0) =
                    kept_gather_b(CB + rr * K, s_list, j0, mk);
    } else {
        // the chunk's codes to Xq (and its outlier values to the compact row)
        auto put = [&](uint4 x, unsigned f, int c) {
            const int pre = (xrow && f) ? chunk_pos(s_fl, s_aux, c) : 0;
            *xq_chunk(Xq, t, K, c, packed) = quant_chunk<kF8>(x, f, amax, r, pre, xrow, sc);
        };
        if constexpr (NC > 0) {
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                const int c = tid + i * kBlock;
                if (c < nchunk)
                    put(v[i], fl[i], c);
            }
        } else {
            for (int c = tid; c < nchunk; c += kBlock)
                put(xr[c], s_fl[c], c);
        }
    }
    if (xrow) {
        for (int64_t j = nout + tid; j < ldo; j += kBlock)
            xrow[j] = 0;
    }
    if (tid == 0)
        a[t] = kF8 ? __builtin_ldexpf(1.0f, -e8) : amax;
}

// ---------------------------------------------------------------------------
// Row quantization for many short rows: one wavefront per row, four rows per
// block, the row held in registers (NC 16-byte chunks per lane, chunk
// c = lane + 64 i, so every load instruction reads 1 KB of the row).  The
// absmax is a wave reduction (no LDS, no block barrier), outlier columns are
// zeroed before the absmax and the pack, so chunks with and without outliers
// take the same arithmetic.  On the GEMM path with short outlier rows the
// block lists the outlier columns once in LDS and each wavefront copies its
// row's values from that list (a per-chunk scatter cost hundreds of
// instructions per row for a handful of values).  Extra blocks build w_out
// as k_rowquant's.
// ---------------------------------------------------------------------------
template <int NC, int kF8 = kF8None>
__global__ __launch_bounds__(kBlock) void k_rowquant_w(const uint16_t *__restrict__ X, int64_t T,
                                                       int64_t K,
                                                       const DetectFlags df,
                                                       int use, int32_t *__restrict__ O,
                                                       OutlierInfoOut io, int8_t *__restrict__ Xq,
                                                       float *__restrict__ a,
                                                       uint16_t *__restrict__ x_out,
                                                       const int8_t *__restrict__ CB,
                                                       const float *__restrict__ SCB, int64_t N,
                                                       void *__restrict__ w_out,
                                                       int64_t row_blocks)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t s_dyn[];
    __shared__ int s_red[4 * kWavesPerBlock];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int nchunk = (int)(K / 8);
    uint8_t *s_fl = s_dyn;
    int *s_aux = reinterpret_cast<int *>(s_dyn + flags_lds_bytes(nchunk));
    if ((int64_t)blockIdx.x >= row_blocks) {
        const OutlierSet os = derive_outliers(df, nchunk, s_fl, s_red);
        gather_block<f8_mode(kF8)>(blockIdx.x - row_blocks,
                                                  gridDim.x - row_blocks, K, nchunk, os, s_fl,
                                                  s_aux, s_red + 2 * kWavesPerBlock, CB, SCB, N,
                                                  w_out);
        return;
    }
    const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    // The row's loads go out with the flag loads, so that their latency runs
    // under the flags' and the prologue.  They are unconditional (a wavefront
    // past the last row re-reads row T-1, chunks past the row re-read chunk
    // 0, both unused): a load under a condition would make the flags' use
    // wait for it too.  When every column is an outlier on the GEMM path the
    // row is loaded and not used.
    const uint4 *xr = reinterpret_cast<const uint4 *>(X + (t < T ? t : T - 1) * K);
    uint4 v[NC];
    const OutlierSet os = derive_outliers(df, nchunk, s_fl, s_red, [&]() {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int c = lane + i * kWave;
            v[i] = xr[c < nchunk ? c : 0];
        }
    });
#pragma unroll
    for (int i = 0; i < NC; ++i)
        if (lane + i * kWave >= nchunk)
            v[i] = make_uint4(0u, 0u, 0u, 0u);
    const bool gx = gathers_x(x_out, use, os);
    if (!row_prologue(os, s_fl, nchunk, K, use, false, nullptr, O, io, s_red, blockIdx.x == 0))
        return;
    // The outlier columns' positions (at most kCompactMaxLd: the gathered
    // rows exist only in the modes with short outlier rows), once per block
    // into LDS; each wavefront then copies its row's outlier values to the
    // compact row with one 2-byte load per entry (the row is in cache).
    const int nout = os.n;
    if (gx && nout > 0) {
        outlier_positions(s_fl, nchunk, nullptr, s_aux, (int)kCompactMaxLd,
                          s_red + 2 * kWavesPerBlock);
        __syncthreads();
    }
    if (t >= T)
        return;
    uint2 *qr = reinterpret_cast<uint2 *>(Xq + t * K);
    const int64_t ldo = outlier_ld(nout);
    if (gx) {
        const uint16_t *xt = X + t * K;
        uint16_t *xrow = x_out + t * ldo;
        for (int64_t j = lane; j < ldo; j += kWave)
            xrow[j] = j < nout ? xt[s_aux[j]] : (uint16_t)0;
    }
    unsigned fl[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = lane + i * kWave;
        fl[i] = c < nchunk ? s_fl[c] : 0u;
    }
    unsigned m = 0;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        if (fl[i])
            v[i] = drop_flagged(v[i], fl[i]);
        m = umax(m, chunk_absmax(v[i]));
    }
    m = wave_max_u32(m);
    const float amax = h2f((uint16_t)m);
    const float r = kF8 ? 0.0f : amax > 0.0f ? 127.0f / amax : 0.0f;
    const int e8 = kF8 ? f8_scale_exp<kF8>(amax) : 0;
    const float sc = kF8 ? __builtin_ldexpf(1.0f, e8) : 0.0f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = lane + i * kWave;
        if (c < nchunk)
            qr[c] = quant8_mode<kF8>(v[i], amax, r, sc);
    }
    if (lane == 0)
        a[t] = kF8 ? __builtin_ldexpf(1.0f, -e8) : amax;
}

// ---------------------------------------------------------------------------
// Zero-point variant (the asymmetric quantizer of the LLM.int8() summary,
// kurtkim.github.io, "8-bit Data Types and Quantization"): per vector the
// range [min(min,0), max(max,0)] is mapped onto [-127, 127] by the
// normalized dynamic range nd = 254/d and the integer zero point zp, and the
// code of x is RNE(nd*x) - zp, so that code + zp is the shifted value the
// page multiplies.  Like the absmax kernels, these are HBM-bound streams.
// ---------------------------------------------------------------------------
// Signed minimum and maximum of the 8 values of a chunk folded into (mn, mx).
__device__ __forceinline__ void chunk_minmax(uint4 v, float &mn, float &mx)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float f = h2f(half_at(v, i));
        mn = __builtin_fminf(mn, f);
        mx = __builtin_fmaxf(mx, f);
    }
}

__device__ __forceinline__ void wave_minmax(float &mn, float &mx)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        mn = __builtin_fminf(mn, __shfl_xor(mn, off, kWave));
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, off, kWave));
    }
}

// RNE(254 x / d), the exact rational rounded to the nearest integer with ties
// to even, for a binary16 value x (as fp32) and d = max' - min' > 0 of its
// vector (exact in fp64), with r = 254/d correctly rounded in fp64.
// y = x*r is within 2^-52 |254 x / d| <= 2^-44 of the rational (two fp64
// roundings), while a rational that is not a tie lies at least 2^-42 from
// every half-integer: 254x/d - (k + 1/2) = (508x - (2k+1) d) / (2d), the
// numerator a nonzero multiple of 2^-24 (binary16 granularity) and d < 2^17.
// So floor(y) + (frac > 1/2) is the answer unless frac is within 2^-40 of
// 1/2; there the sign of 508x - (2k+1) d decides, computed exactly by one
// fused multiply-add (508x has 18 significant bits, (2k+1) d at most 50, and
// their difference is a multiple of 2^-24 below 2^27).
__device__ __forceinline__ int rne254(float x, double d, double r)
{
    const double xd = (double)x;
    const double y = xd * r;
    const double k = __builtin_floor(y);
    const double f = y - k;                    // exact
    int q = (int)k + (f > 0.5 ? 1 : 0);
    if (__builtin_fabs(f - 0.5) < 0x1p-40) {
        const double e = __builtin_fma(-(2.0 * k + 1.0), d, 508.0 * xd);
        q = (int)k + (e > 0.0 ? 1 : e < 0.0 ? 0 : ((int)k & 1));
    }
    return q;
}

// The fp32 value nearest to 254/d (ties to even), from r = 254/d correctly
// rounded in fp64: fp32(r) is that value unless r lies within 2^-52 r of
// the midpoint between two fp32 values (the exact quotient is within
// 2^-53 r of r and could then sit on the midpoint's other side); there the
// sign of mid*d - 254, exact in one fused multiply-add, picks the side.
__device__ __forceinline__ float nearest_f32_254_over(double d, double r)
{
    const float f = (float)r;
    const double fd = (double)f;
    if (fd == r)
        return f;
    const unsigned fb = __builtin_bit_cast(unsigned, f);
    const float g = __builtin_bit_cast(float, r > fd ? fb + 1u : fb - 1u);   // r > 0
    const double mid = 0.5 * (fd + (double)g);                              // exact
    if (__builtin_fabs(r - mid) > 0x1p-52 * r)
        return f;
    const float lo = __builtin_fminf(f, g), hi = __builtin_fmaxf(f, g);
    const double e = __builtin_fma(mid, d, -254.0);
    if (e > 0.0)
        return lo;
    if (e < 0.0)
        return hi;
    return (__builtin_bit_cast(unsigned, lo) & 1u) ? hi : lo;
}

// (nd, zp) of a vector whose range [mn, mx] (binary16 values as fp32)
// already contains 0: nd = 254/d, d = mx - mn, is kept exact for the codes
// (d exact in fp64, r = 254/d in fp64, rne254 rounds the rationals), and the
// stored nd is its nearest fp32 value; zp = RNE(254 mn / d) + 127.  d = 0
// gives nd = 0, zp = 0 (and codes 0).
struct ZpParams {
    double d, r;
    float nd;
    int zp;
};
__device__ __forceinline__ ZpParams zp_params(float mn, float mx)
{
    const double d = (double)mx - (double)mn;
    if (!(d > 0.0))
        return ZpParams{0.0, 0.0, 0.0f, 0};
    const double r = 254.0 / d;
    return ZpParams{d, r, nearest_f32_254_over(d, r), rne254(mn, d, r) + 127};
}

// Codes of 8 values, RNE(254 x / d) - zp: RNE(254 x / d) runs from
// RNE(254 mn / d) = zp - 127 to RNE(254 mn / d + 254) = zp + 127, so every
// code lies in [-127, 127].  The codes' sum is added to *sum; d = 0 gives
// codes 0.
__device__ __forceinline__ uint2 quant8_zp(uint4 v, const ZpParams &p, int &sum)
{
    float s[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int q = p.d > 0.0 ? rne254(h2f(half_at(v, i)), p.d, p.r) - p.zp : 0;
        sum += q;
        s[i] = __builtin_bit_cast(float, q);   // pack_low_bytes takes the low byte of each word
    }
    return pack_low_bytes(s);
}

// ---------------------------------------------------------------------------
// Few rows (T <= 16, the decode regime): the whole quantization in one
// launch of T blocks, block t quantizing row t.  The outlier set depends on
// every row, and at these sizes each block can afford to read all of X (at
// most 16 rows x 16384 columns): every block derives the same flags itself,
// so no detection flags, separate launches or workspace are needed.  A thread
// owns the 8-column chunks c = tid, tid + 512, ... (G of them):
//   1. it loads its chunks of every row, R rows at a time, keeps the column
//      maxima of |x| (the flags follow from them) and row t's chunks;
//   2. a block scan over the chunk flags in column order gives, per chunk,
//      the number of outlier columns before it and n (block 0 also writes
//      the ascending outlier list and n);
//   3. the absmax of row t over the other columns (wave reductions and the 8
//      wave maxima through LDS), then the packed int8 row and the row's
//      outlier values in x_out.
// The tests and the arithmetic are those of k_detect / derive_outliers /
// k_rowquant, so the results are identical bit for bit.
// ---------------------------------------------------------------------------
constexpr int kSmallThreads = 512;
constexpr int kSmallMaxChunks = 16 * kSmallThreads;   // G <= 16: K <= 65536

// kMode kModeZp, the zero-point variant (a receives nd, row_zp {zp, code
// sum}): the range instead of the absmax in step 3, codes by quant8_zp, and
// one more block reduction for the code sum.  kModeF8, the FP8 variant: the
// absmax sets the power-of-two scale, codes by quant8_f8, a receives 2^-e
// (kModeF8: E5M2 codes, kModeF8E4: E4M3).
template <int G, int kMode = kModeAbsmax>
__global__ __launch_bounds__(kSmallThreads) void k_quant_rows(
    const uint16_t *__restrict__ X, int T, int K, unsigned thr_bits, int8_t *__restrict__ Xq,
    float *__restrict__ a, int32_t *__restrict__ O, int32_t *__restrict__ n_out,
    uint16_t *__restrict__ x_out, bool packed, int2 *__restrict__ row_zp = nullptr)
{
    constexpr int R = G >= 16 ? 1 : 32 / G;   // rows per batch: R*G loads in flight
    __shared__ uint8_t s_flags[kSmallMaxChunks];
    __shared__ int s_pre[kSmallMaxChunks];
    __shared__ unsigned s_wmax[kSmallThreads / kWave];
    __shared__ float s_wmn[kMode == kModeZp ? kSmallThreads / kWave : 1];
    __shared__ int s_wave_tot[kSmallThreads / kWave];
    __shared__ int s_n;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int t = blockIdx.x;
    const int nchunk = K / 8;

    // 1. column flags over all rows; row t's chunks stay in registers
    uint4 v[G], cm[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        v[g] = make_uint4(0u, 0u, 0u, 0u);
        cm[g] = make_uint4(0u, 0u, 0u, 0u);
    }
    for (int r0 = 0; r0 < T; r0 += R) {
        uint4 w[R][G];
#pragma unroll
        for (int u = 0; u < R; ++u)
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int r = r0 + u, c = tid + g * kSmallThreads;
                w[u][g] = (r < T && c < nchunk)
                              ? *reinterpret_cast<const uint4 *>(X + (int64_t)r * K + 8 * c)
                              : make_uint4(0u, 0u, 0u, 0u);   // |0| is never above
            }
#pragma unroll
        for (int u = 0; u < R; ++u)
#pragma unroll
            for (int g = 0; g < G; ++g) {
                cm[g] = colmax8(cm[g], w[u][g]);
                if (r0 + u == t)
                    v[g] = w[u][g];
            }
    }
    unsigned fl[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int c = tid + g * kSmallThreads;
        fl[g] = flags8(cm[g], thr_bits);
        if (c < nchunk)
            s_flags[c] = (uint8_t)fl[g];
    }
    __syncthreads();

    // 2. outlier positions in column order (block scan)
    const int per = (nchunk + kSmallThreads - 1) / kSmallThreads;
    const int b0 = tid * per < nchunk ? tid * per : nchunk;
    const int b1 = b0 + per < nchunk ? b0 + per : nchunk;
    int cnt = 0;
    for (int b = b0; b < b1; ++b)
        cnt += __builtin_popcount(s_flags[b]);
    int inc = cnt;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(inc, off, kWave);
        if (lane >= off)
            inc += o;
    }
    if (lane == kWave - 1)
        s_wave_tot[wave] = inc;
    // row t's absmax (zero-point: range) over the non-outlier columns
    if constexpr (kMode == kModeZp) {
        float mn = 0.0f, mx = 0.0f;
#pragma unroll
        for (int g = 0; g < G; ++g)
            chunk_minmax(fl[g] ? drop_flagged(v[g], fl[g]) : v[g], mn, mx);
        wave_minmax(mn, mx);
        if (lane == 0) {
            s_wmn[wave] = mn;
            s_wmax[wave] = __builtin_bit_cast(unsigned, mx);
        }
    } else {
        unsigned m = 0;
#pragma unroll
        for (int g = 0; g < G; ++g)
            m = umax(m, chunk_absmax_masked(v[g], fl[g]));
        m = wave_max_u32(m);
        if (lane == 0)
            s_wmax[wave] = m;
    }
    __syncthreads();
    int j = inc - cnt;
    for (int w = 0; w < wave; ++w)
        j += s_wave_tot[w];
    for (int b = b0; b < b1; ++b) {
        const unsigned mb = s_flags[b];
        s_pre[b] = j;
        if (t == 0) {
            for (int i = 0; i < 8; ++i)
                if ((mb >> i) & 1u)
                    O[j++] = 8 * b + i;
        } else {
            j += __builtin_popcount(mb);
        }
    }
    if (tid == kSmallThreads - 1) {
        if (t == 0)
            *n_out = j;
        s_n = j;
    }
    float amax = 0.0f, r127 = 0.0f, zpf = 0.0f;
    ZpParams p{0.0, 0.0, 0.0f, 0};
    if constexpr (kMode == kModeZp) {
        float mn = 0.0f, mx = 0.0f;
#pragma unroll
        for (int w = 0; w < kSmallThreads / kWave; ++w) {
            mn = __builtin_fminf(mn, s_wmn[w]);
            mx = __builtin_fmaxf(mx, __builtin_bit_cast(float, s_wmax[w]));
        }
        p = zp_params(mn, mx);
    } else {
        unsigned amax_bits = 0;
#pragma unroll
        for (int w = 0; w < kSmallThreads / kWave; ++w)
            amax_bits = umax(amax_bits, s_wmax[w]);
        amax = h2f((uint16_t)amax_bits);
        if constexpr (mode_f8(kMode) != kF8None) {
            const int e8 = f8_scale_exp<mode_f8(kMode)>(amax);
            zpf = __builtin_ldexpf(1.0f, e8);   // the FP8 scale 2^e
            if (tid == 0)
                a[t] = __builtin_ldexpf(1.0f, -e8);
        } else {
            r127 = amax > 0.0f ? 127.0f / amax : 0.0f;
            if (tid == 0)
                a[t] = amax;
        }
    }
    __syncthreads();

    // 3. row t: int8 values and the gathered outlier values
    const int n = s_n;
    const int64_t ldo = outlier_ld(n);
    int sum = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int c = tid + g * kSmallThreads;
        if (c >= nchunk)
            continue;
        const unsigned f = fl[g];
        uint4 x = v[g];
        if (f) {
            if (x_out)
                scatter_outliers(x, f, s_pre[c], x_out + t * ldo);
            x = drop_flagged(x, f);
        }
        uint2 q;
        if constexpr (kMode == kModeZp)
            q = quant8_zp(x, p, sum);
        else if constexpr (mode_f8(kMode) != kF8None)
            q = quant8_f8<mode_f8(kMode)>(x, zpf);
        else
            q = quant8(x, amax, r127);
        *xq_chunk(Xq, t, K, c, packed) = q;
    }
    if (x_out) {
        for (int64_t idx = n + tid; idx < ldo; idx += kSmallThreads)
            x_out[t * ldo + idx] = 0;
    }
    if constexpr (kMode == kModeZp) {
        // the code sum of row t (s_wave_tot is free again: read before the
        // last barrier)
        sum = wave_sum(sum);
        if (lane == 0)
            s_wave_tot[wave] = sum;
        __syncthreads();
        if (tid == 0) {
            int total = 0;
#pragma unroll
            for (int w = 0; w < kSmallThreads / kWave; ++w)
                total += s_wave_tot[w];
            a[t] = p.nd;
            row_zp[t] = make_int2(p.zp, total);
        }
    }
}

// Zero-point weight quantization: one wavefront per row n of W_t (output
// column n of W), over all K.
__global__ __launch_bounds__(kBlock) void k_quantize_weight_zp(const uint16_t *__restrict__ W_t,
                                                               int64_t K, int64_t N,
                                                               int8_t *__restrict__ CB,
                                                               float *__restrict__ ND,
                                                               int32_t *__restrict__ ZP,
                                                               int32_t *__restrict__ RS)
{
    const int lane = threadIdx.x % kWave;
    const int64_t n = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    if (n >= N)
        return;
    const uint4 *row = reinterpret_cast<const uint4 *>(W_t + n * K);
    const int64_t nchunk = K / 8;
    float mn = 0.0f, mx = 0.0f;   // 0 joins the range
    for (int64_t c = lane; c < nchunk; c += kWave)
        chunk_minmax(row[c], mn, mx);
    wave_minmax(mn, mx);
    const ZpParams p = zp_params(mn, mx);
    uint2 *dst = reinterpret_cast<uint2 *>(CB + n * K);
    int sum = 0;
    for (int64_t c = lane; c < nchunk; c += kWave)
        dst[c] = quant8_zp(row[c], p, sum);
    sum = wave_sum(sum);
    if (lane == 0) {
        ND[n] = p.nd;
        ZP[n] = p.zp;
        RS[n] = sum;
    }
}

// Activations: one 256-thread block per row t, as k_rowquant (the row in NC
// 16-byte chunks per thread; NC = 0 re-reads it for very long rows).  The
// range runs over the non-outlier columns (flagged values replaced by 0,
// which is in every range anyway); outlier columns get the code of 0, -zp
// (quant8_zp of a dropped value), and their values go to the compact row of
// x_out.  Extra blocks build w_out with the zero-point dequantization.
template <int NC>
__global__ __launch_bounds__(kBlock) void k_rowquant_zp(
    const uint16_t *__restrict__ X, int64_t T, int64_t K, const DetectFlags df,
    int use, int32_t *__restrict__ O, OutlierInfoOut io, int8_t *__restrict__ Xq,
    float *__restrict__ nd_out, int2 *__restrict__ row_zp, uint16_t *__restrict__ x_out,
    const int8_t *__restrict__ CB, const float *__restrict__ NDw, const int32_t *__restrict__ ZPw,
    int64_t N, void *__restrict__ w_out, bool packed)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t s_dyn[];
    __shared__ float s_mn[kWavesPerBlock], s_mx[kWavesPerBlock];
    __shared__ int s_sum[kWavesPerBlock];
    __shared__ int s_red[4 * kWavesPerBlock];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int nchunk = (int)(K / 8);
    uint8_t *s_fl = s_dyn;
    int *s_aux = reinterpret_cast<int *>(s_dyn + flags_lds_bytes(nchunk));
    const OutlierSet os = derive_outliers(df, nchunk, s_fl, s_red);
    if ((int64_t)blockIdx.x >= T) {
        gather_block<kModeZp>(blockIdx.x - T, gridDim.x - T, K, nchunk, os, s_fl, s_aux,
                              s_red + 2 * kWavesPerBlock, CB, NDw, N, w_out, ZPw);
        return;
    }
    const bool gx = gathers_x(x_out, use, os);
    if (!row_prologue(os, s_fl, nchunk, K, use, gx, s_aux, O, io, s_red, blockIdx.x == 0))
        return;
    const int64_t t = blockIdx.x;
    const uint4 *xr = reinterpret_cast<const uint4 *>(X + t * K);
    const int nout = os.n;
    const int64_t ldo = outlier_ld(nout);
    uint16_t *xrow = gx ? x_out + t * ldo : nullptr;
    float mn = 0.0f, mx = 0.0f;
    uint4 v[NC > 0 ? NC : 1];
    unsigned fl[NC > 0 ? NC : 1];
    if constexpr (NC > 0) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int c = tid + i * kBlock;
            v[i] = c < nchunk ? xr[c] : make_uint4(0, 0, 0, 0);
            fl[i] = c < nchunk ? s_fl[c] : 0u;
        }
#pragma unroll
        for (int i = 0; i < NC; ++i)
            chunk_minmax(fl[i] ? drop_flagged(v[i], fl[i]) : v[i], mn, mx);
    } else {
        for (int c = tid; c < nchunk; c += kBlock) {
            const unsigned f = s_fl[c];
            const uint4 w = xr[c];
            chunk_minmax(f ? drop_flagged(w, f) : w, mn, mx);
        }
    }
    wave_minmax(mn, mx);
    if (lane == 0) {
        s_mn[wave] = mn;
        s_mx[wave] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
        mn = __builtin_fminf(mn, s_mn[w]);
        mx = __builtin_fmaxf(mx, s_mx[w]);
    }
    const ZpParams p = zp_params(mn, mx);
    int sum = 0;
    auto quant = [&](uint4 w, unsigned f, int c) {
        if (f) {
            if (xrow)
                scatter_outliers(w, f, chunk_pos(s_fl, s_aux, c), xrow);
            w = drop_flagged(w, f);
        }
        *xq_chunk(Xq, t, K, c, packed) = quant8_zp(w, p, sum);
    };
    if constexpr (NC > 0) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int c = tid + i * kBlock;
            if (c < nchunk)
                quant(v[i], fl[i], c);
        }
    } else {
        for (int c = tid; c < nchunk; c += kBlock)
            quant(xr[c], s_fl[c], c);
    }
    if (xrow) {
        for (int64_t j = nout + tid; j < ldo; j += kBlock)
            xrow[j] = 0;
    }
    sum = wave_sum(sum);
    if (lane == 0)
        s_sum[wave] = sum;
    __syncthreads();
    if (tid == 0) {
        int total = 0;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w)
            total += s_sum[w];
        nd_out[t] = p.nd;
        row_zp[t] = make_int2(p.zp, total);
    }
}

// Largest binary16 bit pattern whose value is <= thr (thr >= 0, not NaN);
// 0x7c00 (inf) when thr >= 65504 so that no finite value exceeds it.
unsigned threshold_bits(float thr)
{
    if (!(thr < 65504.0f))
        return 0x7c00u;
    unsigned lo = 0, hi = 0x7bffu;   // invariant: value(lo) <= thr
    while (lo < hi) {
        const unsigned mid = (lo + hi + 1) / 2;
        _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)mid);
        if ((float)h <= thr)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// k_detect over all rows into the flag sets of the detection area `mask`
// (see DetectFlags); returns what the row-quantization kernels read.
DetectFlags launch_detect(const uint16_t *X, int64_t T, int64_t K, float threshold,
                          uint8_t *mask, hipStream_t s)
{
    const DetectFlags df = detect_flags(mask, T, K);
    const dim3 grid((unsigned)(K / 64 * df.nr));
    hipLaunchKernelGGL(k_detect, grid, dim3(kDetectThreads), 0, s, X, T, K, df.nr, df.pitch,
                       threshold_bits(threshold), const_cast<uint8_t *>(df.parts));
    return df;
}

// Blocks of a row-quantization launch that build the GEMM path's outlier
// weight operand (past the row blocks): 64 weight rows per block (kOutFew:
// 16 rows per wavefront at once; kOutCompact: a wavefront walks 16 rows),
// at most 1024 blocks sharing the rows.
int64_t gather_blocks(const GatherArgs &g)
{
    if (!g.w_out)
        return 0;
    const int64_t b = (g.N + 63) / 64;
    return b > 1024 ? 1024 : b;
}

}  // namespace

hipError_t launch_quantize_weight(const uint16_t *W_t, int64_t K, int64_t N, int8_t *CB,
                                  float *SCB, hipStream_t s)
{
    const int64_t blocks = (N + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(k_quantize_weight, dim3((unsigned)blocks), dim3(kBlock), 0, s, W_t, K, N,
                       CB, SCB);
    return hipGetLastError();
}

hipError_t launch_quantize_weight_zp(const uint16_t *W_t, int64_t K, int64_t N, int8_t *CB,
                                     float *ND, int32_t *ZP, int32_t *RS, hipStream_t s)
{
    const int64_t blocks = (N + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(k_quantize_weight_zp, dim3((unsigned)blocks), dim3(kBlock), 0, s, W_t, K,
                       N, CB, ND, ZP, RS);
    return hipGetLastError();
}

hipError_t launch_quantize_act_zp(const uint16_t *X, int64_t T, int64_t K, float threshold,
                                  int8_t *Xq, float *nd, int2 *row_zp, int32_t *O,
                                  const OutlierInfoOut &io, uint8_t *mask, uint16_t *x_out,
                                  const GatherArgs &g, bool xq_packed, hipStream_t s)
{
    if ((xq_packed && T > 16) || (g.w_out && !g.zp))
        return hipErrorInvalidValue;
    if (!g.w_out && quantize_act_fits_rows(T, K)) {
        // few rows: one launch (k_quant_rows in its zero-point mode)
        const int64_t per = (K / 8 + kSmallThreads - 1) / kSmallThreads;
        const unsigned tb = threshold_bits(threshold);
        const dim3 grid((unsigned)T);
#define LLMINT8_QROWS_ZP(G)                                                                    \
    hipLaunchKernelGGL((k_quant_rows<G, kModeZp>), grid, dim3(kSmallThreads), 0, s, X, (int)T,    \
                       (int)K, tb, Xq, nd, O, io.info, x_out, xq_packed, row_zp)
        if (per <= 1)
            LLMINT8_QROWS_ZP(1);
        else if (per <= 2)
            LLMINT8_QROWS_ZP(2);
        else if (per <= 4)
            LLMINT8_QROWS_ZP(4);
        else if (per <= 8)
            LLMINT8_QROWS_ZP(8);
        else if (per <= 16)
            LLMINT8_QROWS_ZP(16);
        else
            return hipErrorInvalidValue;
#undef LLMINT8_QROWS_ZP
        return hipGetLastError();
    }
    const int64_t nchunk = K / 8;
    const int use = g.w_out ? kForGemm : x_out ? kForDecode : kForAct;
    const DetectFlags df = launch_detect(X, T, K, threshold, mask, s);
    const dim3 grid((unsigned)(T + gather_blocks(g)));
    const size_t lds = rowquant_lds_bytes(K);
    const int64_t chunks_per_thread = (nchunk + kBlock - 1) / kBlock;
#define LLMINT8_ROWQUANT_ZP(NCV)                                                               \
    hipLaunchKernelGGL(k_rowquant_zp<NCV>, grid, dim3(kBlock), lds, s, X, T, K, df,   use, O,    \
                       io, Xq, nd, row_zp, x_out, g.CB, g.SCB, g.zp, g.N, g.w_out, xq_packed)
    if (chunks_per_thread <= 1)
        LLMINT8_ROWQUANT_ZP(1);
    else if (chunks_per_thread <= 2)
        LLMINT8_ROWQUANT_ZP(2);
    else if (chunks_per_thread <= 4)
        LLMINT8_ROWQUANT_ZP(4);
    else if (chunks_per_thread <= 8)
        LLMINT8_ROWQUANT_ZP(8);
    else
        LLMINT8_ROWQUANT_ZP(0);
#undef LLMINT8_ROWQUANT_ZP
    return hipGetLastError();
}

bool quantize_act_fits_rows(int64_t T, int64_t K)
{
    return T == 1 ? K <= kQuantRowsMaxK1 : T <= kQuantRowsMaxT && K <= kQuantRowsMaxK;
}

hipError_t launch_quantize_act_rows(const uint16_t *X, int64_t T, int64_t K, float threshold,
                                    int8_t *Xq, float *a, int32_t *O, int32_t *n_out,
                                    uint16_t *x_out, bool xq_packed, hipStream_t s)
{
    if (!quantize_act_fits_rows(T, K))
        return hipErrorInvalidValue;
    // G chunks per thread: K/8 <= G * kSmallThreads
    const int64_t per = (K / 8 + kSmallThreads - 1) / kSmallThreads;
    const unsigned tb = threshold_bits(threshold);
    const dim3 grid((unsigned)T);
#define LLMINT8_QROWS(G)                                                                          \
    hipLaunchKernelGGL((k_quant_rows<G>), grid, dim3(kSmallThreads), 0, s, X, (int)T, (int)K, tb, \
                       Xq, a, O, n_out, x_out, xq_packed)
    if (per <= 1)
        LLMINT8_QROWS(1);
    else if (per <= 2)
        LLMINT8_QROWS(2);
    else if (per <= 4)
        LLMINT8_QROWS(4);
    else if (per <= 8)
        LLMINT8_QROWS(8);
    else if (per <= 16)
        LLMINT8_QROWS(16);
    else
        return hipErrorInvalidValue;
#undef LLMINT8_QROWS
    return hipGetLastError();
}

namespace {
// Detection and the row quantization of the absmax kernels (kF8: their FP8
// mode of that format).
template <int kF8>
hipError_t launch_act_absmax(const uint16_t *X, int64_t T, int64_t K, float threshold,
                             int8_t *Xq, float *a, int32_t *O, const OutlierInfoOut &io,
                             uint8_t *mask, uint16_t *x_out, const GatherArgs &g,
                             bool xq_packed, hipStream_t s)
{
    if (xq_packed && T > 16)
        return hipErrorInvalidValue;
    const int64_t nchunk = K / 8;
    const int use = g.w_out ? kForGemm : x_out ? kForDecode : kForAct;
    const DetectFlags df = launch_detect(X, T, K, threshold, mask, s);
    const int64_t gb = gather_blocks(g);
    const size_t lds = rowquant_lds_bytes(K);
    if (T >= kRowQuantWaveMinT && K <= kRowQuantWaveMaxK && !xq_packed && use != kForDecode) {
        // a wavefront per row, the row in NC chunks per lane (its outlier
        // gather lists at most kCompactMaxLd columns: the GEMM path's modes
        // with gathered rows)
        const int64_t per = (nchunk + kWave - 1) / kWave;
        const int64_t row_blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
        const dim3 grid((unsigned)(row_blocks + gb));
#define LLMINT8_ROWQUANT_W(NCV)                                                                \
    hipLaunchKernelGGL((k_rowquant_w<NCV, kF8>), grid, dim3(kBlock), lds, s, X, T, K, df,        \
                       use, O, io, Xq, a, x_out, g.CB, g.SCB, g.N, g.w_out, row_blocks)
        static_assert(kRowQuantWaveMaxK / 8 <= 8 * kWave, "rows of at most 8 chunks per lane");
        if (per <= 2)
            LLMINT8_ROWQUANT_W(2);
        else if (per <= 4)
            LLMINT8_ROWQUANT_W(4);
        else
            LLMINT8_ROWQUANT_W(8);
#undef LLMINT8_ROWQUANT_W
        return hipGetLastError();
    }
    // fewer rows: a block per row keeps more lanes busy; the kept-column mode
    // of the 8-bit part is taken here (absmax and FP8, enough rows, K in range)
    const bool kept = g.cb_kept && use == kForGemm && T >= kKeptMinT && K <= kKeptMaxK;
    int8_t *cb_kept = kept ? g.cb_kept : nullptr;
    const size_t lds_rows = rowquant_lds_bytes(K, kept);
    const dim3 grid((unsigned)(T + gb));
    const int64_t chunks_per_thread = (nchunk + kBlock - 1) / kBlock;
#define LLMINT8_ROWQUANT(NCV)                                                                  \
    hipLaunchKernelGGL((k_rowquant<NCV, kF8>), grid, dim3(kBlock), lds_rows, s, X, T, K, df,     \
                       use, O, io, Xq, a, x_out, g.CB, g.SCB, g.N, g.w_out, xq_packed, cb_kept,   \
                       threshold > 0.0f)
    if (chunks_per_thread <= 1)
        LLMINT8_ROWQUANT(1);
    else if (chunks_per_thread <= 2)
        LLMINT8_ROWQUANT(2);
    else if (chunks_per_thread <= 4)
        LLMINT8_ROWQUANT(4);
    else if (chunks_per_thread <= 8)
        LLMINT8_ROWQUANT(8);
    else if (chunks_per_thread <= 16)
        LLMINT8_ROWQUANT(16);
    else
        LLMINT8_ROWQUANT(0);
#undef LLMINT8_ROWQUANT
    return hipGetLastError();
}
}  // namespace

hipError_t launch_quantize_act(const uint16_t *X, int64_t T, int64_t K, float threshold,
                               int8_t *Xq, float *a, int32_t *O, const OutlierInfoOut &io,
                               uint8_t *mask, uint16_t *x_out, const GatherArgs &g,
                               bool xq_packed, hipStream_t s)
{
    return launch_act_absmax<kF8None>(X, T, K, threshold, Xq, a, O, io, mask, x_out, g,
                                    xq_packed, s);
}

hipError_t launch_quantize_weight_f8(const uint16_t *W_t, int64_t K, int64_t N, uint8_t *CB8,
                                     float *SC8, int fmt, hipStream_t s)
{
    const int64_t blocks = (N + kWavesPerBlock - 1) / kWavesPerBlock;
    if (fmt == kF8E4M3)
        hipLaunchKernelGGL(k_quantize_weight_f8<kF8E4M3>, dim3((unsigned)blocks), dim3(kBlock), 0,
                           s, W_t, K, N, CB8, SC8);
    else if (fmt == kF8E5M2)
        hipLaunchKernelGGL(k_quantize_weight_f8<kF8E5M2>, dim3((unsigned)blocks), dim3(kBlock), 0,
                           s, W_t, K, N, CB8, SC8);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_quantize_act_f8(const uint16_t *X, int64_t T, int64_t K, float threshold,
                                  uint8_t *Xq8, float *sc, int32_t *O, const OutlierInfoOut &io,
                                  uint8_t *mask, uint16_t *x_out, const GatherArgs &g,
                                  bool xq_packed, int fmt, hipStream_t s)
{
    if ((fmt != kF8E5M2 && fmt != kF8E4M3) || (g.w_out && g.f8 != fmt))
        return hipErrorInvalidValue;
    int8_t *Xq = reinterpret_cast<int8_t *>(Xq8);
    if (!g.w_out && quantize_act_fits_rows(T, K)) {
        // few rows: one launch (k_quant_rows in its FP8 mode)
        const int64_t per = (K / 8 + kSmallThreads - 1) / kSmallThreads;
        const unsigned tb = threshold_bits(threshold);
        const dim3 grid((unsigned)T);
#define LLMINT8_QROWS_F8(G)                                                                    \
    if (fmt == kF8E4M3)                                                                        \
        hipLaunchKernelGGL((k_quant_rows<G, kModeF8E4>), grid, dim3(kSmallThreads), 0, s, X,   \
                           (int)T, (int)K, tb, Xq, sc, O, io.info, x_out, xq_packed, nullptr); \
    else                                                                                       \
        hipLaunchKernelGGL((k_quant_rows<G, kModeF8>), grid, dim3(kSmallThreads), 0, s, X,     \
                           (int)T, (int)K, tb, Xq, sc, O, io.info, x_out, xq_packed, nullptr)
        if (per <= 1)
            LLMINT8_QROWS_F8(1);
        else if (per <= 2)
            LLMINT8_QROWS_F8(2);
        else if (per <= 4)
            LLMINT8_QROWS_F8(4);
        else if (per <= 8)
            LLMINT8_QROWS_F8(8);
        else if (per <= 16)
            LLMINT8_QROWS_F8(16);
        else
            return hipErrorInvalidValue;
#undef LLMINT8_QROWS_F8
        return hipGetLastError();
    }
    if (fmt == kF8E4M3)
        return launch_act_absmax<kF8E4M3>(X, T, K, threshold, Xq, sc, O, io, mask, x_out, g,
                                          xq_packed, s);
    return launch_act_absmax<kF8E5M2>(X, T, K, threshold, Xq, sc, O, io, mask, x_out, g,
                                      xq_packed, s);
}

}  // namespace llmint8
