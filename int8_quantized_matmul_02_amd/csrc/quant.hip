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

// FP8 variant: E5M2 codes of 8 values scaled by sc = 2^e (the product is
// exact: a power of two, and |x * 2^e| <= 57344), each rounded to the
// nearest E5M2 value with ties to even by v_cvt_pk_bf8_f32 (two per
// instruction, into the low or high half of a dword).
__device__ __forceinline__ uint2 quant8_f8(uint4 v, float sc)
{
    unsigned w[2];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        int x = 0;
        x = __builtin_amdgcn_cvt_pk_bf8_f32(h2f(half_at(v, 4 * d)) * sc,
                                            h2f(half_at(v, 4 * d + 1)) * sc, x, false);
        x = __builtin_amdgcn_cvt_pk_bf8_f32(h2f(half_at(v, 4 * d + 2)) * sc,
                                            h2f(half_at(v, 4 * d + 3)) * sc, x, true);
        w[d] = (unsigned)x;
    }
    return make_uint2(w[0], w[1]);
}

// The row quantization of an absmax-type kernel: int8 codes from (amax, r =
// 127/amax), or (kF8) E5M2 codes from sc = 2^e.
template <bool kF8>
__device__ __forceinline__ uint2 quant8_mode(uint4 v, float amax, float r, float sc)
{
    if constexpr (kF8)
        return quant8_f8(v, sc);
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
// the row's absmax, E5M2 codes, and the stored scale 2^-e.
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
    const int e = f8_scale_exp(h2f((uint16_t)m));
    const float sc = __builtin_ldexpf(1.0f, e);
    uint2 *dst = reinterpret_cast<uint2 *>(CB8 + n * K);
    for (int64_t c = lane; c < nchunk; c += kWave)
        dst[c] = quant8_f8(row[c], sc);
    if (lane == 0)
        SC8[n] = __builtin_ldexpf(1.0f, -e);
}

// ---------------------------------------------------------------------------
// Outlier-column detection, in two launches and without atomics or a
// clearing pass.  k_detect splits the rows into kDetectSplits ranges; a lane
// keeps the running column maxima of |x| of 8 columns over its rows, the
// flags "maximum above the threshold" are ORed over the block's row groups
// and written as byte partial[chunk * kDetectSplits + split] (every byte is
// written, also for empty ranges).  k_compact ORs the 16 bytes of a chunk.
// The comparison |x| > threshold is done on binary16 bit patterns against the
// largest binary16 value not above the threshold (computed on the host), which
// is the same test as comparing the exact values.
// ---------------------------------------------------------------------------
constexpr int kDetectThreads = 1024;
constexpr int kDetectRowGroups = kDetectThreads / 32;   // 32 lanes (chunks) per row group

__global__ __launch_bounds__(kDetectThreads) void k_detect(const uint16_t *__restrict__ X,
                                                           int64_t T, int64_t K,
                                                           unsigned thr_bits, int64_t rows_per,
                                                           uint8_t *__restrict__ partial)
{
    // byte rg of chunk lane c at s_bits[c * kDetectRowGroups + rg]
    __shared__ unsigned s_bits[32 * kDetectRowGroups / 4];
    const int c = threadIdx.x & 31, rg = threadIdx.x >> 5;
    const int64_t col8 = (int64_t)blockIdx.x * 32 + c;    // 8-column chunk
    const int64_t nchunk = K / 8;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per;
    const int64_t r1 = r0 + rows_per < T ? r0 + rows_per : T;
    unsigned bits = 0;
    if (col8 < nchunk) {
        constexpr int kRowsInFlight = 8;
        uint4 cm = make_uint4(0u, 0u, 0u, 0u);
        for (int64_t t0 = r0 + rg; t0 < r1; t0 += kRowsInFlight * kDetectRowGroups) {
            uint4 v[kRowsInFlight];
#pragma unroll
            for (int u = 0; u < kRowsInFlight; ++u) {
                const int64_t t = t0 + (int64_t)u * kDetectRowGroups;
                v[u] = t < r1 ? *reinterpret_cast<const uint4 *>(X + t * K + col8 * 8)
                              : make_uint4(0u, 0u, 0u, 0u);   // |0| is never above
            }
#pragma unroll
            for (int u = 0; u < kRowsInFlight; ++u)
                cm = colmax8(cm, v[u]);
        }
        bits = flags8(cm, thr_bits);
    }
    reinterpret_cast<uint8_t *>(s_bits)[c * kDetectRowGroups + rg] = (uint8_t)bits;
    __syncthreads();
    if (rg == 0 && col8 < nchunk) {
        unsigned o = 0;
#pragma unroll
        for (int w = 0; w < kDetectRowGroups / 4; ++w)
            o |= s_bits[c * (kDetectRowGroups / 4) + w];
        o |= o >> 16;
        o |= o >> 8;
        partial[col8 * kDetectSplits + blockIdx.y] = (uint8_t)(o & 0xffu);
    }
}

// The OR of a chunk's kDetectSplits partial bytes: its 8 outlier flags.
__device__ __forceinline__ unsigned chunk_flags(const uint8_t *__restrict__ partial, int64_t c)
{
    static_assert(kDetectSplits == 16, "one 16-byte load per chunk");
    const uint4 p = *reinterpret_cast<const uint4 *>(partial + c * kDetectSplits);
    unsigned o = p.x | p.y | p.z | p.w;
    o |= o >> 16;
    o |= o >> 8;
    return o & 0xffu;
}

constexpr int kCompactThreads = 1024;
constexpr int kMaxChunks = 133144 / 8 + 1;   // K/8 for the largest K

// One block.  Every thread ORs the partial bytes of its chunks (one 16-byte
// load each, all independent) into an LDS flag byte; then mask[b] = the flags
// of 8-column chunk b, the ascending outlier list O, its length n, and
// chunk_pre[b] = the number of outlier columns before chunk b (the position
// of its first one in O).  Each thread owns a contiguous run of chunks so a
// block-wide exclusive scan of the per-thread counts gives the positions.
__global__ __launch_bounds__(kCompactThreads) void k_compact(const uint8_t *__restrict__ partial,
                                                             int64_t K,
                                                             uint8_t *__restrict__ mask,
                                                             int32_t *__restrict__ O,
                                                             int32_t *__restrict__ n_out,
                                                             int32_t *__restrict__ chunk_pre)
{
    __shared__ uint8_t s_fl[kMaxChunks];
    __shared__ int wave_tot[kCompactThreads / kWave];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    // 32-bit indexing: K <= 133144 keeps every count here far below 2^31
    const int nchunk = (int)(K / 8);
    constexpr int kBatch = 4;   // independent loads in flight per thread
    for (int base = tid; base < nchunk; base += kBatch * kCompactThreads) {
        unsigned f[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int c = base + u * kCompactThreads;
            f[u] = c < nchunk ? chunk_flags(partial, c) : 0u;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int c = base + u * kCompactThreads;
            if (c < nchunk)
                s_fl[c] = (uint8_t)f[u];
        }
    }
    __syncthreads();
    const int per = (nchunk + kCompactThreads - 1) / kCompactThreads;
    const int b0 = tid * per < nchunk ? tid * per : nchunk;
    const int b1 = b0 + per < nchunk ? b0 + per : nchunk;
    int cnt = 0;
    for (int b = b0; b < b1; ++b) {
        const unsigned m = s_fl[b];
        mask[b] = (uint8_t)m;
        cnt += __builtin_popcount(m);
    }
    int inc = cnt;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(inc, off, kWave);
        if (lane >= off)
            inc += o;
    }
    if (lane == kWave - 1)
        wave_tot[wave] = inc;
    __syncthreads();
    int j = inc - cnt;
    for (int w = 0; w < wave; ++w)
        j += wave_tot[w];
    for (int b = b0; b < b1; ++b) {
        const unsigned m = s_fl[b];
        chunk_pre[b] = j;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if ((m >> i) & 1u)
                O[j++] = b * 8 + i;
    }
    if (tid == kCompactThreads - 1)
        *n_out = j;
}

// ---------------------------------------------------------------------------
// Row quantization: one 256-thread block per row t (so that even a handful of
// rows keeps many lanes busy).  The row is read once into registers (NC
// 16-byte chunks per thread; NC = 0 re-reads it from cache for very long
// rows), its absmax over the non-outlier columns is reduced with shuffles and
// LDS, then the int8 row is packed with outlier columns as 0, and the outlier
// values are gathered into the compact fp16 row x_out[t, .] (row stride
// outlier_ld(n), zero-padded): the outlier columns of chunk c start at
// chunk_pre[c], loaded once per such chunk while the absmax is reduced.
// Chunks without outlier columns (nearly all of them) take a branch-free path.
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
template <bool kF8 = false>
__device__ __forceinline__ void quant_chunk(uint4 v, unsigned fl, float amax, float r, int pre,
                                           uint16_t *__restrict__ xrow, uint2 *dst, float sc = 0.0f)
{
    if (fl) {
        if (xrow)
            scatter_outliers(v, fl, pre, xrow);
        v = drop_flagged(v, fl);
    }
    *dst = quant8_mode<kF8>(v, amax, r, sc);
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

// Dequantized outlier weight rows for the GEMM, w_out[r, j] = fp16(CB[r, O[j]]
// * SCB[r] / 127), zero up to outlier_ld(n): blocks gb = 0 .. nb-1 of a
// launch share the N rows.  Up to 32 outliers (one 32-half row each) a lane
// takes one 8-column group of one row, 16 rows per wavefront, and computes
// its at most 8 values directly.  More outliers: one wavefront per row, which
// first tabulates the row's 255 possible values in LDS (tab, 256 entries of
// this wavefront); each lane then gathers 8 consecutive outlier columns and
// stores them at once.  (LDS operations of one wavefront complete in order,
// so the table is complete before any lane reads it, and the reads of one
// row are done before the next row's table overwrites it.)  Entries of O at
// or past n are stale: column 0 is read in their place and the value is 0.
// kMode 0: absmax.  1, zero-point variant: SCB holds each row's nd, ZP its
// zp, and the values are fp16((cb + zp) / nd).  2, FP8 variant: the bytes
// are E5M2 codes and SCB the scales 2^-e.
constexpr int kModeAbsmax = 0, kModeZp = 1, kModeF8 = 2;
template <int kMode>
__device__ __forceinline__ uint16_t dequant_row(int cb, float sc, int zp)
{
    if constexpr (kMode == kModeF8)
        return dequant_w_f8((unsigned)cb & 0xffu, sc);
    else if constexpr (kMode == kModeZp)
        return dequant_w_zp(cb, zp, sc);
    else
        return dequant_w(cb, sc);
}

template <int kMode = kModeAbsmax>
__device__ __forceinline__ void gather_w_out(int64_t gb, int64_t nb, int64_t K,
                                             const int32_t *__restrict__ n_out,
                                             const int8_t *__restrict__ CB,
                                             const float *__restrict__ SCB,
                                             const int32_t *__restrict__ O, int64_t N,
                                             uint16_t *__restrict__ w_out, uint16_t *tab,
                                             const int32_t *__restrict__ ZP = nullptr)
{
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int n = *n_out;
    const int64_t ldo = outlier_ld(n);
    if (ldo == kOutlierPad) {
        constexpr int kGroups = kOutlierPad / 8, kRowsPerWave = kWave / kGroups;
        const int g = lane % kGroups;
        int o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int j = 8 * g + e;   // < 32 <= K: in bounds of O
            o[e] = j < n ? O[j] : 0;
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
            *reinterpret_cast<uint4 *>(w_out + r * kOutlierPad + 8 * g) =
                make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                           h[6] | (h[7] << 16));
        }
        return;
    }
    for (int64_t r = gb * kWavesPerBlock + wave; r < N; r += nb * kWavesPerBlock) {
        const float sc = SCB[r];
        const int zr = kMode == kModeZp ? ZP[r] : 0;
        // table index: code + 127 of an int8 code (255 entries), or the E5M2
        // code itself (256)
        constexpr int kBias = kMode == kModeF8 ? 0 : 127;
        for (int i = lane; i < 256 - (kBias ? 1 : 0); i += kWave)
            tab[i] = dequant_row<kMode>(i - kBias, sc, zr);
        const int8_t *cbr = CB + r * K;
        for (int64_t j0 = 8 * lane; j0 < ldo; j0 += 8 * kWave) {
            const int4 o0 = *reinterpret_cast<const int4 *>(O + j0);
            const int4 o1 = *reinterpret_cast<const int4 *>(O + j0 + 4);
            const int o[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
            unsigned h[8];
            if (j0 + 8 <= n && o[7] == o[0] + 7 && (o[0] & 7) == 0) {
                // 8 consecutive outlier columns (every column, at threshold 0):
                // one 8-byte load of the weight row (8-byte aligned; K % 64 == 0)
                const uint2 raw = *reinterpret_cast<const uint2 *>(cbr + o[0]);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int cb = (int)(int8_t)(((e < 4 ? raw.x : raw.y) >> (8 * (e & 3))) & 0xffu);
                    h[e] = tab[(cb + kBias) & 255];
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int oc = j0 + e < n ? o[e] : 0;
                    const unsigned v = tab[(cbr[oc] + kBias) & 255];
                    h[e] = j0 + e < n ? v : 0u;
                }
            }
            *reinterpret_cast<uint4 *>(w_out + r * ldo + j0) =
                make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                           h[6] | (h[7] << 16));
        }
    }
}

template <int NC, bool kF8 = false>
__global__ __launch_bounds__(kBlock) void k_rowquant(const uint16_t *__restrict__ X, int64_t T,
                                                     int64_t K, const uint8_t *__restrict__ mask,
                                                     const int32_t *__restrict__ chunk_pre,
                                                     const int32_t *__restrict__ n_out,
                                                     int8_t *__restrict__ Xq,
                                                     float *__restrict__ a,
                                                     uint16_t *__restrict__ x_out,
                                                     const int8_t *__restrict__ CB,
                                                     const float *__restrict__ SCB,
                                                     const int32_t *__restrict__ O, int64_t N,
                                                     uint16_t *__restrict__ w_out, bool packed)
{
    __shared__ unsigned s_max[kWavesPerBlock];
    __shared__ uint16_t s_tab[kWavesPerBlock][256];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    if ((int64_t)blockIdx.x >= T) {
        gather_w_out<kF8 ? kModeF8 : kModeAbsmax>(blockIdx.x - T, gridDim.x - T, K, n_out, CB, SCB,
                                                  O, N, w_out, s_tab[wave]);
        return;
    }
    const int64_t t = blockIdx.x;
    const uint4 *xr = reinterpret_cast<const uint4 *>(X + t * K);
    const int nout = x_out ? *n_out : 0;
    const int64_t ldo = outlier_ld(nout);
    const int64_t nchunk = K / 8;
    uint16_t *xrow = x_out ? x_out + t * ldo : nullptr;
    unsigned m = 0;
    uint4 v[NC > 0 ? NC : 1];
    unsigned fl[NC > 0 ? NC : 1];
    int pre[NC > 0 ? NC : 1];
    if constexpr (NC > 0) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int64_t c = tid + (int64_t)i * kBlock;
            v[i] = c < nchunk ? xr[c] : make_uint4(0, 0, 0, 0);
            fl[i] = c < nchunk ? mask[c] : 0u;
        }
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int64_t c = tid + (int64_t)i * kBlock;
            pre[i] = (xrow && fl[i] != 0u) ? chunk_pre[c] : 0;   // lands during the reduction
        }
#pragma unroll
        for (int i = 0; i < NC; ++i)
            m = umax(m, chunk_absmax_masked(v[i], fl[i]));
    } else {
        for (int64_t c = tid; c < nchunk; c += kBlock)
            m = umax(m, chunk_absmax_masked(xr[c], mask[c]));
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
    const int e8 = kF8 ? f8_scale_exp(amax) : 0;
    const float sc = kF8 ? __builtin_ldexpf(1.0f, e8) : 0.0f;
    if constexpr (NC > 0) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int64_t c = tid + (int64_t)i * kBlock;
            if (c < nchunk)
                quant_chunk<kF8>(v[i], fl[i], amax, r, pre[i], xrow,
                                 xq_chunk(Xq, t, K, c, packed), sc);
        }
    } else {
        for (int64_t c = tid; c < nchunk; c += kBlock) {
            const unsigned f = mask[c];
            quant_chunk<kF8>(xr[c], f, amax, r, (xrow && f != 0u) ? chunk_pre[c] : 0, xrow,
                             xq_chunk(Xq, t, K, c, packed), sc);
        }
    }
    if (x_out) {
        for (int j = nout + tid; j < ldo; j += kBlock)
            x_out[t * ldo + j] = 0;
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
// take the same arithmetic, and the outlier values go to the compact row of
// x_out at positions from a wavefront prefix count of the flags (ballots), so
// no per-chunk position table is read.  Extra blocks build w_out as
// k_rowquant's.
// ---------------------------------------------------------------------------
// Outlier columns before this lane's chunk within one 64-chunk step of a
// wavefront (lanes below it), and in the whole step: per flag bit, a ballot
// and its masked population count.
__device__ __forceinline__ void step_prefix(unsigned fl, uint64_t below, int &pre, int &tot)
{
    pre = 0;
    tot = 0;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const uint64_t m = __ballot((fl >> b) & 1u);
        pre += __popcll(m & below);
        tot += __popcll(m);
    }
}

template <int NC, bool kF8 = false>
__global__ __launch_bounds__(kBlock) void k_rowquant_w(const uint16_t *__restrict__ X, int64_t T,
                                                       int64_t K, const uint8_t *__restrict__ mask,
                                                       const int32_t *__restrict__ n_out,
                                                       int8_t *__restrict__ Xq,
                                                       float *__restrict__ a,
                                                       uint16_t *__restrict__ x_out,
                                                       const int8_t *__restrict__ CB,
                                                       const float *__restrict__ SCB,
                                                       const int32_t *__restrict__ O, int64_t N,
                                                       uint16_t *__restrict__ w_out,
                                                       int64_t row_blocks)
{
    __shared__ uint16_t s_tab[kWavesPerBlock][256];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    if ((int64_t)blockIdx.x >= row_blocks) {
        gather_w_out<kF8 ? kModeF8 : kModeAbsmax>(blockIdx.x - row_blocks, gridDim.x - row_blocks,
                                                  K, n_out, CB, SCB, O, N, w_out, s_tab[wave]);
        return;
    }
    const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if (t >= T)
        return;
    const uint4 *xr = reinterpret_cast<const uint4 *>(X + t * K);
    uint2 *qr = reinterpret_cast<uint2 *>(Xq + t * K);
    const int64_t nchunk = K / 8;
    const int nout = x_out ? *n_out : 0;
    const int64_t ldo = outlier_ld(nout);
    uint16_t *xrow = x_out ? x_out + t * ldo : nullptr;
    const uint64_t below = (1ull << lane) - 1ull;
    uint4 v[NC];
    unsigned fl[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int64_t c = lane + (int64_t)i * kWave;
        v[i] = c < nchunk ? xr[c] : make_uint4(0u, 0u, 0u, 0u);
        fl[i] = c < nchunk ? mask[c] : 0u;
    }
    // the outlier values first, then they are zeroed in place
    if (xrow && nout > 0) {
        int base = 0;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            if (__ballot(fl[i] != 0u) == 0ull)
                continue;
            int pre, tot;
            step_prefix(fl[i], below, pre, tot);
            if (fl[i])
                scatter_outliers(v[i], fl[i], base + pre, xrow);
            base += tot;
        }
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
    const int e8 = kF8 ? f8_scale_exp(amax) : 0;
    const float sc = kF8 ? __builtin_ldexpf(1.0f, e8) : 0.0f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int64_t c = lane + (int64_t)i * kWave;
        if (c < nchunk)
            qr[c] = quant8_mode<kF8>(v[i], amax, r, sc);
    }
    if (xrow) {
        for (int64_t j = nout + lane; j < ldo; j += kWave)
            xrow[j] = 0;
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

__device__ __forceinline__ int wave_sum(int v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    return v;
}

// (nd, zp) of a vector whose range [mn, mx] already contains 0:
// d = fp32(mx - mn) and nd = fp32(254/d), each rounded once (the division is
// IEEE-correct: the library is built with correctly rounded fp32 division);
// zp = RNE(nd*mn) + 127, the product rounded exactly once by the fused
// multiply-add with kRoundMagic (|nd*mn| <= 254.0001, so the sum sits where
// the fp32 spacing is 1).  d = 0 gives (0, 0).
struct ZpParams {
    float nd;
    int zp;
};
__device__ __forceinline__ ZpParams zp_params(float mn, float mx)
{
    const float d = mx - mn;
    if (!(d > 0.0f))
        return ZpParams{0.0f, 0};
    const float nd = 254.0f / d;
    const float s = __builtin_fmaf(mn, nd, kRoundMagic);
    return ZpParams{nd, (int)(s - kRoundMagic) + 127};
}

// Codes of 8 values, min(RNE(nd*x) - zp, 127): one fused multiply-add per
// value with the addend kRoundMagic rounds the exact product to an integer
// (ties to even, kRoundMagic being even; an odd addend such as
// kRoundMagic - zp would send ties to odd), then zp (zpf, an integer, so the
// subtraction is exact within [2^23, 2^24)) is subtracted, the clamp is an
// fp32 min, and the code is the low byte.  The codes' sum is added to *sum
// (bits(kRoundMagic + q) - bits(kRoundMagic) = q).
__device__ __forceinline__ uint2 quant8_zp(uint4 v, float nd, float zpf, int &sum)
{
    float s[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        s[i] = __builtin_fminf(__builtin_fmaf(h2f(half_at(v, i)), nd, kRoundMagic) - zpf,
                               kRoundMagic + 127.0f);
        sum += (int)(__builtin_bit_cast(unsigned, s[i]) - __builtin_bit_cast(unsigned, kRoundMagic));
    }
    return pack_low_bytes(s);
}

// ---------------------------------------------------------------------------
// Few rows (T <= 16, the decode regime): the whole quantization in one
// launch of T blocks, block t quantizing row t.  The outlier set depends on
// every row, and at these sizes each block can afford to read all of X (at
// most 16 rows x 16384 columns): every block derives the same flags itself,
// so no partial flags, compaction launch or workspace are needed.  A thread
// owns the 8-column chunks c = tid, tid + 512, ... (G of them):
//   1. it loads its chunks of every row, R rows at a time, keeps the column
//      maxima of |x| (the flags follow from them) and row t's chunks;
//   2. a block scan over the chunk flags in column order gives, per chunk,
//      the number of outlier columns before it and n (block 0 also writes
//      the ascending outlier list and n);
//   3. the absmax of row t over the other columns (wave reductions and the 8
//      wave maxima through LDS), then the packed int8 row and the row's
//      outlier values in x_out.
// The tests and the arithmetic are those of k_detect / k_compact /
// k_rowquant, so the results are identical bit for bit.
// ---------------------------------------------------------------------------
constexpr int kSmallThreads = 512;
constexpr int kSmallMaxChunks = 16 * kSmallThreads;   // G <= 16: K <= 65536

// kMode kModeZp, the zero-point variant (a receives nd, row_zp {zp, code
// sum}): the range instead of the absmax in step 3, codes by quant8_zp, and
// one more block reduction for the code sum.  kModeF8, the FP8 variant: the
// absmax sets the power-of-two scale, codes by quant8_f8, a receives 2^-e.
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
    ZpParams p{0.0f, 0};
    if constexpr (kMode == kModeZp) {
        float mn = 0.0f, mx = 0.0f;
#pragma unroll
        for (int w = 0; w < kSmallThreads / kWave; ++w) {
            mn = __builtin_fminf(mn, s_wmn[w]);
            mx = __builtin_fmaxf(mx, __builtin_bit_cast(float, s_wmax[w]));
        }
        p = zp_params(mn, mx);
        zpf = (float)p.zp;
    } else {
        unsigned amax_bits = 0;
#pragma unroll
        for (int w = 0; w < kSmallThreads / kWave; ++w)
            amax_bits = umax(amax_bits, s_wmax[w]);
        amax = h2f((uint16_t)amax_bits);
        if constexpr (kMode == kModeF8) {
            const int e8 = f8_scale_exp(amax);
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
            q = quant8_zp(x, p.nd, zpf, sum);
        else if constexpr (kMode == kModeF8)
            q = quant8_f8(x, zpf);
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
    const float zpf = (float)p.zp;
    uint2 *dst = reinterpret_cast<uint2 *>(CB + n * K);
    int sum = 0;
    for (int64_t c = lane; c < nchunk; c += kWave)
        dst[c] = quant8_zp(row[c], p.nd, zpf, sum);
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
    const uint16_t *__restrict__ X, int64_t T, int64_t K, const uint8_t *__restrict__ mask,
    const int32_t *__restrict__ chunk_pre, const int32_t *__restrict__ n_out,
    int8_t *__restrict__ Xq, float *__restrict__ nd_out, int2 *__restrict__ row_zp,
    uint16_t *__restrict__ x_out, const int8_t *__restrict__ CB, const float *__restrict__ NDw,
    const int32_t *__restrict__ ZPw, const int32_t *__restrict__ O, int64_t N,
    uint16_t *__restrict__ w_out, bool packed)
{
    __shared__ float s_mn[kWavesPerBlock], s_mx[kWavesPerBlock];
    __shared__ int s_sum[kWavesPerBlock];
    __shared__ uint16_t s_tab[kWavesPerBlock][256];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    if ((int64_t)blockIdx.x >= T) {
        gather_w_out<kModeZp>(blockIdx.x - T, gridDim.x - T, K, n_out, CB, NDw, O, N, w_out,
                              s_tab[wave], ZPw);
        return;
    }
    const int64_t t = blockIdx.x;
    const uint4 *xr = reinterpret_cast<const uint4 *>(X + t * K);
    const int nout = x_out ? *n_out : 0;
    const int64_t ldo = outlier_ld(nout);
    const int64_t nchunk = K / 8;
    uint16_t *xrow = x_out ? x_out + t * ldo : nullptr;
    float mn = 0.0f, mx = 0.0f;
    uint4 v[NC > 0 ? NC : 1];
    unsigned fl[NC > 0 ? NC : 1];
    int pre[NC > 0 ? NC : 1];
    if constexpr (NC > 0) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int64_t c = tid + (int64_t)i * kBlock;
            v[i] = c < nchunk ? xr[c] : make_uint4(0, 0, 0, 0);
            fl[i] = c < nchunk ? mask[c] : 0u;
        }
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int64_t c = tid + (int64_t)i * kBlock;
            pre[i] = (xrow && fl[i] != 0u) ? chunk_pre[c] : 0;
        }
#pragma unroll
        for (int i = 0; i < NC; ++i)
            chunk_minmax(fl[i] ? drop_flagged(v[i], fl[i]) : v[i], mn, mx);
    } else {
        for (int64_t c = tid; c < nchunk; c += kBlock) {
            const unsigned f = mask[c];
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
    const float zpf = (float)p.zp;
    int sum = 0;
    auto quant = [&](uint4 w, unsigned f, int pr, int64_t c) {
        if (f) {
            if (xrow)
                scatter_outliers(w, f, pr, xrow);
            w = drop_flagged(w, f);
        }
        *xq_chunk(Xq, t, K, c, packed) = quant8_zp(w, p.nd, zpf, sum);
    };
    if constexpr (NC > 0) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int64_t c = tid + (int64_t)i * kBlock;
            if (c < nchunk)
                quant(v[i], fl[i], pre[i], c);
        }
    } else {
        for (int64_t c = tid; c < nchunk; c += kBlock) {
            const unsigned f = mask[c];
            quant(xr[c], f, (xrow && f != 0u) ? chunk_pre[c] : 0, c);
        }
    }
    if (x_out) {
        for (int j = nout + tid; j < ldo; j += kBlock)
            x_out[t * ldo + j] = 0;
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
                                  int32_t *n_out, uint8_t *partial, uint8_t *mask,
                                  int32_t *chunk_pre, uint16_t *x_out, const GatherArgs &g,
                                  bool xq_packed, hipStream_t s)
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
                       (int)K, tb, Xq, nd, O, n_out, x_out, xq_packed, row_zp)
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
    const int64_t rows_per = (T + kDetectSplits - 1) / kDetectSplits;
    const dim3 det_grid((unsigned)((nchunk + 31) / 32), (unsigned)kDetectSplits);
    hipLaunchKernelGGL(k_detect, det_grid, dim3(kDetectThreads), 0, s, X, T, K,
                       threshold_bits(threshold), rows_per, partial);
    hipLaunchKernelGGL(k_compact, dim3(1), dim3(kCompactThreads), 0, s, partial, K, mask, O, n_out,
                       chunk_pre);
    int64_t gather_blocks = 0;
    if (g.w_out) {
        gather_blocks = (g.N + kWavesPerBlock - 1) / kWavesPerBlock;
        if (gather_blocks > 2048)
            gather_blocks = 2048;
    }
    const dim3 grid((unsigned)(T + gather_blocks));
    const int64_t chunks_per_thread = (nchunk + kBlock - 1) / kBlock;
#define LLMINT8_ROWQUANT_ZP(NCV)                                                              \
    hipLaunchKernelGGL(k_rowquant_zp<NCV>, grid, dim3(kBlock), 0, s, X, T, K, mask, chunk_pre, \
                       n_out, Xq, nd, row_zp, x_out, g.CB, g.SCB, g.zp, O, g.N, g.w_out,     \
                       xq_packed)
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
// Detection, compaction and the row quantization of the absmax kernels
// (kF8: their FP8 mode).
template <bool kF8>
hipError_t launch_act_absmax(const uint16_t *X, int64_t T, int64_t K, float threshold,
                             int8_t *Xq, float *a, int32_t *O, int32_t *n_out, uint8_t *partial,
                             uint8_t *mask, int32_t *chunk_pre, uint16_t *x_out,
                             const GatherArgs &g, bool xq_packed, hipStream_t s)
{
    if (xq_packed && T > 16)
        return hipErrorInvalidValue;
    const int64_t nchunk = K / 8;
    const int64_t rows_per = (T + kDetectSplits - 1) / kDetectSplits;
    const dim3 det_grid((unsigned)((nchunk + 31) / 32), (unsigned)kDetectSplits);
    hipLaunchKernelGGL(k_detect, det_grid, dim3(kDetectThreads), 0, s, X, T, K,
                       threshold_bits(threshold), rows_per, partial);
    hipLaunchKernelGGL(k_compact, dim3(1), dim3(kCompactThreads), 0, s, partial, K, mask, O, n_out,
                       chunk_pre);
    // w_out blocks: one wavefront per row when many columns are outliers; with
    // up to 32 a block covers 64 rows and the rest exit at once
    int64_t gather_blocks = 0;
    if (g.w_out) {
        gather_blocks = (g.N + kWavesPerBlock - 1) / kWavesPerBlock;
        if (gather_blocks > 2048)
            gather_blocks = 2048;
    }
    if (T >= kRowQuantWaveMinT && K <= kRowQuantWaveMaxK) {
        // a wavefront per row, the row in NC chunks per lane
        const int64_t per = (nchunk + kWave - 1) / kWave;
        const int64_t row_blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
        const dim3 grid((unsigned)(row_blocks + gather_blocks));
#define LLMINT8_ROWQUANT_W(NCV)                                                                  \
    hipLaunchKernelGGL((k_rowquant_w<NCV, kF8>), grid, dim3(kBlock), 0, s, X, T, K, mask, n_out, \
                       Xq, a,                                                            \
                       x_out, g.CB, g.SCB, O, g.N, g.w_out, row_blocks)
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
    // fewer rows: a block per row keeps more lanes busy
    const dim3 grid((unsigned)(T + gather_blocks));
    const int64_t chunks_per_thread = (nchunk + kBlock - 1) / kBlock;
#define LLMINT8_ROWQUANT(NCV)                                                                   \
    hipLaunchKernelGGL((k_rowquant<NCV, kF8>), grid, dim3(kBlock), 0, s, X, T, K, mask, chunk_pre, \
                       n_out,                                                           \
                       Xq, a, x_out, g.CB, g.SCB, O, g.N, g.w_out, xq_packed)
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
                               int8_t *Xq, float *a, int32_t *O, int32_t *n_out,
                               uint8_t *partial, uint8_t *mask, int32_t *chunk_pre,
                               uint16_t *x_out, const GatherArgs &g, bool xq_packed,
                               hipStream_t s)
{
    return launch_act_absmax<false>(X, T, K, threshold, Xq, a, O, n_out, partial, mask, chunk_pre,
                                    x_out, g, xq_packed, s);
}

hipError_t launch_quantize_weight_f8(const uint16_t *W_t, int64_t K, int64_t N, uint8_t *CB8,
                                     float *SC8, hipStream_t s)
{
    const int64_t blocks = (N + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(k_quantize_weight_f8, dim3((unsigned)blocks), dim3(kBlock), 0, s, W_t, K,
                       N, CB8, SC8);
    return hipGetLastError();
}

hipError_t launch_quantize_act_f8(const uint16_t *X, int64_t T, int64_t K, float threshold,
                                  uint8_t *Xq8, float *sc, int32_t *O, int32_t *n_out,
                                  uint8_t *partial, uint8_t *mask, int32_t *chunk_pre,
                                  uint16_t *x_out, const GatherArgs &g, bool xq_packed,
                                  hipStream_t s)
{
    if (g.w_out && !g.f8)
        return hipErrorInvalidValue;
    int8_t *Xq = reinterpret_cast<int8_t *>(Xq8);
    if (!g.w_out && quantize_act_fits_rows(T, K)) {
        // few rows: one launch (k_quant_rows in its FP8 mode)
        const int64_t per = (K / 8 + kSmallThreads - 1) / kSmallThreads;
        const unsigned tb = threshold_bits(threshold);
        const dim3 grid((unsigned)T);
#define LLMINT8_QROWS_F8(G)                                                                    \
    hipLaunchKernelGGL((k_quant_rows<G, kModeF8>), grid, dim3(kSmallThreads), 0, s, X, (int)T, \
                       (int)K, tb, Xq, sc, O, n_out, x_out, xq_packed, nullptr)
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
    return launch_act_absmax<true>(X, T, K, threshold, Xq, sc, O, n_out, partial, mask, chunk_pre,
                                   x_out, g, xq_packed, s);
}

}  // namespace llmint8
