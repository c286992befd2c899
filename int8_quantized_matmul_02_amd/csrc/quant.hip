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

__device__ __forceinline__ uint16_t half_at(uint4 v, int i)
{
    unsigned w = i < 2 ? v.x : i < 4 ? v.y : i < 6 ? v.z : v.w;
    return (uint16_t)((i & 1) ? (w >> 16) : (w & 0xffffu));
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
    for (int64_t c = lane; c < nchunk; c += kWave) {
        uint4 v = row[c];
        unsigned packed[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int q = amax > 0.0f ? quant127(h2f(half_at(v, i)), amax) : 0;
            packed[i >> 2] |= ((unsigned)q & 0xffu) << (8 * (i & 3));
        }
        dst[c] = make_uint2(packed[0], packed[1]);
    }
    if (lane == 0)
        SCB[n] = amax;
}

// ---------------------------------------------------------------------------
// Outlier-column detection.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_clear_flags(uint32_t *flags32, int64_t words)
{
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < words;
         i += (int64_t)gridDim.x * kBlock)
        flags32[i] = 0u;
}

constexpr int kDetectRows = 32;   // rows per block; each wavefront takes every 4th

// Block (x, y): columns [512x, 512x+512) (8 per lane), rows [32y, 32y+32).
// A column's flag is set to 1 when some |x| in it exceeds the threshold; many
// blocks may store the same 1, which is benign.
__global__ __launch_bounds__(kBlock) void k_detect(const uint16_t *__restrict__ X, int64_t T,
                                                   int64_t K, float threshold,
                                                   uint8_t *__restrict__ flags)
{
    const int lane = threadIdx.x % kWave;
    const int wy = threadIdx.x / kWave;
    const int64_t c8 = (int64_t)blockIdx.x * kWave + lane;   // 8-column chunk
    if (c8 * 8 >= K)
        return;
    unsigned m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // grid.y is capped, so row groups are taken in a grid-stride loop
    for (int64_t t0 = (int64_t)blockIdx.y * kDetectRows; t0 < T;
         t0 += (int64_t)gridDim.y * kDetectRows) {
        const int64_t t1 = t0 + kDetectRows < T ? t0 + kDetectRows : T;
        for (int64_t t = t0 + wy; t < t1; t += kWavesPerBlock) {
            uint4 v = *reinterpret_cast<const uint4 *>(X + t * K + c8 * 8);
            m[0] = umax(m[0], abs_lo(v.x));
            m[1] = umax(m[1], abs_hi(v.x));
            m[2] = umax(m[2], abs_lo(v.y));
            m[3] = umax(m[3], abs_hi(v.y));
            m[4] = umax(m[4], abs_lo(v.z));
            m[5] = umax(m[5], abs_hi(v.z));
            m[6] = umax(m[6], abs_lo(v.w));
            m[7] = umax(m[7], abs_hi(v.w));
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (h2f((uint16_t)m[i]) > threshold)
            flags[c8 * 8 + i] = 1;
}

constexpr int kCompactThreads = 1024;

// One block turns the flags into the ascending index list O, the count n and
// the column -> position map (colmap[k] = j for k = O[j], -1 otherwise).
__global__ __launch_bounds__(kCompactThreads) void k_compact(const uint8_t *__restrict__ flags,
                                                             int64_t K, int32_t *__restrict__ O,
                                                             int32_t *__restrict__ n_out,
                                                             int32_t *__restrict__ colmap)
{
    __shared__ int wave_tot[kCompactThreads / kWave];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int64_t per = (K + kCompactThreads - 1) / kCompactThreads;
    const int64_t k0 = tid * per < K ? tid * per : K;
    const int64_t k1 = k0 + per < K ? k0 + per : K;
    int cnt = 0;
    for (int64_t k = k0; k < k1; ++k)
        cnt += flags[k] != 0;
    // inclusive scan within the wavefront
    int inc = cnt;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int o = __shfl_up(inc, off, kWave);
        if (lane >= off)
            inc += o;
    }
    if (lane == kWave - 1)
        wave_tot[wave] = inc;
    __syncthreads();
    int base = inc - cnt;
    for (int w = 0; w < wave; ++w)
        base += wave_tot[w];
    int j = base;
    for (int64_t k = k0; k < k1; ++k) {
        if (flags[k]) {
            O[j] = (int32_t)k;
            colmap[k] = j;
            ++j;
        } else {
            colmap[k] = -1;
        }
    }
    if (tid == kCompactThreads - 1)
        *n_out = j;
}

// ---------------------------------------------------------------------------
// Row quantization: one wavefront per row t.  Pass 1 takes the absmax over
// the non-outlier columns, pass 2 (re-reading the row from cache) writes the
// int8 row with outlier columns as 0, and gathers the outlier values into the
// compact fp16 row x_out[t, colmap[k]] padded with zeros to a multiple of 32.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_rowquant(const uint16_t *__restrict__ X, int64_t T,
                                                     int64_t K, const uint8_t *__restrict__ flags,
                                                     const int32_t *__restrict__ colmap,
                                                     const int32_t *__restrict__ n_out,
                                                     int8_t *__restrict__ Xq,
                                                     float *__restrict__ a,
                                                     uint16_t *__restrict__ x_out)
{
    const int lane = threadIdx.x % kWave;
    const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    if (t >= T)
        return;
    const uint4 *xr = reinterpret_cast<const uint4 *>(X + t * K);
    const uint2 *fr = reinterpret_cast<const uint2 *>(flags);
    const int64_t nchunk = K / 8;
    unsigned m = 0;
    for (int64_t c = lane; c < nchunk; c += kWave) {
        uint4 v = xr[c];
        uint2 f = fr[c];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            unsigned fl = ((i < 4 ? f.x : f.y) >> (8 * (i & 3))) & 0xffu;
            if (!fl)
                m = umax(m, half_at(v, i) & 0x7fffu);
        }
    }
    m = wave_max_u32(m);
    const float amax = h2f((uint16_t)m);
    uint2 *dst = reinterpret_cast<uint2 *>(Xq + t * K);
    for (int64_t c = lane; c < nchunk; c += kWave) {
        uint4 v = xr[c];
        uint2 f = fr[c];
        unsigned packed[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            unsigned fl = ((i < 4 ? f.x : f.y) >> (8 * (i & 3))) & 0xffu;
            uint16_t h = half_at(v, i);
            int q = 0;
            if (fl) {
                if (x_out)
                    x_out[t * K + colmap[c * 8 + i]] = h;
            } else if (amax > 0.0f) {
                q = quant127(h2f(h), amax);
            }
            packed[i >> 2] |= ((unsigned)q & 0xffu) << (8 * (i & 3));
        }
        dst[c] = make_uint2(packed[0], packed[1]);
    }
    if (x_out) {
        const int n = *n_out;
        const int npad = (n + kOutlierPad - 1) / kOutlierPad * kOutlierPad;
        for (int j = n + lane; j < npad; j += kWave)
            x_out[t * K + j] = 0;
    }
    if (lane == 0)
        a[t] = amax;
}

// ---------------------------------------------------------------------------
// Dequantized outlier weight rows for the GEMM epilogue.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_gather_outlier_weights(
    const int8_t *__restrict__ CB, const float *__restrict__ SCB, const int32_t *__restrict__ O,
    const int32_t *__restrict__ n_out, int64_t K, int64_t N, uint16_t *__restrict__ w_out)
{
    const int lane = threadIdx.x % kWave;
    const int n = *n_out;
    const int npad = (n + kOutlierPad - 1) / kOutlierPad * kOutlierPad;
    for (int64_t r = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; r < N;
         r += (int64_t)gridDim.x * kWavesPerBlock) {
        const float s = SCB[r];
        for (int j = lane; j < npad; j += kWave)
            w_out[r * K + j] = j < n ? dequant_w(CB[r * K + O[j]], s) : (uint16_t)0;
    }
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

hipError_t launch_quantize_act(const uint16_t *X, int64_t T, int64_t K, float threshold,
                               int8_t *Xq, float *a, int32_t *O, int32_t *n_out,
                               uint8_t *flags, int32_t *colmap, uint16_t *x_out,
                               hipStream_t s)
{
    const int64_t words = K / 4;
    const int64_t clear_blocks = (words + kBlock - 1) / kBlock;
    hipLaunchKernelGGL(k_clear_flags, dim3((unsigned)clear_blocks), dim3(kBlock), 0, s,
                       reinterpret_cast<uint32_t *>(flags), words);
    int64_t det_y = (T + kDetectRows - 1) / kDetectRows;
    if (det_y > 65535)
        det_y = 65535;
    const dim3 det_grid((unsigned)((K / 8 + kWave - 1) / kWave), (unsigned)det_y);
    hipLaunchKernelGGL(k_detect, det_grid, dim3(kBlock), 0, s, X, T, K, threshold, flags);
    hipLaunchKernelGGL(k_compact, dim3(1), dim3(kCompactThreads), 0, s, flags, K, O, n_out,
                       colmap);
    const int64_t rq_blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(k_rowquant, dim3((unsigned)rq_blocks), dim3(kBlock), 0, s, X, T, K, flags,
                       colmap, n_out, Xq, a, x_out);
    return hipGetLastError();
}

hipError_t launch_gather_outlier_weights(const int8_t *CB, const float *SCB, const int32_t *O,
                                         const int32_t *n_out, int64_t K, int64_t N,
                                         uint16_t *w_out, hipStream_t s)
{
    int64_t blocks = (N + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks > 4096)
        blocks = 4096;
    hipLaunchKernelGGL(k_gather_outlier_weights, dim3((unsigned)blocks), dim3(kBlock), 0, s, CB,
                       SCB, O, n_out, K, N, w_out);
    return hipGetLastError();
}

}  // namespace llmint8
