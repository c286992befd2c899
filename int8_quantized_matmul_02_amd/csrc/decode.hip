// decode.hip -- weight-streaming kernel for T <= 16 rows (the decode regime).
//
// With at most 16 activation rows the product is bound by reading CB once
// from HBM (K*N bytes against at most 16*K*N*2 int8 ops), so there is no
// output tiling to reuse: each wavefront owns 16 output columns, streams their
// CB rows with 16-byte loads and feeds them to the 16x16x64 int8 MFMA with the
// (zero-padded) activation rows as the other operand.  The epilogue is the
// same decomposition as the tiled GEMM (LLM.int8() summary, kurtkim.github.io,
// sections "Vector-wise Quantization" and "The Core of LLM.int8():
// Mixed-precision Decomposition"): dequantize by a[t]*SCB[n]/127^2, add the
// fp16 outlier product with the weight dequantized as CB*SCB/127 (agentlenshq
// write-up, Int8Params note) and the bias, round once to fp16.

#include "internal.h"

namespace llmint8 {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kCols = 16;        // output columns per wavefront
constexpr int kUnroll = 4;       // 64-byte k-steps per loop trip

template <bool kRawI32>
__global__ __launch_bounds__(kThreads) void k_decode(const int8_t *__restrict__ A,
                                                     const int8_t *__restrict__ B, int64_t T,
                                                     int64_t K, int64_t N, EpilogueArgs ep)
{
    const int lane = threadIdx.x % kWave;
    const int64_t n0 = ((int64_t)blockIdx.x * kWaves + threadIdx.x / kWave) * kCols;
    if (n0 >= N)
        return;
    const int r = lane % 16, kb = (lane / 16) * 16;
    const int8_t *pb = B + (n0 + r) * K + kb;
    const bool arow = r < T;
    const int8_t *pa = A + (arow ? r : 0) * K + kb;
    v4i acc = v4i{0, 0, 0, 0};
    const v4i zero = v4i{0, 0, 0, 0};
    int64_t k = 0;
    for (; k + 64 * kUnroll <= K; k += 64 * kUnroll) {
        v4i b[kUnroll], a[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            b[u] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(pb + k + 64 * u));
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            a[u] = arow ? *reinterpret_cast<const v4i *>(pa + k + 64 * u) : zero;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u], b[u], acc, 0, 0, 0);
    }
    for (; k < K; k += 64) {
        v4i b = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(pb + k));
        v4i a = arow ? *reinterpret_cast<const v4i *>(pa + k) : zero;
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc, 0, 0, 0);
    }

    // 16x16 accumulator layout: lane holds column lane%16, rows 4*(lane/16) + q.
    const int64_t n = n0 + lane % 16;
    if constexpr (kRawI32) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t t = 4 * (lane / 16) + q;
            if (t < T)
                ep.c_i32[t * N + n] = acc[q];
        }
    } else {
        const float sn = ep.scb[n];
        const float sn_d = sn * (1.0f / 16129.0f);
        const int nout = *ep.n_out;
        const float b = ep.bias ? h2f(ep.bias[n]) : 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t t = 4 * (lane / 16) + q;
            if (t >= T)
                continue;
            float v = (float)acc[q] * (ep.a[t] * sn_d);
            for (int j = 0; j < nout; ++j)
                v += h2f(ep.x_out[t * K + j]) * h2f(dequant_w(B[n * K + ep.O[j]], sn));
            ep.out[t * N + n] = f2h(v + b);
        }
    }
}

}  // namespace

hipError_t launch_decode(const int8_t *Xq, const int8_t *CB, int64_t T, int64_t K, int64_t N,
                         const EpilogueArgs &ep, hipStream_t s)
{
    const int64_t blocks = (N + kWaves * kCols - 1) / (kWaves * kCols);
    if (ep.c_i32)
        hipLaunchKernelGGL(k_decode<true>, dim3((unsigned)blocks), dim3(kThreads), 0, s, Xq, CB, T,
                           K, N, ep);
    else
        hipLaunchKernelGGL(k_decode<false>, dim3((unsigned)blocks), dim3(kThreads), 0, s, Xq, CB,
                           T, K, N, ep);
    return hipGetLastError();
}

}  // namespace llmint8
