// decode_kernel.h -- weight-streaming kernel for T <= 16 rows (the decode regime).
//
// With at most 16 activation rows the product is bound by reading CB once
// from HBM (K*N bytes against at most 16*K*N*2 int8 ops), so there is no
// output tiling to reuse.  Each wavefront owns 16*NT output columns and
// streams their CB rows with 16-byte non-temporal loads, UNROLL 64-byte
// k-steps in flight, feeding the 16x16x64 int8 MFMA with the zero-padded
// activation rows as the other operand (one activation fragment serves NT
// MFMAs).  The k order inside an MFMA is irrelevant for the exact integer sum
// because both operands use the same lane -> k mapping.
//
// The epilogue is the decomposition of the LLM.int8() summary
// (kurtkim.github.io, sections "Vector-wise Quantization" and "The Core of
// LLM.int8(): Mixed-precision Decomposition"): dequantize by
// a[t]*SCB[n]/127^2, add the fp16 outlier product with the weight
// dequantized as CB*SCB/127 (agentlenshq.com write-up, Int8Params note) and
// the bias, round once to fp16.
#pragma once

#include "internal.h"

namespace llmint8 {
namespace decode {
namespace {   // internal linkage: nothing here is exported from the library

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <int NT_, int UNROLL_>
struct Cfg {
    static constexpr int NT = NT_, UNROLL = UNROLL_;
    static constexpr int kCols = 16 * NT;   // output columns per wavefront
};

template <class C, bool kRawI32>
__global__ __launch_bounds__(kThreads) void k_decode(const int8_t *__restrict__ A,
                                                     const int8_t *__restrict__ B, int64_t T,
                                                     int64_t K, int64_t N, EpilogueArgs ep)
{
    const int lane = threadIdx.x % kWave;
    const int64_t n0 = ((int64_t)blockIdx.x * kWaves + threadIdx.x / kWave) * C::kCols;
    if (n0 >= N)
        return;
    const int r = lane % 16, kb = (lane / 16) * 16;
    const bool arow = r < T;
    const int8_t *pa = A + (arow ? r : 0) * K + kb;
    const int8_t *pb[C::NT];
#pragma unroll
    for (int j = 0; j < C::NT; ++j) {
        int64_t row = n0 + j * 16 + r;
        row = row < N ? row : N - 1;   // a partial last group (N % kCols) reads row N-1, stores masked
        pb[j] = B + row * K + kb;
    }
    v4i acc[C::NT];
#pragma unroll
    for (int j = 0; j < C::NT; ++j)
        acc[j] = v4i{0, 0, 0, 0};
    const v4i zero = v4i{0, 0, 0, 0};
    int64_t k = 0;
    for (; k + 64 * C::UNROLL <= K; k += 64 * C::UNROLL) {
        v4i b[C::UNROLL][C::NT], a[C::UNROLL];
#pragma unroll
        for (int u = 0; u < C::UNROLL; ++u)
#pragma unroll
            for (int j = 0; j < C::NT; ++j)
                b[u][j] = __builtin_nontemporal_load(
                    reinterpret_cast<const v4i *>(pb[j] + k + 64 * u));
#pragma unroll
        for (int u = 0; u < C::UNROLL; ++u)
            a[u] = arow ? *reinterpret_cast<const v4i *>(pa + k + 64 * u) : zero;
#pragma unroll
        for (int u = 0; u < C::UNROLL; ++u)
#pragma unroll
            for (int j = 0; j < C::NT; ++j)
                acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u], b[u][j], acc[j], 0, 0, 0);
    }
    for (; k < K; k += 64) {
        const v4i a = arow ? *reinterpret_cast<const v4i *>(pa + k) : zero;
#pragma unroll
        for (int j = 0; j < C::NT; ++j) {
            const v4i b = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(pb[j] + k));
            acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[j], 0, 0, 0);
        }
    }

    // 16x16 accumulator layout: lane holds column lane%16, rows 4*(lane/16) + q.
#pragma unroll
    for (int j = 0; j < C::NT; ++j) {
        const int64_t n = n0 + j * 16 + lane % 16;
        if (n >= N)
            continue;
        if constexpr (kRawI32) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t t = 4 * (lane / 16) + q;
                if (t < T)
                    ep.c_i32[t * N + n] = acc[j][q];
            }
        } else {
            const float sn = ep.scb[n];
            const float sn_d = sn * (1.0f / 16129.0f);
            const int nout = *ep.n_out;
            const float bias = ep.bias ? h2f(ep.bias[n]) : 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t t = 4 * (lane / 16) + q;
                if (t >= T)
                    continue;
                float v = (float)acc[j][q] * (ep.a[t] * sn_d);
                for (int o = 0; o < nout; ++o)
                    v += h2f(ep.x_out[t * K + o]) * h2f(dequant_w(B[n * K + ep.O[o]], sn));
                ep.out[t * N + n] = f2h(v + bias);
            }
        }
    }
}

template <class C>
hipError_t launch(const int8_t *Xq, const int8_t *CB, int64_t T, int64_t K, int64_t N,
                  const EpilogueArgs &ep, hipStream_t s, hipEvent_t ev0 = nullptr,
                  hipEvent_t ev1 = nullptr)
{
    const int64_t blocks = (N + kWaves * C::kCols - 1) / (kWaves * C::kCols);
    if (ev0) {
        const hipError_t e = hipEventRecord(ev0, s);
        if (e != hipSuccess)
            return e;
    }
    if (ep.c_i32)
        hipLaunchKernelGGL((k_decode<C, true>), dim3((unsigned)blocks), dim3(kThreads), 0, s, Xq,
                           CB, T, K, N, ep);
    else
        hipLaunchKernelGGL((k_decode<C, false>), dim3((unsigned)blocks), dim3(kThreads), 0, s, Xq,
                           CB, T, K, N, ep);
    if (ev1) {
        const hipError_t e = hipEventRecord(ev1, s);
        if (e != hipSuccess)
            return e;
    }
    return hipGetLastError();
}


// ---------------------------------------------------------------------------
// LDS-staged variant.  A load instruction whose 64 lanes fetch 16 bytes of
// 16 different rows turns into 64-byte requests scattered over 16 DRAM pages;
// here every load instruction instead fetches 1 KB contiguous from one CB row
// straight into LDS (global_load_lds), and the MFMA fragments are read back
// from LDS.  Each wavefront stages only its own 16 rows (16 KB per stage), so
// it synchronizes with nothing but its own loads (s_waitcnt).  The 16-byte
// chunks of staged row r are XOR-swizzled by r, which makes the fragment
// reads (16 rows, one chunk each) hit distinct LDS banks.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

template <int n>
__device__ __forceinline__ void wait_vm()
{
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ROWBYTES of each of a wavefront's 16 CB rows per stage, STAGES stages per
// wavefront, WAVES wavefronts per block.
template <int STAGES_, int ROWBYTES_, int WAVES_>
struct CfgLds {
    static constexpr int STAGES = STAGES_, ROWBYTES = ROWBYTES_, WAVES = WAVES_;
    static constexpr int kThreads = 64 * WAVES;
    static constexpr int kCols = 16;
    static constexpr int kStageWave = 16 * ROWBYTES;
    static constexpr int kLoads = kStageWave / 1024;    // 1 KB load instructions per stage
    static constexpr int kSteps = ROWBYTES / 64;        // 16x16x64 MFMA k-steps per stage
    static constexpr int kLdsBytes = WAVES * STAGES * kStageWave;
    static_assert(ROWBYTES >= 256 && ROWBYTES % 256 == 0 && kLoads >= 1, "stage shape");
    static_assert((STAGES - 1) * kLoads + kSteps < 64, "vmcnt range");
};

template <class C, bool kRawI32>
__global__ __launch_bounds__(C::kThreads) void k_decode_lds(const int8_t *__restrict__ A,
                                                            const int8_t *__restrict__ B,
                                                            int64_t T, int64_t K, int64_t N,
                                                            EpilogueArgs ep)
{
    __shared__ __attribute__((aligned(1024))) char smem[C::kLdsBytes];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int64_t n0 = ((int64_t)blockIdx.x * C::WAVES + wave) * 16;
    if (n0 >= N)
        return;   // whole wavefront: N is a multiple of 16
    char *wl = smem + wave * C::STAGES * C::kStageWave;
    const int r = lane % 16, g = lane / 16;
    const bool arow = r < T;
    const int8_t *pa = A + (arow ? r : 0) * K + 16 * g;
    const int64_t nchunks = (K + C::ROWBYTES - 1) / C::ROWBYTES;
    // Stage c holds bytes [c*ROWBYTES, (c+1)*ROWBYTES) of the wavefront's 16
    // rows, row i at offset i*ROWBYTES, its 16-byte chunk q in slot q ^ i.
    // Load instruction m fills the m-th KB: lane l lands at byte m*1024 + 16*l.
    const int8_t *rowp[C::kLoads];
    int col[C::kLoads];
#pragma unroll
    for (int m = 0; m < C::kLoads; ++m) {
        const int byte = m * 1024 + 16 * lane;
        const int row = byte / C::ROWBYTES, slot = (byte % C::ROWBYTES) / 16;
        rowp[m] = B + (n0 + row) * K;
        col[m] = 16 * (slot ^ (row & 15));
    }
    auto issue = [&](int64_t c) {
        const int kc = (int)(c * C::ROWBYTES);
        char *dst = wl + (c % C::STAGES) * C::kStageWave;
#pragma unroll
        for (int m = 0; m < C::kLoads; ++m) {
            // past the end of a row: a harmless address inside it, never read back
            const int off = kc + col[m] < K ? kc + col[m] : 0;
            __builtin_amdgcn_global_load_lds((const void *)(rowp[m] + off),
                                             (lds_void *)(dst + m * 1024), 16, 0, 0);
        }
    };
    v4i acc = v4i{0, 0, 0, 0};
    const v4i zero = v4i{0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < C::STAGES - 1; ++c)
        if (c < nchunks)
            issue(c);
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t kc = c * C::ROWBYTES;
        const int steps = K - kc >= C::ROWBYTES ? C::kSteps : (int)((K - kc) / 64);
        v4i a[C::kSteps];
#pragma unroll
        for (int s2 = 0; s2 < C::kSteps; ++s2)
            a[s2] = (arow && s2 < steps) ? *reinterpret_cast<const v4i *>(pa + kc + 64 * s2) : zero;
        if (c + C::STAGES - 1 < nchunks) {
            issue(c + C::STAGES - 1);
            // stage c landed; the newer stages and the a[] loads may still be in flight
            wait_vm<(C::STAGES - 1) * C::kLoads + C::kSteps>();
        } else {
            wait_vm<C::kSteps>();   // a[] loads are the newest; everything older has landed
        }
        const char *src = wl + (c % C::STAGES) * C::kStageWave + r * C::ROWBYTES;
#pragma unroll
        for (int s2 = 0; s2 < C::kSteps; ++s2) {
            if (s2 < steps) {
                const v4i b = *reinterpret_cast<const v4i *>(src + (((4 * s2 + g) ^ r) * 16));
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[s2], b, acc, 0, 0, 0);
            }
        }
    }

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
        const float bias = ep.bias ? h2f(ep.bias[n]) : 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t t = 4 * (lane / 16) + q;
            if (t >= T)
                continue;
            float v = (float)acc[q] * (ep.a[t] * sn_d);
            for (int o = 0; o < nout; ++o)
                v += h2f(ep.x_out[t * K + o]) * h2f(dequant_w(B[n * K + ep.O[o]], sn));
            ep.out[t * N + n] = f2h(v + bias);
        }
    }
}

template <class C>
hipError_t launch_lds(const int8_t *Xq, const int8_t *CB, int64_t T, int64_t K, int64_t N,
                      const EpilogueArgs &ep, hipStream_t s, hipEvent_t ev0 = nullptr,
                      hipEvent_t ev1 = nullptr)
{
    const int64_t blocks = (N + C::WAVES * 16 - 1) / (C::WAVES * 16);
    if (ev0) {
        const hipError_t e = hipEventRecord(ev0, s);
        if (e != hipSuccess)
            return e;
    }
    if (ep.c_i32)
        hipLaunchKernelGGL((k_decode_lds<C, true>), dim3((unsigned)blocks), dim3(C::kThreads), 0,
                           s, Xq, CB, T, K, N, ep);
    else
        hipLaunchKernelGGL((k_decode_lds<C, false>), dim3((unsigned)blocks), dim3(C::kThreads), 0,
                           s, Xq, CB, T, K, N, ep);
    if (ev1) {
        const hipError_t e = hipEventRecord(ev1, s);
        if (e != hipSuccess)
            return e;
    }
    return hipGetLastError();
}

}  // namespace
}  // namespace decode
}  // namespace llmint8
