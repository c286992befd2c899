// decode_kernel.h -- weight-streaming kernels for T <= 16 rows (the decode regime).
//
// With at most 16 activation rows the product is bound by reading CB once
// from HBM (K*N bytes against at most 16*K*N*2 int8 ops), so there is no
// output tiling to reuse: every wavefront owns 16 consecutive CB rows (16
// output columns) and streams them once, feeding the 16x16x64 int8 MFMA with
// the zero-padded activation rows as the other operand.  The k order inside
// an MFMA is irrelevant for the exact integer sum because both operands use
// the same lane -> k mapping.
//
// What decides the speed is the HBM access pattern.  A load instruction whose
// 64 lanes fetch 16 bytes from 16 different rows scatters 64-byte requests
// over 16 DRAM pages; here every load instruction fetches 1 KB contiguous
// from one CB row.  The MFMA, however, needs the 16 rows spread across lanes,
// so each stage is loaded into registers with 1 KB row-contiguous loads and
// transposed through a wavefront-private LDS buffer (k_decode_rs).  The
// 16-byte chunks of staged row r are XOR-swizzled by r, which makes both the
// 1 KB writes and the fragment reads (16 rows, one chunk each) hit distinct
// LDS banks.  Every wavefront synchronizes with nothing but its own
// loads (s_waitcnt).
//
// The epilogue is the decomposition of the LLM.int8() summary
// (kurtkim.github.io, sections "Vector-wise Quantization" and "The Core of
// LLM.int8(): Mixed-precision Decomposition"): dequantize by
// a[t]*SCB[n]/127^2, add the fp16 outlier product with the weight
// dequantized as CB*SCB/127 (agentlenshq.com write-up, Int8Params note) and
// the bias, round once to fp16.
#pragma once

#include <type_traits>
#include <utility>

#include "internal.h"

namespace llmint8 {
namespace decode {
namespace {   // internal linkage: nothing here is exported from the library

typedef __attribute__((address_space(3))) void lds_void;

template <int n>
__device__ __forceinline__ void wait_vm()
{
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

constexpr int kPrefetchOutliers = 8;

// Outlier weight bytes CB[n, O[j]] for the first kPrefetchOutliers outlier
// columns, fetched before the weight stream so their latency is hidden.
struct OutlierPrefetch {
    int nout;
    int8_t w[kPrefetchOutliers];
};

template <bool kRawI32>
__device__ __forceinline__ OutlierPrefetch prefetch_outliers(const int8_t *B, int64_t n, int64_t K,
                                                             const EpilogueArgs &ep)
{
    OutlierPrefetch p{};
    if constexpr (!kRawI32) {
        p.nout = *ep.n_out;
        // unconditional loads (O holds K >= 64 entries; unused ones read column 0)
#pragma unroll
        for (int j = 0; j < kPrefetchOutliers; ++j) {
            const int o = ep.O[j];
            p.w[j] = B[n * K + (j < p.nout ? o : 0)];
        }
    }
    return p;
}

// 16x16 accumulator layout: lane holds column n = n0 + lane%16 and rows
// t = 4*(lane/16) + q.
// Zero-point variant (kZp): ep.a and ep.scb hold nd of the rows and columns,
// and the integer part is the shifted sum C + zp_b*(rs_a + K*zp_a) +
// zp_a*rs_b, exact in wrapping 32-bit arithmetic (its true value fits int32),
// divided by nd_a*nd_b; the outlier weights are fp16((cb + zp_b)/nd_b).
// FP8 variant (kF8, the format): fp32 sums of the FP8 products, scaled by
// the row and column scales (powers of two); the outlier weights are
// fp16(code value * scale).
template <bool kRawI32, bool kRelu = false, bool kZp = false, int kF8 = kF8None>
__device__ __forceinline__ void epilogue(const std::conditional_t<kF8 != kF8None, v4f, v4i> acc,
                                         int lane,
                                         int64_t n, int64_t T, int64_t K, int64_t N,
                                         const int8_t *B, const EpilogueArgs &ep,
                                         const OutlierPrefetch &pre)
{
    const int t0 = 4 * (lane / 16);
    if constexpr (kRawI32) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (t0 + q < T)
                ep.c_i32[(t0 + q) * N + n] = acc[q];
    } else {
        const float sn = ep.scb[n];
        const float bias = ep.bias ? h2f(ep.bias[n]) : 0.0f;
        const int zb = kZp ? ep.zp_b[n] : 0;
        float v[4];
        if constexpr (kZp) {
            const float ib = zp_inv(sn);
            const unsigned rb = (unsigned)ep.rs_b[n];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t t = t0 + q < T ? t0 + q : T - 1;
                const int2 z = ep.row_zp[t];
                const unsigned ra = (unsigned)z.y + (unsigned)K * (unsigned)z.x;
                const unsigned c = (unsigned)acc[q] + (unsigned)zb * ra + (unsigned)z.x * rb;
                v[q] = (float)(int)c * (zp_inv(ep.a[t]) * ib);
            }
        } else {
            const float sn_d = kF8 ? sn : sn * (1.0f / 16129.0f);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t t = t0 + q < T ? t0 + q : T - 1;
                v[q] = (float)acc[q] * (ep.a[t] * sn_d);
            }
        }
        // Outlier columns in ascending order, kPrefetchOutliers at a time.  All
        // loads are unconditional so that none waits on its own: x_out rows
        // are zero-padded to a multiple of 32 >= o0 + kPrefetchOutliers, and
        // an unused slot gets weight 0.
        const int64_t ldo = outlier_ld(pre.nout);
        for (int o0 = 0; o0 < pre.nout; o0 += kPrefetchOutliers) {
            float w[kPrefetchOutliers];
#pragma unroll
            for (int j = 0; j < kPrefetchOutliers; ++j) {
                int cb = pre.w[j];
                if (o0 > 0) {
                    const int o = o0 + j < pre.nout ? ep.O[o0 + j] : 0;
                    cb = B[n * K + o];
                }
                uint16_t wd;
                if constexpr (kF8 != kF8None)
                    wd = dequant_w_f8<kF8>((unsigned)cb & 0xffu, sn);
                else if constexpr (kZp)
                    wd = dequant_w_zp(cb, zb, sn);
                else
                    wd = dequant_w(cb, sn);
                w[j] = o0 + j < pre.nout ? h2f(wd) : 0.0f;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t t = t0 + q < T ? t0 + q : T - 1;
                const uint16_t *xo = ep.x_out + t * ldo + o0;
#pragma unroll
                for (int j = 0; j < kPrefetchOutliers; ++j)
                    v[q] += h2f(xo[j]) * w[j];
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (t0 + q < T)
                ep.out[(t0 + q) * N + n] = f2h_act<kRelu>(v[q] + bias);
    }
}

// ---------------------------------------------------------------------------
// Register-staged: per stage a wavefront loads ROWB bytes of each of its 16
// rows (16*ROWB/1024 load instructions of 1 KB, 1024/ROWB rows each) into one
// of NB register buffers, writes the oldest buffer to its LDS stage and runs
// the MFMAs from there, then refills that buffer with stage c+NB.  NB-1
// stages stay in flight while one is consumed.  The activation fragments of
// a stage are issued NB-1 stages ahead too (NB-1 fragment buffers), right
// before the weights of the stage after it, so that one s_waitcnt per stage
// covers both without waiting for anything newer.
//
// Addresses: a load's base (weight block + stage + its first row) is
// wavefront-uniform and lives in scalar registers; each lane adds one fixed
// 32-bit offset.  The last stage is shifted back to end exactly at K and the
// k-steps it shares with the previous stage are left out of its MFMAs, so no
// load ever needs a per-lane bound.  Stages past the end (issued while the last
// ones are consumed) re-read the last stage's addresses and are never used:
// every pass issues the same loads, which keeps the compiler's own s_waitcnt
// placement exact.
// ---------------------------------------------------------------------------
template <int ROWB_, int WAVES_, int NB_ = 2, bool PACKED_A_ = false, int READ_GROUP_ = 8>
struct CfgRs {
    static constexpr int ROWB = ROWB_, WAVES = WAVES_, NB = NB_;
    // activations packed as [K/64][4][16][16]: k-step, 16-byte chunk, row, byte
    static constexpr bool kPackedA = PACKED_A_;
    // With packed activations every wavefront reads the same 1 KB fragment per
    // k-step; a barrier per stage keeps a block's wavefronts on the same stage
    // so that all but the first read it from the L1 cache instead of L2 (at
    // 16 rows the fragments are otherwise as much L2 traffic as the weights).
    // Needs every wavefront of a block active: N a multiple of 16 * WAVES.
    static constexpr bool kSync = PACKED_A_;
    static constexpr int kThreads = 64 * WAVES;
    static constexpr int kStage = 16 * ROWB;            // bytes per wavefront stage
    static constexpr int kRowsPerLoad = 1024 / ROWB;    // rows one 1 KB load instruction covers
    static constexpr int kLoads = 16 / kRowsPerLoad;    // load instructions per stage
    static constexpr int kSteps = ROWB / 64;            // 16x16x64 MFMA k-steps per stage
    static constexpr int kReadGroup = READ_GROUP_ < kSteps ? READ_GROUP_ : kSteps;
    static constexpr int NA = NB - 1;                   // activation fragment buffers
    static constexpr int kUnroll = NB * NA;             // lcm(NB, NB-1): buffer rotation period
    // loads younger than stage c's weights and activations when it is consumed
    static constexpr int kWait = (NB - 1) * kLoads + (NA - 1) * kSteps;
    static constexpr int kLdsBytes = WAVES * kStage;
    static_assert(NB >= 2 && NB <= 4, "register buffers");
    static_assert(ROWB >= 64 && 1024 % ROWB == 0, "stage shape");
    static_assert(kSteps % kReadGroup == 0, "read groups");
    static_assert(kWait < 64, "vmcnt range");
};

// One 16x16x32 FP8 MFMA on 8-byte fragments of format kFmt (fp8 = E4M3,
// bf8 = E5M2), fp32 accumulators.
template <int kFmt>
__device__ __forceinline__ v4f mfma_f8_16(long a, long b, v4f c)
{
    if constexpr (kFmt == kF8E4M3)
        return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf8_bf8(a, b, c, 0, 0, 0);
}

template <class C, bool kRawI32, bool kRelu = false, bool kZp = false, int kF8 = kF8None>
__global__ __launch_bounds__(C::kThreads) void k_decode_rs(const int8_t *__restrict__ A,
                                                           const int8_t *__restrict__ B,
                                                           int64_t T, int64_t K, int64_t N,
                                                           EpilogueArgs ep)
{
    __shared__ __attribute__((aligned(1024))) char smem[C::kLdsBytes];
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t n0 = ((int64_t)blockIdx.x * C::WAVES + wave) * 16;
    if (n0 >= N)
        return;   // whole wavefront: N is a multiple of 16 (never with kSync)
    const OutlierPrefetch pre = prefetch_outliers<kRawI32>(B, n0 + lane % 16, K, ep);
    char *wl = smem + wave * C::kStage;
    const int8_t *bw = B + n0 * K;
    const int r = lane % 16, g = lane / 16;
    const int8_t *pa = A + (r < T ? r : T - 1) * K + 16 * g;
    const int kk = (int)K;   // K <= 133144: every in-block offset fits 32 bits
    const int nch = (kk + C::ROWB - 1) / C::ROWB;

    // Piece m of a stage (one load instruction): lane l holds row
    // m*kRowsPerLoad + lrow, bytes [lcol, lcol+16) of the stage's k range;
    // in LDS, row i keeps its 16-byte chunk q at i*ROWB + 16*(q ^ (i & 15)).
    const int lrow = (16 * lane) / C::ROWB, lcol = (16 * lane) % C::ROWB;
    const int lane_off = lrow * kk + lcol;
    auto lds_off = [&](int m) {
        const int row = m * C::kRowsPerLoad + lrow;
        return row * C::ROWB + 16 * ((lcol / 16) ^ (row & 15));
    };
    // First k of the stage consumed c-th.  Each block takes the stages before
    // the last in a rotated order, starting at stage blockIdx % (nch - 1):
    // when every wavefront reads the same k window of its rows (rows K bytes
    // apart) the requests crowd a few HBM channels, rotated they spread (on
    // the 12288 x 49152 weight: 71 % -> 80 % of the HBM peak).  The int32
    // sums do not depend on the order.  The last stage stays last; it ends at
    // K (K >= ROWB), and so does any stage past it.
    const int nrot = nch > 1 ? nch - 1 : 1;
    const int rot = (int)(blockIdx.x % (unsigned)nrot);
    auto stage_k = [&](int c) {
        const int p = c >= nch - 1 ? nch - 1 : c + rot < nrot ? c + rot : c + rot - nrot;
        return min(p * C::ROWB, kk - C::ROWB);
    };

    const v4i zero = v4i{0, 0, 0, 0};
    auto load_b = [&](v4i(&R)[C::kLoads], int c) {
        const int kc = stage_k(c);
#pragma unroll
        for (int m = 0; m < C::kLoads; ++m) {
            const int8_t *sp = bw + (int64_t)(m * C::kRowsPerLoad) * K + kc;
            R[m] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(sp + lane_off));
        }
    };
    auto store_b = [&](const v4i(&R)[C::kLoads]) {
#pragma unroll
        for (int m = 0; m < C::kLoads; ++m)
            *reinterpret_cast<v4i *>(wl + lds_off(m)) = R[m];
    };
    // Activation fragments: lane (r, g) holds row r, chunk g of each 64-byte
    // k-step.  Rows r >= T read row T-1: an MFMA output row depends only on
    // its own activation row, and rows >= T are never stored.  No value is
    // masked after its load, so no load waits on its own.
    auto load_a = [&](v4i(&a)[C::kSteps], int c) {
        const int kc = stage_k(c);
#pragma unroll
        for (int s2 = 0; s2 < C::kSteps; ++s2) {
            if constexpr (C::kPackedA)
                a[s2] = *reinterpret_cast<const v4i *>(A + (kc + 64 * s2) * 16 + 16 * lane);
            else
                a[s2] = *reinterpret_cast<const v4i *>(pa + kc + 64 * s2);
        }
    };
    std::conditional_t<kF8 != kF8None, v4f, v4i> acc = {0, 0, 0, 0};
    // Fragment reads in groups of kReadGroup, each group issued before its
    // MFMAs (each MFMA waits only for its own read).  The first `skip` bytes
    // of the last stage were already summed by the previous stage: their
    // k-steps (skip is a multiple of 64) are left out by a uniform test.
    auto compute = [&](const v4i(&a)[C::kSteps], int skip) {
        const char *src = wl + r * C::ROWB;
#pragma unroll
        for (int s0 = 0; s0 < C::kSteps; s0 += C::kReadGroup) {
            v4i b[C::kReadGroup];
#pragma unroll
            for (int i = 0; i < C::kReadGroup; ++i)
                b[i] = *reinterpret_cast<const v4i *>(src + (((4 * (s0 + i) + g) ^ r) * 16));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < C::kReadGroup; ++i)
                if (64 * (s0 + i) >= skip) {
                    if constexpr (kF8 != kF8None) {
                        // FP8: two 16x16x32 MFMAs, the low and the high 8
                        // bytes of both fragments (the same k's in both)
                        const v4i x = a[s0 + i], y = b[i];
                        acc = mfma_f8_16<kF8>(((long)(unsigned)x[1] << 32) | (unsigned)x[0],
                                              ((long)(unsigned)y[1] << 32) | (unsigned)y[0], acc);
                        acc = mfma_f8_16<kF8>(((long)(unsigned)x[3] << 32) | (unsigned)x[2],
                                              ((long)(unsigned)y[3] << 32) | (unsigned)y[2], acc);
                    } else {
                        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[s0 + i], b[i], acc, 0, 0, 0);
                    }
                }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    v4i R[C::NB][C::kLoads];
    v4i a[C::NA][C::kSteps];
    if (nch == 1) {
        // K <= ROWB: bytes past K come from column 0 of the row and are
        // stored as zeros; activation addresses past K are clamped likewise
#pragma unroll
        for (int m = 0; m < C::kLoads; ++m) {
            const int8_t *sp = bw + (int64_t)(m * C::kRowsPerLoad) * K;
            R[0][m] = *reinterpret_cast<const v4i *>(sp + lrow * kk + (lcol < kk ? lcol : 0));
        }
#pragma unroll
        for (int s2 = 0; s2 < C::kSteps; ++s2) {
            const int k = 64 * s2 < kk ? 64 * s2 : 0;
            if constexpr (C::kPackedA)
                a[0][s2] = *reinterpret_cast<const v4i *>(A + k * 16 + 16 * lane);
            else
                a[0][s2] = *reinterpret_cast<const v4i *>(pa + k);
        }
        wait_vm<0>();
#pragma unroll
        for (int m = 0; m < C::kLoads; ++m)
            *reinterpret_cast<v4i *>(wl + lds_off(m)) = lcol < kk ? R[0][m] : zero;
        compute(a[0], 0);
    } else {
        // Issue order, oldest first, when stage c is consumed:
        //   R(c) a(c) R(c+1) a(c+1) ... R(c+NB-2) a(c+NB-2) R(c+NB-1)
        // Step c waits for R(c) and a(c), stores and consumes them, then
        // issues a(c+NB-1) into a(c)'s buffer and R(c+NB) into R(c)'s.
        // The phases stay in this order (sched_barrier): hoisting the next
        // loads above the LDS stores would need another set of registers.
#pragma unroll
        for (int j = 0; j < C::NB; ++j) {
            load_b(R[j], j);
            if (j < C::NA)
                load_a(a[j], j);
        }
        // step u of a rotation period (buffer indices are compile-time); only
        // the final stage can overlap the one before it
        auto step = [&]<int u, bool kLast>(std::integral_constant<int, u>,
                                           std::bool_constant<kLast>, int cc) {
            if constexpr (C::kSync)
                __builtin_amdgcn_s_barrier();
            wait_vm<C::kWait>();
            store_b(R[u % C::NB]);
            __builtin_amdgcn_sched_barrier(0);
            compute(a[u % C::NA], kLast ? cc * C::ROWB - stage_k(cc) : 0);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (!kLast) {
                load_a(a[u % C::NA], cc + C::NA);
                load_b(R[u % C::NB], cc + C::NB);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        auto steps = [&]<int... U>(std::integer_sequence<int, U...>, int c0, auto last) {
            constexpr int n = sizeof...(U);
            (step(std::integral_constant<int, U>{},
                  std::bool_constant<decltype(last)::value && U + 1 == n>{}, c0 + U),
             ...);
        };
        // Whole rotation periods in a single-exit loop that leaves 1 to
        // kUnroll stages, then those as one straight-line sequence picked by
        // their count: every block is entered with the same loads in flight,
        // which keeps the compiler's own s_waitcnt placement exact.
        int c = 0;
        for (; c + C::kUnroll < nch; c += C::kUnroll)
            steps(std::make_integer_sequence<int, C::kUnroll>{}, c, std::false_type{});
        const int rem = nch - c;
        [&]<int... Q>(std::integer_sequence<int, Q...>) {
            ((rem == Q + 1
                  ? (steps(std::make_integer_sequence<int, Q + 1>{}, c, std::true_type{}), 0)
                  : 0),
             ...);
        }(std::make_integer_sequence<int, C::kUnroll>{});
    }
    epilogue<kRawI32, kRelu, kZp, kF8>(acc, lane, n0 + lane % 16, T, K, N, B, ep, pre);
}

template <class C, bool R, bool kRelu = false, bool kZp = false, int kF8 = kF8None>
struct RsKernel {
    static constexpr auto fn = k_decode_rs<C, R, kRelu, kZp, kF8>;
};
template <class C, bool R>
using RsKernelF8 = RsKernel<C, R, false, false, kF8E5M2>;
template <class C, bool R>
using RsKernelF8E4 = RsKernel<C, R, false, false, kF8E4M3>;
template <class C, bool R>
using RsKernelRelu = RsKernel<C, R, true>;
template <class C, bool R>
using RsKernelZp = RsKernel<C, R, false, true>;
// One block per C::WAVES * 16 output columns.
template <class C, template <class, bool> class Kernel>
hipError_t launch_kernel(const int8_t *Xq, const int8_t *CB, int64_t T, int64_t K, int64_t N,
                         const EpilogueArgs &ep, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1)
{
    const int64_t blocks = (N + C::WAVES * 16 - 1) / (C::WAVES * 16);
    if (ev0) {
        const hipError_t e = hipEventRecord(ev0, s);
        if (e != hipSuccess)
            return e;
    }
    if (ep.c_i32)
        hipLaunchKernelGGL((Kernel<C, true>::fn), dim3((unsigned)blocks), dim3(C::kThreads), 0, s,
                           Xq, CB, T, K, N, ep);
    else
        hipLaunchKernelGGL((Kernel<C, false>::fn), dim3((unsigned)blocks), dim3(C::kThreads), 0,
                           s, Xq, CB, T, K, N, ep);
    if (ev1) {
        const hipError_t e = hipEventRecord(ev1, s);
        if (e != hipSuccess)
            return e;
    }
    return hipGetLastError();
}

template <class C>
hipError_t launch_rs(const int8_t *Xq, const int8_t *CB, int64_t T, int64_t K, int64_t N,
                     const EpilogueArgs &ep, hipStream_t s, hipEvent_t ev0 = nullptr,
                     hipEvent_t ev1 = nullptr)
{
    if (C::kSync && N % (16 * C::WAVES) != 0)
        return hipErrorInvalidValue;   // a block's wavefronts must all reach the barriers
    if (ep.f8 == kF8E4M3 && !ep.c_i32)
        return launch_kernel<C, RsKernelF8E4>(Xq, CB, T, K, N, ep, s, ev0, ev1);
    if (ep.f8 && !ep.c_i32)
        return launch_kernel<C, RsKernelF8>(Xq, CB, T, K, N, ep, s, ev0, ev1);
    if (ep.row_zp && !ep.c_i32)
        return launch_kernel<C, RsKernelZp>(Xq, CB, T, K, N, ep, s, ev0, ev1);
    if (ep.act && !ep.c_i32)
        return launch_kernel<C, RsKernelRelu>(Xq, CB, T, K, N, ep, s, ev0, ev1);
    return launch_kernel<C, RsKernel>(Xq, CB, T, K, N, ep, s, ev0, ev1);
}

}  // namespace
}  // namespace decode
}  // namespace llmint8
