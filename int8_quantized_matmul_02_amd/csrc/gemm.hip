// gemm.hip -- tiled int8 MFMA GEMM with the fused LLM.int8() epilogue.
//
// C[t,n] = sum_k Xq[t,k] * CB[n,k] accumulates exactly in int32 (LLM.int8()
// summary, kurtkim.github.io, section "Int8 Matrix Multiplication with 16-bit
// Float Inputs and Outputs").  The epilogue dequantizes by the outer product
// of the row and column scales, a[t] * SCB[n] / 127^2 (section "Vector-wise
// Quantization"), adds the fp16 product of the outlier columns of X with the
// matching dequantized weight rows and the bias, and rounds once to fp16
// (section "The Core of LLM.int8(): Mixed-precision Decomposition"; the
// agentlenshq.com write-up, "Core idea" step 3).
//
// Both operands are K-contiguous ([T,K] and [N,K]), so the MFMA A and B
// fragments are the same shape: each lane reads 16 consecutive bytes of one
// row.  The k order inside one MFMA does not matter for an exact integer sum
// as long as A and B use the same lane -> k mapping, which they do here.

#include "internal.h"

namespace llmint8 {
namespace {

constexpr int kThreads = 256;          // 4 wavefronts, 2 x 2 over the tile
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kLds = BK + 16;          // padded LDS row stride (bytes): conflict-free 16-B reads
constexpr int kChunksPerThread = BM * BK / 16 / kThreads;   // 16-byte chunks per operand

template <bool kRawI32>
__global__ __launch_bounds__(kThreads) void k_gemm(const int8_t *__restrict__ A,
                                                   const int8_t *__restrict__ B, int64_t T,
                                                   int64_t K, int64_t N, EpilogueArgs ep)
{
    __shared__ __attribute__((aligned(16))) int8_t sA[BM * kLds];
    __shared__ __attribute__((aligned(16))) int8_t sB[BN * kLds];

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;

    // global -> LDS assignment: chunk c covers row c/4, bytes (c%4)*16 .. +16
    const int8_t *gA[kChunksPerThread];
    const int8_t *gB[kChunksPerThread];
    int sOff[kChunksPerThread];
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
        const int c = tid + u * kThreads;
        const int row = c / (BK / 16), col = (c % (BK / 16)) * 16;
        const int64_t ar = m0 + row < T ? m0 + row : T - 1;   // ragged T: clamp, store masked
        const int64_t br = n0 + row < N ? n0 + row : N - 1;
        gA[u] = A + ar * K + col;
        gB[u] = B + br * K + col;
        sOff[u] = row * kLds + col;
    }

    v16i acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

    v4i ra[kChunksPerThread], rb[kChunksPerThread];
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
        ra[u] = *reinterpret_cast<const v4i *>(gA[u]);
        rb[u] = *reinterpret_cast<const v4i *>(gB[u]);
    }

    const int frag_row = lane % 32, frag_k = (lane / 32) * 16;
    for (int64_t k0 = 0; k0 < K; k0 += BK) {
        __syncthreads();   // every wavefront is done reading the previous tile
#pragma unroll
        for (int u = 0; u < kChunksPerThread; ++u) {
            *reinterpret_cast<v4i *>(sA + sOff[u]) = ra[u];
            *reinterpret_cast<v4i *>(sB + sOff[u]) = rb[u];
        }
        __syncthreads();
        if (k0 + BK < K) {   // prefetch the next tile into registers while computing
#pragma unroll
            for (int u = 0; u < kChunksPerThread; ++u) {
                ra[u] = *reinterpret_cast<const v4i *>(gA[u] + k0 + BK);
                rb[u] = *reinterpret_cast<const v4i *>(gB[u] + k0 + BK);
            }
        }
#pragma unroll
        for (int s = 0; s < BK / 32; ++s) {
            v4i fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                fa[i] = *reinterpret_cast<const v4i *>(
                    sA + (wm * 64 + i * 32 + frag_row) * kLds + s * 32 + frag_k);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                fb[j] = *reinterpret_cast<const v4i *>(
                    sB + (wn * 64 + j * 32 + frag_row) * kLds + s * 32 + frag_k);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] =
                        __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
    }

    // 32x32 accumulator layout: lane holds column lane%32 and, for register r,
    // row 8*(r/4) + 4*(lane/32) + r%4 of its 32x32 sub-tile.
    const int col_in = lane % 32, row_in = 4 * (lane / 32);
    if constexpr (kRawI32) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t t = m0 + wm * 64 + i * 32 + 8 * (r / 4) + row_in + (r % 4);
                    const int64_t n = n0 + wn * 64 + j * 32 + col_in;
                    if (t < T && n < N)
                        ep.c_i32[t * N + n] = acc[i][j][r];
                }
        return;
    } else {
        // dequantize: C * a[t] * SCB[n] / 127^2, in fp32
        v16f accf[2][2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t n = n0 + wn * 64 + j * 32 + col_in;
            const float sn = ep.scb[n < N ? n : N - 1] * (1.0f / 16129.0f);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    int64_t t = m0 + wm * 64 + i * 32 + 8 * (r / 4) + row_in + (r % 4);
                    t = t < T ? t : T - 1;
                    accf[i][j][r] = (float)acc[i][j][r] * (ep.a[t] * sn);
                }
        }
        // fp16 outlier product on fp16 MFMA, accumulated onto the dequantized values.
        const int nout = *ep.n_out;
        const int nchunks = (nout + 15) / 16;
        const int hk = (lane / 32) * 8;
        for (int jc = 0; jc < nchunks; ++jc) {
            v8h xa[2], wb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                int64_t t = m0 + wm * 64 + i * 32 + frag_row;
                t = t < T ? t : T - 1;
                xa[i] = *reinterpret_cast<const v8h *>(ep.x_out + t * K + jc * 16 + hk);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                int64_t n = n0 + wn * 64 + j * 32 + frag_row;
                n = n < N ? n : N - 1;
                wb[j] = *reinterpret_cast<const v8h *>(ep.w_out + n * K + jc * 16 + hk);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    accf[i][j] =
                        __builtin_amdgcn_mfma_f32_32x32x16_f16(xa[i], wb[j], accf[i][j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t n = n0 + wn * 64 + j * 32 + col_in;
            if (n >= N)
                continue;
            const float b = ep.bias ? h2f(ep.bias[n]) : 0.0f;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t t = m0 + wm * 64 + i * 32 + 8 * (r / 4) + row_in + (r % 4);
                    if (t < T)
                        ep.out[t * N + n] = f2h(accf[i][j][r] + b);
                }
        }
    }
}

}  // namespace

hipError_t launch_gemm(const int8_t *Xq, const int8_t *CB, int64_t T, int64_t K, int64_t N,
                       const EpilogueArgs &ep, hipStream_t s)
{
    const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((T + BM - 1) / BM));
    if (ep.c_i32)
        hipLaunchKernelGGL(k_gemm<true>, grid, dim3(kThreads), 0, s, Xq, CB, T, K, N, ep);
    else
        hipLaunchKernelGGL(k_gemm<false>, grid, dim3(kThreads), 0, s, Xq, CB, T, K, N, ep);
    return hipGetLastError();
}

}  // namespace llmint8
