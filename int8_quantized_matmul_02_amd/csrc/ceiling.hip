// ceiling.hip -- the MFMA issue rate the chip sustains on given operand bytes
// with nothing else in the loop (a benchmark hook, include/llmint8_test.h).
//
// The dense MFMA peaks are quoted at the chip's top clock; a GEMM that keeps
// the matrix cores busy draws enough power for the clock to drop, and how far
// depends on the operands' bits.  This kernel measures that ceiling on the
// workload's own data: every wavefront loads 4 + 4 fragments of two k-steps
// from the two operand matrices (a 128 x 128 output tile, as a GEMM
// wavefront owns, at a tile position that differs per wavefront) into
// registers once, then issues only MFMAs on 16 independent accumulators.
#include "../../include/llmint8_test.h"
#include "internal.h"

namespace llmint8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kCeilWaves = 4;

template <bool kF16>
__global__ __launch_bounds__(64 * kCeilWaves) void k_mfma_ceiling(
    const char *__restrict__ A, int64_t T, const char *__restrict__ B, int64_t N,
    int64_t row_bytes, int iters, int32_t *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const int64_t g = (int64_t)blockIdx.x * kCeilWaves + (threadIdx.x >> 6);
    const int64_t ntm = T / 128, ntn = N / 128, nk = row_bytes / 64;
    const int64_t m0 = (g % ntm) * 128, n0 = ((g / ntm) % ntn) * 128, k0 = (g * 7 % nk) * 64;
    v4i a[4][2], b[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int64_t kb = k0 + 32 * ks + 16 * (lane >> 5);
            a[i][ks] = *reinterpret_cast<const v4i *>(A + (m0 + 32 * i + (lane & 31)) * row_bytes + kb);
            b[i][ks] = *reinterpret_cast<const v4i *>(B + (n0 + 32 * i + (lane & 31)) * row_bytes + kb);
        }
    using Acc = std::conditional_t<kF16, v16f, v16i>;
    Acc acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (kF16)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            __builtin_bit_cast(v8h, a[i][ks]), __builtin_bit_cast(v8h, b[j][ks]),
                            acc[i][j], 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i][ks], b[j][ks],
                                                                          acc[i][j], 0, 0, 0);
                }
    }
    // one value per lane keeps every product live
    std::conditional_t<kF16, float, int32_t> s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s += acc[i][j][r];
    out[g * 64 + lane] = __builtin_bit_cast(int32_t, s);
}

}  // namespace
}  // namespace llmint8

using namespace llmint8;

extern "C" llmint8_status_t llmint8_mfma_ceiling(const void *A, int64_t T, const void *B,
                                                 int64_t N, int64_t K, int kind, int blocks,
                                                 int iters, int32_t *out, hipEvent_t start,
                                                 hipEvent_t stop, hipStream_t stream)
{
    const int64_t row_bytes = kind == 1 ? 2 * K : K;
    if (!A || !B || !out || (kind != 0 && kind != 1) || blocks <= 0 || iters <= 0 ||
        T < 128 || N < 128 || K <= 0 || (((uintptr_t)A | (uintptr_t)B) & 15u) != 0)
        return LLMINT8_ERR_INVALID_ARG;
    if (row_bytes % 64 != 0)
        return LLMINT8_ERR_UNSUPPORTED_SHAPE;
    if (start && hipEventRecord(start, stream) != hipSuccess)
        return LLMINT8_ERR_HIP;
    if (kind == 1)
        hipLaunchKernelGGL(k_mfma_ceiling<true>, dim3(blocks), dim3(64 * kCeilWaves), 0, stream,
                           static_cast<const char *>(A), T, static_cast<const char *>(B), N,
                           row_bytes, iters, out);
    else
        hipLaunchKernelGGL(k_mfma_ceiling<false>, dim3(blocks), dim3(64 * kCeilWaves), 0, stream,
                           static_cast<const char *>(A), T, static_cast<const char *>(B), N,
                           row_bytes, iters, out);
    if (hipGetLastError() != hipSuccess)
        return LLMINT8_ERR_HIP;
    if (stop && hipEventRecord(stop, stream) != hipSuccess)
        return LLMINT8_ERR_HIP;
    return LLMINT8_OK;
}
