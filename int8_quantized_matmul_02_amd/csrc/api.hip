// api.hip -- the C ABI: argument checks, workspace layout, kernel dispatch.
// The operations and their sources are documented in include/llmint8.h.

#include <math.h>

#include "../../include/llmint8.h"
#include "internal.h"

namespace llmint8 {

namespace {
constexpr int64_t kMaxK = 133144;   // floor((2^31 - 1) / 127^2): K * 127^2 fits in int32
constexpr int64_t kDecodeMaxT = 16;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

llmint8_status_t check_shape(int64_t T, int64_t K, int64_t N)
{
    if (T <= 0 || K <= 0 || N <= 0)
        return LLMINT8_ERR_INVALID_ARG;
    if (K % 64 != 0 || N % 64 != 0 || K > kMaxK)
        return LLMINT8_ERR_UNSUPPORTED_SHAPE;
    return LLMINT8_OK;
}

bool bad_threshold(float thr) { return isnan(thr) || thr < 0.0f; }

llmint8_status_t check_shape_zp(int64_t T, int64_t K, int64_t N)
{
    const llmint8_status_t st = check_shape(T, K, N);
    if (st != LLMINT8_OK)
        return st;
    return K > kMaxKZp ? LLMINT8_ERR_UNSUPPORTED_SHAPE : LLMINT8_OK;
}
}  // namespace

MatmulWorkspace matmul_workspace_layout(int64_t T, int64_t K, int64_t N)
{
    MatmulWorkspace L;
    size_t off = 0;
    const size_t t = (size_t)T, k = (size_t)K, n = (size_t)N;
    L.partial = off;     off += align256((size_t)kDetectSplits * (k / 8));
    L.mask = off;        off += align256(k / 8);
    L.chunk_pre = off;   off += align256(4 * k);   // K/8 entries used
    L.outlier_idx = off; off += align256(4 * k);
    L.n_outliers = off;  off += 256;
    L.row_absmax = off;  off += align256(4 * t);   // a (zero-point variant: nd)
    L.row_zp = off;      off += align256(8 * t);   // zero-point variant: {zp, code sum}
    L.xq = off;          off += align256((t > 16 ? t : 16) * k);   // decode: 16-row fragment order
    L.x_out = off;       off += align256(2 * t * k);
    L.w_out = off;       off += align256(2 * n * k);
    L.total = off;
    return L;
}

size_t act_workspace_bytes(int64_t K)
{
    const size_t k = (size_t)K;
    return align256((size_t)kDetectSplits * (k / 8)) + align256(k / 8) + align256(4 * k);
}

}  // namespace llmint8

using namespace llmint8;

extern "C" {

const char *llmint8_status_string(int status)
{
    switch (status) {
    case LLMINT8_OK: return "LLMINT8_OK";
    case LLMINT8_ERR_INVALID_ARG: return "LLMINT8_ERR_INVALID_ARG: null/misaligned pointer, non-positive size or NaN/negative threshold";
    case LLMINT8_ERR_UNSUPPORTED_SHAPE: return "LLMINT8_ERR_UNSUPPORTED_SHAPE: K and N must be multiples of 64, K <= 133144 (K <= 33286 for the zero-point variant; T <= 16 for the weight-streaming path)";
    case LLMINT8_ERR_WORKSPACE: return "LLMINT8_ERR_WORKSPACE: workspace smaller than the size query";
    case LLMINT8_ERR_HIP: return "LLMINT8_ERR_HIP: a kernel launch failed";
    default: return "LLMINT8: unknown status";
    }
}

size_t llmint8_workspace_bytes(int64_t T, int64_t K, int64_t N)
{
    if (T <= 0 || K <= 0 || N <= 0)
        return 0;
    return matmul_workspace_layout(T, K, N).total;
}

size_t llmint8_quantize_act_workspace_bytes(int64_t K)
{
    if (K <= 0)
        return 0;
    return act_workspace_bytes(K);
}

llmint8_status_t llmint8_quantize_weight(const uint16_t *W_t, int64_t K, int64_t N, int8_t *CB,
                                         float *SCB, hipStream_t stream)
{
    if (!W_t || !CB || !SCB || !aligned16(W_t) || !aligned16(CB))
        return LLMINT8_ERR_INVALID_ARG;
    llmint8_status_t st = check_shape(1, K, N);
    if (st != LLMINT8_OK)
        return st;
    return launch_quantize_weight(W_t, K, N, CB, SCB, stream) == hipSuccess ? LLMINT8_OK
                                                                            : LLMINT8_ERR_HIP;
}

llmint8_status_t llmint8_quantize_act(const uint16_t *X, int64_t T, int64_t K, float threshold,
                                      int8_t *Xq, float *row_absmax, int32_t *outlier_idx,
                                      int32_t *n_outliers, void *ws, size_t ws_bytes,
                                      hipStream_t stream)
{
    if (!X || !Xq || !row_absmax || !outlier_idx || !n_outliers || !ws || !aligned16(X) ||
        !aligned16(Xq) || !aligned16(ws) || bad_threshold(threshold))
        return LLMINT8_ERR_INVALID_ARG;
    llmint8_status_t st = check_shape(T, K, 64);
    if (st != LLMINT8_OK)
        return st;
    if (ws_bytes < act_workspace_bytes(K))
        return LLMINT8_ERR_WORKSPACE;
    uint8_t *base = static_cast<uint8_t *>(ws);
    uint8_t *partial = base;
    uint8_t *mask = base + align256((size_t)kDetectSplits * ((size_t)K / 8));
    int32_t *chunk_pre = reinterpret_cast<int32_t *>(mask + align256((size_t)K / 8));
    const GatherArgs none{nullptr, nullptr, 0, nullptr};
    hipError_t e =
        quantize_act_fits_rows(T, K)
            ? launch_quantize_act_rows(X, T, K, threshold, Xq, row_absmax, outlier_idx,
                                       n_outliers, nullptr, false, stream)
            : launch_quantize_act(X, T, K, threshold, Xq, row_absmax, outlier_idx, n_outliers,
                                  partial, mask, chunk_pre, nullptr, none, false, stream);
    return e == hipSuccess ? LLMINT8_OK : LLMINT8_ERR_HIP;
}

namespace {
llmint8_status_t matmul_impl(const uint16_t *X, int64_t T, int64_t K, int64_t N, const int8_t *CB,
                             const float *SCB, const uint16_t *bias, float threshold,
                             int activation, uint16_t *out, void *ws, size_t ws_bytes, int path,
                             hipEvent_t main_start, hipEvent_t main_stop, hipStream_t stream)
{
    if (!X || !CB || !SCB || !out || !ws || !aligned16(X) || !aligned16(CB) ||
        !aligned16(out) || !aligned16(ws) || bad_threshold(threshold) || path < 0 || path > 2 ||
        (activation != LLMINT8_ACT_NONE && activation != LLMINT8_ACT_RELU))
        return LLMINT8_ERR_INVALID_ARG;
    llmint8_status_t st = check_shape(T, K, N);
    if (st != LLMINT8_OK)
        return st;
    if (path == 2 && T > kDecodeMaxT)
        return LLMINT8_ERR_UNSUPPORTED_SHAPE;
    const MatmulWorkspace L = matmul_workspace_layout(T, K, N);
    if (ws_bytes < L.total)
        return LLMINT8_ERR_WORKSPACE;
    const bool decode = path == 2 || (path == 0 && T <= kDecodeMaxT);

    uint8_t *base = static_cast<uint8_t *>(ws);
    uint8_t *partial = base + L.partial;
    uint8_t *mask = base + L.mask;
    int32_t *chunk_pre = reinterpret_cast<int32_t *>(base + L.chunk_pre);
    int32_t *O = reinterpret_cast<int32_t *>(base + L.outlier_idx);
    int32_t *n_out = reinterpret_cast<int32_t *>(base + L.n_outliers);
    float *a = reinterpret_cast<float *>(base + L.row_absmax);
    int8_t *Xq = reinterpret_cast<int8_t *>(base + L.xq);
    uint16_t *x_out = reinterpret_cast<uint16_t *>(base + L.x_out);
    uint16_t *w_out = reinterpret_cast<uint16_t *>(base + L.w_out);

    // the GEMM path also needs the dequantized outlier weight rows; the
    // decode path takes more than a few activation rows in fragment order
    const GatherArgs g{CB, SCB, N, decode ? nullptr : w_out};
    const bool packed = decode && T >= kDecodePackedMinT;
    const hipError_t eq =
        decode && quantize_act_fits_rows(T, K)
            ? launch_quantize_act_rows(X, T, K, threshold, Xq, a, O, n_out, x_out, packed, stream)
            : launch_quantize_act(X, T, K, threshold, Xq, a, O, n_out, partial, mask, chunk_pre,
                                  x_out, g, packed, stream);
    if (eq != hipSuccess)
        return LLMINT8_ERR_HIP;
    EpilogueArgs ep{a, SCB, x_out, w_out, O, n_out, bias, out, nullptr,
                    activation == LLMINT8_ACT_RELU ? 1 : 0};
    const hipError_t e =
        decode ? launch_decode(Xq, CB, T, K, N, ep, packed, stream, main_start, main_stop)
               : launch_gemm(Xq, CB, T, K, N, ep, stream, main_start, main_stop);
    return e == hipSuccess ? LLMINT8_OK : LLMINT8_ERR_HIP;
}
}  // namespace

llmint8_status_t llmint8_matmul_path(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                                     const int8_t *CB, const float *SCB, const uint16_t *bias,
                                     float threshold, uint16_t *out, void *ws, size_t ws_bytes,
                                     int path, hipEvent_t main_start, hipEvent_t main_stop,
                                     hipStream_t stream)
{
    return matmul_impl(X, T, K, N, CB, SCB, bias, threshold, LLMINT8_ACT_NONE, out, ws, ws_bytes,
                       path, main_start, main_stop, stream);
}

llmint8_status_t llmint8_matmul_act(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                                    const int8_t *CB, const float *SCB, const uint16_t *bias,
                                    float threshold, int activation, uint16_t *out, void *ws,
                                    size_t ws_bytes, hipStream_t stream)
{
    return matmul_impl(X, T, K, N, CB, SCB, bias, threshold, activation, out, ws, ws_bytes, 0,
                       nullptr, nullptr, stream);
}

llmint8_status_t llmint8_matmul(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                                const int8_t *CB, const float *SCB, const uint16_t *bias,
                                float threshold, uint16_t *out, void *ws, size_t ws_bytes,
                                hipStream_t stream)
{
    return llmint8_matmul_path(X, T, K, N, CB, SCB, bias, threshold, out, ws, ws_bytes, 0,
                               nullptr, nullptr, stream);
}

llmint8_status_t llmint8_quantize_weight_zp(const uint16_t *W_t, int64_t K, int64_t N, int8_t *CB,
                                            float *ND, int32_t *ZP, int32_t *RS,
                                            hipStream_t stream)
{
    if (!W_t || !CB || !ND || !ZP || !RS || !aligned16(W_t) || !aligned16(CB))
        return LLMINT8_ERR_INVALID_ARG;
    llmint8_status_t st = check_shape_zp(1, K, N);
    if (st != LLMINT8_OK)
        return st;
    return launch_quantize_weight_zp(W_t, K, N, CB, ND, ZP, RS, stream) == hipSuccess
               ? LLMINT8_OK
               : LLMINT8_ERR_HIP;
}

llmint8_status_t llmint8_quantize_act_zp(const uint16_t *X, int64_t T, int64_t K, float threshold,
                                         int8_t *Xq, float *nd, int32_t *row_zp,
                                         int32_t *outlier_idx, int32_t *n_outliers, void *ws,
                                         size_t ws_bytes, hipStream_t stream)
{
    if (!X || !Xq || !nd || !row_zp || !outlier_idx || !n_outliers || !ws || !aligned16(X) ||
        !aligned16(Xq) || !aligned16(ws) || ((uintptr_t)row_zp & 7u) || bad_threshold(threshold))
        return LLMINT8_ERR_INVALID_ARG;
    llmint8_status_t st = check_shape_zp(T, K, 64);
    if (st != LLMINT8_OK)
        return st;
    if (ws_bytes < act_workspace_bytes(K))
        return LLMINT8_ERR_WORKSPACE;
    uint8_t *base = static_cast<uint8_t *>(ws);
    uint8_t *partial = base;
    uint8_t *mask = base + align256((size_t)kDetectSplits * ((size_t)K / 8));
    int32_t *chunk_pre = reinterpret_cast<int32_t *>(mask + align256((size_t)K / 8));
    const GatherArgs none{nullptr, nullptr, 0, nullptr};
    const hipError_t e = launch_quantize_act_zp(X, T, K, threshold, Xq, nd,
                                                reinterpret_cast<int2 *>(row_zp), outlier_idx,
                                                n_outliers, partial, mask, chunk_pre, nullptr,
                                                none, false, stream);
    return e == hipSuccess ? LLMINT8_OK : LLMINT8_ERR_HIP;
}

llmint8_status_t llmint8_matmul_zp_path(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                                        const int8_t *CB, const float *ND, const int32_t *ZP,
                                        const int32_t *RS, const uint16_t *bias, float threshold,
                                        uint16_t *out, void *ws, size_t ws_bytes, int path,
                                        hipEvent_t main_start, hipEvent_t main_stop,
                                        hipStream_t stream)
{
    if (!X || !CB || !ND || !ZP || !RS || !out || !ws || !aligned16(X) || !aligned16(CB) ||
        !aligned16(ZP) || !aligned16(RS) || !aligned16(ND) || !aligned16(out) || !aligned16(ws) ||
        bad_threshold(threshold) || path < 0 || path > 2)
        return LLMINT8_ERR_INVALID_ARG;
    llmint8_status_t st = check_shape_zp(T, K, N);
    if (st != LLMINT8_OK)
        return st;
    if (path == 2 && T > kDecodeMaxT)
        return LLMINT8_ERR_UNSUPPORTED_SHAPE;
    const MatmulWorkspace L = matmul_workspace_layout(T, K, N);
    if (ws_bytes < L.total)
        return LLMINT8_ERR_WORKSPACE;
    const bool decode = path == 2 || (path == 0 && T <= kDecodeMaxT);

    uint8_t *base = static_cast<uint8_t *>(ws);
    uint8_t *partial = base + L.partial;
    uint8_t *mask = base + L.mask;
    int32_t *chunk_pre = reinterpret_cast<int32_t *>(base + L.chunk_pre);
    int32_t *O = reinterpret_cast<int32_t *>(base + L.outlier_idx);
    int32_t *n_out = reinterpret_cast<int32_t *>(base + L.n_outliers);
    float *nd = reinterpret_cast<float *>(base + L.row_absmax);
    int2 *row_zp = reinterpret_cast<int2 *>(base + L.row_zp);
    int8_t *Xq = reinterpret_cast<int8_t *>(base + L.xq);
    uint16_t *x_out = reinterpret_cast<uint16_t *>(base + L.x_out);
    uint16_t *w_out = reinterpret_cast<uint16_t *>(base + L.w_out);

    const GatherArgs g{CB, ND, N, decode ? nullptr : w_out, ZP};
    const bool packed = decode && T >= kDecodePackedMinT;
    const hipError_t eq = launch_quantize_act_zp(X, T, K, threshold, Xq, nd, row_zp, O, n_out,
                                                 partial, mask, chunk_pre, x_out, g, packed,
                                                 stream);
    if (eq != hipSuccess)
        return LLMINT8_ERR_HIP;
    EpilogueArgs ep{nd, ND, x_out, w_out, O, n_out, bias, out, nullptr, 0, row_zp, ZP, RS};
    const hipError_t e =
        decode ? launch_decode(Xq, CB, T, K, N, ep, packed, stream, main_start, main_stop)
               : launch_gemm(Xq, CB, T, K, N, ep, stream, main_start, main_stop);
    return e == hipSuccess ? LLMINT8_OK : LLMINT8_ERR_HIP;
}

llmint8_status_t llmint8_matmul_zp(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                                   const int8_t *CB, const float *ND, const int32_t *ZP,
                                   const int32_t *RS, const uint16_t *bias, float threshold,
                                   uint16_t *out, void *ws, size_t ws_bytes, hipStream_t stream)
{
    return llmint8_matmul_zp_path(X, T, K, N, CB, ND, ZP, RS, bias, threshold, out, ws, ws_bytes,
                                  0, nullptr, nullptr, stream);
}

llmint8_status_t llmint8_quantize_weight_f8(const uint16_t *W_t, int64_t K, int64_t N, uint8_t *CB8,
                                            float *SC8, hipStream_t stream)
{
    if (!W_t || !CB8 || !SC8 || !aligned16(W_t) || !aligned16(CB8))
        return LLMINT8_ERR_INVALID_ARG;
    llmint8_status_t st = check_shape(1, K, N);
    if (st != LLMINT8_OK)
        return st;
    return launch_quantize_weight_f8(W_t, K, N, CB8, SC8, stream) == hipSuccess ? LLMINT8_OK
                                                                                : LLMINT8_ERR_HIP;
}

llmint8_status_t llmint8_quantize_act_f8(const uint16_t *X, int64_t T, int64_t K, float threshold,
                                         uint8_t *Xq8, float *row_scale, int32_t *outlier_idx,
                                         int32_t *n_outliers, void *ws, size_t ws_bytes,
                                         hipStream_t stream)
{
    if (!X || !Xq8 || !row_scale || !outlier_idx || !n_outliers || !ws || !aligned16(X) ||
        !aligned16(Xq8) || !aligned16(ws) || bad_threshold(threshold))
        return LLMINT8_ERR_INVALID_ARG;
    llmint8_status_t st = check_shape(T, K, 64);
    if (st != LLMINT8_OK)
        return st;
    if (ws_bytes < act_workspace_bytes(K))
        return LLMINT8_ERR_WORKSPACE;
    uint8_t *base = static_cast<uint8_t *>(ws);
    uint8_t *partial = base;
    uint8_t *mask = base + align256((size_t)kDetectSplits * ((size_t)K / 8));
    int32_t *chunk_pre = reinterpret_cast<int32_t *>(mask + align256((size_t)K / 8));
    GatherArgs none{nullptr, nullptr, 0, nullptr};
    none.f8 = true;
    const hipError_t e = launch_quantize_act_f8(X, T, K, threshold, Xq8, row_scale, outlier_idx,
                                                n_outliers, partial, mask, chunk_pre, nullptr,
                                                none, false, stream);
    return e == hipSuccess ? LLMINT8_OK : LLMINT8_ERR_HIP;
}

llmint8_status_t llmint8_matmul_f8_path(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                                        const uint8_t *CB8, const float *SC8, const uint16_t *bias,
                                        float threshold, uint16_t *out, void *ws, size_t ws_bytes,
                                        int path, hipEvent_t main_start, hipEvent_t main_stop,
                                        hipStream_t stream)
{
    if (!X || !CB8 || !SC8 || !out || !ws || !aligned16(X) || !aligned16(CB8) ||
        !aligned16(SC8) || !aligned16(out) || !aligned16(ws) || bad_threshold(threshold) ||
        path < 0 || path > 2)
        return LLMINT8_ERR_INVALID_ARG;
    llmint8_status_t st = check_shape(T, K, N);
    if (st != LLMINT8_OK)
        return st;
    if (path == 2 && T > kDecodeMaxT)
        return LLMINT8_ERR_UNSUPPORTED_SHAPE;
    const MatmulWorkspace L = matmul_workspace_layout(T, K, N);
    if (ws_bytes < L.total)
        return LLMINT8_ERR_WORKSPACE;
    const bool decode = path == 2 || (path == 0 && T <= kDecodeMaxT);

    uint8_t *base = static_cast<uint8_t *>(ws);
    uint8_t *partial = base + L.partial;
    uint8_t *mask = base + L.mask;
    int32_t *chunk_pre = reinterpret_cast<int32_t *>(base + L.chunk_pre);
    int32_t *O = reinterpret_cast<int32_t *>(base + L.outlier_idx);
    int32_t *n_out = reinterpret_cast<int32_t *>(base + L.n_outliers);
    float *sc = reinterpret_cast<float *>(base + L.row_absmax);
    uint8_t *Xq8 = base + L.xq;
    uint16_t *x_out = reinterpret_cast<uint16_t *>(base + L.x_out);
    uint16_t *w_out = reinterpret_cast<uint16_t *>(base + L.w_out);
    const int8_t *CB = reinterpret_cast<const int8_t *>(CB8);

    GatherArgs g{CB, SC8, N, decode ? nullptr : w_out};
    g.f8 = true;
    const bool packed = decode && T >= kDecodePackedMinT;
    const hipError_t eq = launch_quantize_act_f8(X, T, K, threshold, Xq8, sc, O, n_out, partial,
                                                 mask, chunk_pre, x_out, g, packed, stream);
    if (eq != hipSuccess)
        return LLMINT8_ERR_HIP;
    EpilogueArgs ep{sc, SC8, x_out, w_out, O, n_out, bias, out, nullptr, 0};
    ep.f8 = true;
    const int8_t *Xq = reinterpret_cast<const int8_t *>(Xq8);
    const hipError_t e =
        decode ? launch_decode(Xq, CB, T, K, N, ep, packed, stream, main_start, main_stop)
               : launch_gemm(Xq, CB, T, K, N, ep, stream, main_start, main_stop);
    return e == hipSuccess ? LLMINT8_OK : LLMINT8_ERR_HIP;
}

llmint8_status_t llmint8_matmul_f8(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                                   const uint8_t *CB8, const float *SC8, const uint16_t *bias,
                                   float threshold, uint16_t *out, void *ws, size_t ws_bytes,
                                   hipStream_t stream)
{
    return llmint8_matmul_f8_path(X, T, K, N, CB8, SC8, bias, threshold, out, ws, ws_bytes, 0,
                                  nullptr, nullptr, stream);
}

llmint8_status_t llmint8_igemm_i32(const int8_t *Xq, int64_t T, int64_t K, int64_t N,
                                   const int8_t *CB, int32_t *C, int path, hipStream_t stream)
{
    if (!Xq || !CB || !C || !aligned16(Xq) || !aligned16(CB) || path < 0 || path > 2)
        return LLMINT8_ERR_INVALID_ARG;
    llmint8_status_t st = check_shape(T, K, N);
    if (st != LLMINT8_OK)
        return st;
    if (path == 2 && T > kDecodeMaxT)
        return LLMINT8_ERR_UNSUPPORTED_SHAPE;
    const bool decode = path == 2 || (path == 0 && T <= kDecodeMaxT);
    EpilogueArgs ep{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, C};
    hipError_t e = decode ? launch_decode(Xq, CB, T, K, N, ep, false, stream)
                          : launch_gemm(Xq, CB, T, K, N, ep, stream);
    return e == hipSuccess ? LLMINT8_OK : LLMINT8_ERR_HIP;
}

}  // extern "C"
