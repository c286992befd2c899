// api.hip -- the C ABI: argument checks, workspace layout, kernel dispatch.
// The operations and their sources are documented in include/llmint8.h (the
// method) and include/llmint8_test.h (test and benchmark hooks).

#include <math.h>

#include <atomic>
#include <mutex>

#include "../../include/llmint8_test.h"
#include "internal.h"

namespace llmint8 {

namespace {
constexpr int64_t kMaxK = 133144;   // floor((2^31 - 1) / 127^2): K * 127^2 fits in int32
constexpr int64_t kDecodeMaxT = 16;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
// The output epilogues read four column scales with one 16-byte load and four
// bias values with one 8-byte load; the bias is optional.
bool bias_ok(const uint16_t *bias) { return ((uintptr_t)bias & 7u) == 0; }

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

MatmulWorkspace matmul_workspace_layout(int64_t T, int64_t K, int64_t N, bool decode)
{
    MatmulWorkspace L;
    size_t off = 0;
    const size_t t = (size_t)T, k = (size_t)K, n = (size_t)N;
    // the GEMM path's gathered operands hold at most kCompactMaxLd columns
    // (more outlier columns are read in place, see internal.h); the
    // weight-streaming path gathers the activations of every outlier column
    // and no weights
    const size_t ldx = decode ? k : (k < (size_t)kCompactMaxLd ? k : (size_t)kCompactMaxLd);
    L.mask = off;        off += detect_area_bytes(K);   // outlier flags of the 8-column chunks
    L.groups = off;      off += align256(4 * (k / 64));
    L.outlier_idx = off; off += align256(4 * k);
    L.info = off;        off += 256;
    L.row_absmax = off;  off += align256(4 * t);   // a (zero-point variant: nd)
    L.row_zp = off;      off += align256(8 * t);   // zero-point variant: {zp, code sum}
    L.xq = off;          off += align256((t > 16 ? t : 16) * k);   // decode: 16-row fragment order
    L.x_out = off;       off += align256(2 * t * ldx);
    L.w_out = off;       off += decode ? 0 : align256(n * ldx);   // >= 64: kOutFew's fp16 [N,32]
    // the kept-column mode's weight operand [N, kc], last so that a call can
    // run without it (see llmint8_matmul_noalloc)
    L.kept = off;
    if (!decode && T >= kKeptMinT && K <= kKeptMaxK)
        off += align256(n * (size_t)kept_cap(K));
    L.total = off;
    return L;
}

size_t act_workspace_bytes(int64_t K)
{
    return detect_area_bytes(K);   // the outlier flags of the 8-column chunks
}

namespace {
// The segments of a matmul call's workspace.
struct WsPtrs {
    uint8_t *mask;
    int32_t *groups, *O, *info;
    float *a;
    int2 *row_zp;
    int8_t *xq;
    uint16_t *x_out;
    void *w_out;
    int8_t *kept;   // null: no kept-column segment
};
WsPtrs ws_ptrs(void *ws, const MatmulWorkspace &L, bool decode)
{
    uint8_t *base = static_cast<uint8_t *>(ws);
    WsPtrs p;
    p.mask = base + L.mask;
    p.groups = reinterpret_cast<int32_t *>(base + L.groups);
    p.O = reinterpret_cast<int32_t *>(base + L.outlier_idx);
    p.info = reinterpret_cast<int32_t *>(base + L.info);
    p.a = reinterpret_cast<float *>(base + L.row_absmax);
    p.row_zp = reinterpret_cast<int2 *>(base + L.row_zp);
    p.xq = reinterpret_cast<int8_t *>(base + L.xq);
    p.x_out = reinterpret_cast<uint16_t *>(base + L.x_out);
    p.w_out = decode ? nullptr : base + L.w_out;
    p.kept = L.total > L.kept ? reinterpret_cast<int8_t *>(base + L.kept) : nullptr;
    return p;
}

// The outlier summary a call's row quantization writes: the GEMM path also
// needs the non-empty groups.
OutlierInfoOut info_out(const WsPtrs &p, bool decode)
{
    OutlierInfoOut io{p.info};
    if (!decode) {
        io.groups = p.groups;
        io.mask = p.mask;
    }
    return io;
}

// The GEMM path's dense-mode operands in the epilogue arguments.
void dense_args(EpilogueArgs &ep, const uint16_t *X, const WsPtrs &p)
{
    ep.X = X;
    ep.mask = p.mask;
    ep.groups = p.groups;
}

}  // namespace

}  // namespace llmint8

// The workspace of llmint8_matmul_noalloc: one copy per device, allocated
// when the code object is loaded on it and held until the process ends.  In
// host code the name stands for a host-side placeholder, not for device
// memory: kernels get the device address that device_scratch resolves.
static __device__ __align__(256) unsigned char scratch[LLMINT8_NOALLOC_SCRATCH_BYTES];

namespace llmint8 {
namespace {
constexpr size_t kNoAllocBytes = LLMINT8_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxScratchDevices = 64;
std::atomic<void *> g_scratch[kMaxScratchDevices];
std::mutex g_scratch_mu;

// This device's copy of `scratch`: its address is looked up once per device,
// with that device current, and kept for every later call.
hipError_t device_scratch(void **p)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxScratchDevices)
        return hipErrorInvalidDevice;
    void *q = g_scratch[dev].load(std::memory_order_acquire);
    if (!q) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        q = g_scratch[dev].load(std::memory_order_relaxed);
        if (!q) {
            e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
            if (e != hipSuccess)
                return e;
            if (!q || ((uintptr_t)q & 255u) != 0)
                return hipErrorInvalidSymbol;
            g_scratch[dev].store(q, std::memory_order_release);
        }
    }
    *p = q;
    return hipSuccess;
}
}  // namespace
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
    case LLMINT8_ERR_SCRATCH: return "LLMINT8_ERR_SCRATCH: the call needs more workspace than the static scratch of llmint8_matmul_noalloc (LLMINT8_NOALLOC_SCRATCH_BYTES = 64 MiB)";
    default: return "LLMINT8: unknown status";
    }
}

size_t llmint8_workspace_bytes(int64_t T, int64_t K, int64_t N)
{
    return llmint8_workspace_bytes_path(T, K, N, 0);
}

size_t llmint8_workspace_bytes_path(int64_t T, int64_t K, int64_t N, int path)
{
    if (T <= 0 || K <= 0 || N <= 0 || path < 0 || path > 2)
        return 0;
    return matmul_workspace_layout(T, K, N, path == 2 || (path == 0 && T <= kDecodeMaxT)).total;
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
    uint8_t *mask = static_cast<uint8_t *>(ws);
    const GatherArgs none{nullptr, nullptr, 0, nullptr};
    hipError_t e =
        quantize_act_fits_rows(T, K)
            ? launch_quantize_act_rows(X, T, K, threshold, Xq, row_absmax, outlier_idx,
                                       n_outliers, nullptr, false, stream)
            : launch_quantize_act(X, T, K, threshold, Xq, row_absmax, outlier_idx,
                                  OutlierInfoOut{n_outliers}, mask, nullptr, none, false,
                                  stream);
    return e == hipSuccess ? LLMINT8_OK : LLMINT8_ERR_HIP;
}

namespace {
// The argument and shape checks of a matmul call, in the documented order
// (the workspace is checked by the caller).
llmint8_status_t matmul_check(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                              const int8_t *CB, const float *SCB, const uint16_t *bias,
                              float threshold, int activation, const uint16_t *out, int path)
{
    if (!X || !CB || !SCB || !out || !aligned16(X) || !aligned16(CB) || !aligned16(SCB) ||
        !bias_ok(bias) || !aligned16(out) || bad_threshold(threshold) || path < 0 || path > 2 ||
        (activation != LLMINT8_ACT_NONE && activation != LLMINT8_ACT_RELU))
        return LLMINT8_ERR_INVALID_ARG;
    const llmint8_status_t st = check_shape(T, K, N);
    if (st != LLMINT8_OK)
        return st;
    if (path == 2 && T > kDecodeMaxT)
        return LLMINT8_ERR_UNSUPPORTED_SHAPE;
    return LLMINT8_OK;
}

llmint8_status_t matmul_impl(const uint16_t *X, int64_t T, int64_t K, int64_t N, const int8_t *CB,
                             const float *SCB, const uint16_t *bias, float threshold,
                             int activation, uint16_t *out, void *ws, size_t ws_bytes, int path,
                             hipEvent_t main_start, hipEvent_t main_stop, hipStream_t stream,
                             bool with_kept = true)
{
    if (!ws || !aligned16(ws))
        return LLMINT8_ERR_INVALID_ARG;
    const llmint8_status_t st =
        matmul_check(X, T, K, N, CB, SCB, bias, threshold, activation, out, path);
    if (st != LLMINT8_OK)
        return st;
    const bool decode = path == 2 || (path == 0 && T <= kDecodeMaxT);
    MatmulWorkspace L = matmul_workspace_layout(T, K, N, decode);
    if (!with_kept)
        L.total = L.kept;   // no kept-column segment: the int8 part runs over all K
    if (ws_bytes < L.total)
        return LLMINT8_ERR_WORKSPACE;
    const WsPtrs p = ws_ptrs(ws, L, decode);

    // the GEMM path also builds its outlier weight operand (and, with many
    // outlier columns, the kept-column operand); the decode path takes more
    // than a few activation rows in fragment order
    GatherArgs g{CB, SCB, N, p.w_out};
    g.cb_kept = p.kept;
    const bool packed = decode && T >= kDecodePackedMinT;
    const hipError_t eq =
        decode && quantize_act_fits_rows(T, K)
            ? launch_quantize_act_rows(X, T, K, threshold, p.xq, p.a, p.O, p.info, p.x_out,
                                       packed, stream)
            : launch_quantize_act(X, T, K, threshold, p.xq, p.a, p.O, info_out(p, decode),
                                  p.mask, p.x_out, g, packed, stream);
    if (eq != hipSuccess)
        return LLMINT8_ERR_HIP;
    EpilogueArgs ep{p.a, SCB, p.x_out, p.w_out, p.O, p.info, bias, out, nullptr,
                    activation == LLMINT8_ACT_RELU ? 1 : 0};
    dense_args(ep, X, p);
    ep.cb_kept = p.kept;
    const hipError_t e =
        decode ? launch_decode(p.xq, CB, T, K, N, ep, packed, stream, main_start, main_stop)
               : launch_gemm(p.xq, CB, T, K, N, ep, stream, main_start, main_stop);
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

llmint8_status_t llmint8_matmul_noalloc(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                                        const int8_t *CB, const float *SCB, const uint16_t *bias,
                                        float threshold, uint16_t *out, hipStream_t stream)
{
    const llmint8_status_t st =
        matmul_check(X, T, K, N, CB, SCB, bias, threshold, LLMINT8_ACT_NONE, out, 0);
    if (st != LLMINT8_OK)
        return st;
    // the kept-column segment is optional: without room for it the int8
    // part runs over all of K
    const MatmulWorkspace L = matmul_workspace_layout(T, K, N, T <= kDecodeMaxT);
    if (L.kept > kNoAllocBytes)
        return LLMINT8_ERR_SCRATCH;
    void *ws = nullptr;
    if (device_scratch(&ws) != hipSuccess)
        return LLMINT8_ERR_HIP;
    return matmul_impl(X, T, K, N, CB, SCB, bias, threshold, LLMINT8_ACT_NONE, out, ws,
                       kNoAllocBytes, 0, nullptr, nullptr, stream, L.total <= kNoAllocBytes);
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
    uint8_t *mask = static_cast<uint8_t *>(ws);
    const GatherArgs none{nullptr, nullptr, 0, nullptr};
    const hipError_t e = launch_quantize_act_zp(X, T, K, threshold, Xq, nd,
                                                reinterpret_cast<int2 *>(row_zp), outlier_idx,
                                                OutlierInfoOut{n_outliers}, mask, nullptr,
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
        !aligned16(ZP) || !aligned16(RS) || !aligned16(ND) || !bias_ok(bias) || !aligned16(out) ||
        !aligned16(ws) || bad_threshold(threshold) || path < 0 || path > 2)
        return LLMINT8_ERR_INVALID_ARG;
    llmint8_status_t st = check_shape_zp(T, K, N);
    if (st != LLMINT8_OK)
        return st;
    if (path == 2 && T > kDecodeMaxT)
        return LLMINT8_ERR_UNSUPPORTED_SHAPE;
    const bool decode = path == 2 || (path == 0 && T <= kDecodeMaxT);
    const MatmulWorkspace L = matmul_workspace_layout(T, K, N, decode);
    if (ws_bytes < L.total)
        return LLMINT8_ERR_WORKSPACE;
    const WsPtrs p = ws_ptrs(ws, L, decode);

    const GatherArgs g{CB, ND, N, p.w_out, ZP};
    const bool packed = decode && T >= kDecodePackedMinT;
    const hipError_t eq = launch_quantize_act_zp(X, T, K, threshold, p.xq, p.a, p.row_zp, p.O,
                                                 info_out(p, decode), p.mask, p.x_out, g,
                                                 packed, stream);
    if (eq != hipSuccess)
        return LLMINT8_ERR_HIP;
    EpilogueArgs ep{p.a, ND, p.x_out, p.w_out, p.O, p.info, bias, out, nullptr, 0, p.row_zp, ZP, RS};
    dense_args(ep, X, p);
    const hipError_t e =
        decode ? launch_decode(p.xq, CB, T, K, N, ep, packed, stream, main_start, main_stop)
               : launch_gemm(p.xq, CB, T, K, N, ep, stream, main_start, main_stop);
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

namespace {
// The FP8 entry points of both formats (fmt kF8E5M2 or kF8E4M3).
llmint8_status_t quantize_weight_fp8(const uint16_t *W_t, int64_t K, int64_t N, uint8_t *CB8,
                                     float *SC8, int fmt, hipStream_t stream)
{
    if (!W_t || !CB8 || !SC8 || !aligned16(W_t) || !aligned16(CB8))
        return LLMINT8_ERR_INVALID_ARG;
    llmint8_status_t st = check_shape(1, K, N);
    if (st != LLMINT8_OK)
        return st;
    return launch_quantize_weight_f8(W_t, K, N, CB8, SC8, fmt, stream) == hipSuccess
               ? LLMINT8_OK
               : LLMINT8_ERR_HIP;
}

llmint8_status_t quantize_act_fp8(const uint16_t *X, int64_t T, int64_t K, float threshold,
                                  uint8_t *Xq8, float *row_scale, int32_t *outlier_idx,
                                  int32_t *n_outliers, void *ws, size_t ws_bytes, int fmt,
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
    uint8_t *mask = static_cast<uint8_t *>(ws);
    GatherArgs none{nullptr, nullptr, 0, nullptr};
    none.f8 = fmt;
    const hipError_t e = launch_quantize_act_f8(X, T, K, threshold, Xq8, row_scale, outlier_idx,
                                                OutlierInfoOut{n_outliers}, mask, nullptr,
                                                none, false, fmt, stream);
    return e == hipSuccess ? LLMINT8_OK : LLMINT8_ERR_HIP;
}

llmint8_status_t matmul_fp8_path(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                                 const uint8_t *CB8, const float *SC8, const uint16_t *bias,
                                 float threshold, uint16_t *out, void *ws, size_t ws_bytes,
                                 int path, hipEvent_t main_start, hipEvent_t main_stop, int fmt,
                                 hipStream_t stream)
{
    if (!X || !CB8 || !SC8 || !out || !ws || !aligned16(X) || !aligned16(CB8) ||
        !aligned16(SC8) || !bias_ok(bias) || !aligned16(out) || !aligned16(ws) ||
        bad_threshold(threshold) || path < 0 || path > 2)
        return LLMINT8_ERR_INVALID_ARG;
    llmint8_status_t st = check_shape(T, K, N);
    if (st != LLMINT8_OK)
        return st;
    if (path == 2 && T > kDecodeMaxT)
        return LLMINT8_ERR_UNSUPPORTED_SHAPE;
    const bool decode = path == 2 || (path == 0 && T <= kDecodeMaxT);
    const MatmulWorkspace L = matmul_workspace_layout(T, K, N, decode);
    if (ws_bytes < L.total)
        return LLMINT8_ERR_WORKSPACE;
    const WsPtrs p = ws_ptrs(ws, L, decode);
    const int8_t *CB = reinterpret_cast<const int8_t *>(CB8);

    GatherArgs g{CB, SC8, N, p.w_out};
    g.f8 = fmt;
    g.cb_kept = p.kept;
    const bool packed = decode && T >= kDecodePackedMinT;
    const hipError_t eq = launch_quantize_act_f8(X, T, K, threshold,
                                                 reinterpret_cast<uint8_t *>(p.xq), p.a, p.O,
                                                 info_out(p, decode), p.mask, p.x_out, g,
                                                 packed, fmt, stream);
    if (eq != hipSuccess)
        return LLMINT8_ERR_HIP;
    EpilogueArgs ep{p.a, SC8, p.x_out, p.w_out, p.O, p.info, bias, out, nullptr, 0};
    ep.f8 = fmt;
    dense_args(ep, X, p);
    ep.cb_kept = p.kept;
    const hipError_t e =
        decode ? launch_decode(p.xq, CB, T, K, N, ep, packed, stream, main_start, main_stop)
               : launch_gemm(p.xq, CB, T, K, N, ep, stream, main_start, main_stop);
    return e == hipSuccess ? LLMINT8_OK : LLMINT8_ERR_HIP;
}
}  // namespace

llmint8_status_t llmint8_quantize_weight_f8(const uint16_t *W_t, int64_t K, int64_t N, uint8_t *CB8,
                                            float *SC8, hipStream_t stream)
{
    return quantize_weight_fp8(W_t, K, N, CB8, SC8, kF8E5M2, stream);
}

llmint8_status_t llmint8_quantize_act_f8(const uint16_t *X, int64_t T, int64_t K, float threshold,
                                         uint8_t *Xq8, float *row_scale, int32_t *outlier_idx,
                                         int32_t *n_outliers, void *ws, size_t ws_bytes,
                                         hipStream_t stream)
{
    return quantize_act_fp8(X, T, K, threshold, Xq8, row_scale, outlier_idx, n_outliers, ws,
                            ws_bytes, kF8E5M2, stream);
}

llmint8_status_t llmint8_matmul_f8_path(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                                        const uint8_t *CB8, const float *SC8, const uint16_t *bias,
                                        float threshold, uint16_t *out, void *ws, size_t ws_bytes,
                                        int path, hipEvent_t main_start, hipEvent_t main_stop,
                                        hipStream_t stream)
{
    return matmul_fp8_path(X, T, K, N, CB8, SC8, bias, threshold, out, ws, ws_bytes, path,
                           main_start, main_stop, kF8E5M2, stream);
}

llmint8_status_t llmint8_matmul_f8(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                                   const uint8_t *CB8, const float *SC8, const uint16_t *bias,
                                   float threshold, uint16_t *out, void *ws, size_t ws_bytes,
                                   hipStream_t stream)
{
    return llmint8_matmul_f8_path(X, T, K, N, CB8, SC8, bias, threshold, out, ws, ws_bytes, 0,
                                  nullptr, nullptr, stream);
}

llmint8_status_t llmint8_quantize_weight_e4m3(const uint16_t *W_t, int64_t K, int64_t N,
                                              uint8_t *CB8, float *SC8, hipStream_t stream)
{
    return quantize_weight_fp8(W_t, K, N, CB8, SC8, kF8E4M3, stream);
}

llmint8_status_t llmint8_quantize_act_e4m3(const uint16_t *X, int64_t T, int64_t K,
                                           float threshold, uint8_t *Xq8, float *row_scale,
                                           int32_t *outlier_idx, int32_t *n_outliers, void *ws,
                                           size_t ws_bytes, hipStream_t stream)
{
    return quantize_act_fp8(X, T, K, threshold, Xq8, row_scale, outlier_idx, n_outliers, ws,
                            ws_bytes, kF8E4M3, stream);
}

llmint8_status_t llmint8_matmul_e4m3_path(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                                          const uint8_t *CB8, const float *SC8,
                                          const uint16_t *bias, float threshold, uint16_t *out,
                                          void *ws, size_t ws_bytes, int path,
                                          hipEvent_t main_start, hipEvent_t main_stop,
                                          hipStream_t stream)
{
    return matmul_fp8_path(X, T, K, N, CB8, SC8, bias, threshold, out, ws, ws_bytes, path,
                           main_start, main_stop, kF8E4M3, stream);
}

llmint8_status_t llmint8_matmul_e4m3(const uint16_t *X, int64_t T, int64_t K, int64_t N,
                                     const uint8_t *CB8, const float *SC8, const uint16_t *bias,
                                     float threshold, uint16_t *out, void *ws, size_t ws_bytes,
                                     hipStream_t stream)
{
    return llmint8_matmul_e4m3_path(X, T, K, N, CB8, SC8, bias, threshold, out, ws, ws_bytes, 0,
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
