"""Python binding of libllmint8.so: argument marshalling only.

Each function has the name of the C entry point it calls (see
include/llmint8.h for the operation, layouts, ownership and errors, and
include/llmint8_test.h for the kernel-forcing and timing hooks).  Every
step of the computation runs in the library's HIP kernels; torch only
provides device memory (outputs and workspace, allocated here when the caller
passes none) and the current stream.  There is no fallback: if the library is
not built, or a call returns an error status, these functions raise.
"""
import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libllmint8.so")
_lib = None

LLMINT8_OK = 0
LLMINT8_ERR_SCRATCH = 5
PATH_AUTO, PATH_GEMM, PATH_DECODE = 0, 1, 2
ACT_NONE, ACT_RELU = 0, 1

EXPORTS = (
    "llmint8_status_string",
    "llmint8_workspace_bytes",
    "llmint8_workspace_bytes_path",
    "llmint8_quantize_act_workspace_bytes",
    "llmint8_quantize_weight",
    "llmint8_quantize_act",
    "llmint8_matmul",
    "llmint8_matmul_act",
    "llmint8_matmul_path",
    "llmint8_igemm_i32",
    "llmint8_quantize_weight_zp",
    "llmint8_quantize_act_zp",
    "llmint8_matmul_zp",
    "llmint8_matmul_zp_path",
    "llmint8_quantize_weight_f8",
    "llmint8_quantize_act_f8",
    "llmint8_matmul_f8",
    "llmint8_matmul_f8_path",
    "llmint8_quantize_weight_e4m3",
    "llmint8_quantize_act_e4m3",
    "llmint8_matmul_e4m3",
    "llmint8_matmul_e4m3_path",
    "llmint8_mfma_ceiling",
    "llmint8_matmul_noalloc",
)


class LLMInt8Error(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s failed: %s" % (fn, _load().llmint8_status_string(status).decode()))


def library_path():
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            "libllmint8.so is not built (expected at %s); run "
            "`python -m int8_quantized_matmul_02_amd.build` or __graft_entry__.build()" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, F, SZ, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_int
    lib.llmint8_status_string.argtypes = [I]
    lib.llmint8_status_string.restype = ctypes.c_char_p
    lib.llmint8_workspace_bytes.argtypes = [I64, I64, I64]
    lib.llmint8_workspace_bytes.restype = SZ
    lib.llmint8_workspace_bytes_path.argtypes = [I64, I64, I64, I]
    lib.llmint8_workspace_bytes_path.restype = SZ
    lib.llmint8_quantize_act_workspace_bytes.argtypes = [I64]
    lib.llmint8_quantize_act_workspace_bytes.restype = SZ
    lib.llmint8_quantize_weight.argtypes = [P, I64, I64, P, P, P]
    lib.llmint8_quantize_act.argtypes = [P, I64, I64, F, P, P, P, P, P, SZ, P]
    lib.llmint8_matmul.argtypes = [P, I64, I64, I64, P, P, P, F, P, P, SZ, P]
    lib.llmint8_matmul_act.argtypes = [P, I64, I64, I64, P, P, P, F, I, P, P, SZ, P]
    lib.llmint8_matmul_path.argtypes = [P, I64, I64, I64, P, P, P, F, P, P, SZ, I, P, P, P]
    lib.llmint8_igemm_i32.argtypes = [P, I64, I64, I64, P, P, I, P]
    lib.llmint8_quantize_weight_zp.argtypes = [P, I64, I64, P, P, P, P, P]
    lib.llmint8_quantize_act_zp.argtypes = [P, I64, I64, F, P, P, P, P, P, P, SZ, P]
    lib.llmint8_matmul_zp.argtypes = [P, I64, I64, I64, P, P, P, P, P, F, P, P, SZ, P]
    lib.llmint8_matmul_zp_path.argtypes = [P, I64, I64, I64, P, P, P, P, P, F, P, P, SZ, I, P,
                                           P, P]
    for f8 in ("f8", "e4m3"):
        getattr(lib, "llmint8_quantize_weight_" + f8).argtypes = [P, I64, I64, P, P, P]
        getattr(lib, "llmint8_quantize_act_" + f8).argtypes = [P, I64, I64, F, P, P, P, P, P, SZ,
                                                               P]
        getattr(lib, "llmint8_matmul_" + f8).argtypes = [P, I64, I64, I64, P, P, P, F, P, P, SZ,
                                                         P]
        getattr(lib, "llmint8_matmul_%s_path" % f8).argtypes = [P, I64, I64, I64, P, P, P, F, P,
                                                                P, SZ, I, P, P, P]
    lib.llmint8_mfma_ceiling.argtypes = [P, I64, P, I64, I64, I, I, I, P, P, P, P]
    lib.llmint8_matmul_noalloc.argtypes = [P, I64, I64, I64, P, P, P, F, P, P]
    for fn in ("llmint8_quantize_weight", "llmint8_quantize_act", "llmint8_matmul",
               "llmint8_matmul_act", "llmint8_matmul_path", "llmint8_igemm_i32",
               "llmint8_quantize_weight_zp", "llmint8_quantize_act_zp", "llmint8_matmul_zp",
               "llmint8_matmul_zp_path", "llmint8_quantize_weight_f8", "llmint8_quantize_act_f8",
               "llmint8_matmul_f8", "llmint8_matmul_f8_path", "llmint8_quantize_weight_e4m3",
               "llmint8_quantize_act_e4m3", "llmint8_matmul_e4m3", "llmint8_matmul_e4m3_path",
               "llmint8_mfma_ceiling", "llmint8_matmul_noalloc"):
        getattr(lib, fn).restype = I
    _lib = lib
    return lib


def _check(fn, rc):
    if rc != LLMINT8_OK:
        raise LLMInt8Error(fn, rc)


def _arg(t, name, dtypes, shape=None, min_numel=None):
    """Check a tensor argument before its pointer reaches the library: type,
    dtype, shape (or at least min_numel elements) and contiguity.  A mismatch
    raises TypeError (type, dtype) or ValueError.  That it is device memory is
    checked by _on_device once every argument has passed these checks."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError("%s holds %d elements, at least %d are needed" % (name, t.numel(), min_numel))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _on_device(**tensors):
    """Every tensor argument (None = absent) must be device memory on one device."""
    devs = set()
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError("%s must be a device (cuda) tensor" % name)
        devs.add(t.device)
    if len(devs) > 1:
        raise ValueError("tensor arguments are on different devices: %s" % sorted(map(str, devs)))


def _new_or(t, name, dtypes, shape, device, min_numel=None):
    """The caller's tensor, checked, or a new device tensor of `shape`."""
    if t is None:
        return torch.empty(shape, dtype=dtypes[0], device=device)
    return _arg(t, name, dtypes, shape=None if min_numel is not None else shape,
                min_numel=min_numel)


def _ws(ws, need, device):
    """The caller's workspace (a contiguous device tensor; the library checks
    its size), or a new one of `need` bytes."""
    if ws is None:
        return torch.empty((need,), dtype=torch.uint8, device=device)
    return _arg(ws, "ws", (torch.uint8, torch.int8))


def _matmul_operands(X, CB, SCB, bias, cb_dtypes, scb_name="SCB"):
    """Shapes of a matmul call: X [T,K] fp16, CB [N,K], the per-column vector
    SCB [N] f32, bias [N] fp16 or None."""
    _arg(X, "X", _H)
    if X.dim() != 2:
        raise ValueError("X must be 2-D [T,K], got shape %s" % (tuple(X.shape),))
    T, K = X.shape
    _arg(CB, "CB", cb_dtypes)
    if CB.dim() != 2 or CB.shape[1] != K:
        raise ValueError("shape mismatch: X %s, CB %s" % (tuple(X.shape), tuple(CB.shape)))
    N = CB.shape[0]
    _arg(SCB, scb_name, (torch.float32,), shape=(N,))
    if bias is not None:
        _arg(bias, "bias", _H, shape=(N,))
    return T, K, N


_H = (torch.float16, torch.int16)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ev(e):
    return ctypes.c_void_p(e) if e else None


def _ptr(t):
    return t.data_ptr() if t is not None else None


def _nbytes(t):
    return t.numel() * t.element_size()


def llmint8_status_string(status):
    return _load().llmint8_status_string(int(status)).decode()


def llmint8_workspace_bytes(T, K, N):
    return int(_load().llmint8_workspace_bytes(T, K, N))


def llmint8_workspace_bytes_path(T, K, N, path=PATH_AUTO):
    return int(_load().llmint8_workspace_bytes_path(T, K, N, int(path)))


def llmint8_quantize_act_workspace_bytes(K):
    return int(_load().llmint8_quantize_act_workspace_bytes(K))


def llmint8_quantize_weight(W_t, CB=None, SCB=None):
    """W_t: fp16 [N,K] (the nn.Linear weight layout).  Returns (CB int8 [N,K], SCB f32 [N])."""
    lib = _load()
    _arg(W_t, "W_t", _H)
    N, K = W_t.shape
    CB = _new_or(CB, "CB", (torch.int8,), (N, K), W_t.device)
    SCB = _new_or(SCB, "SCB", (torch.float32,), (N,), W_t.device)
    _on_device(W_t=W_t, CB=CB, SCB=SCB)
    _check("llmint8_quantize_weight",
           lib.llmint8_quantize_weight(W_t.data_ptr(), K, N, CB.data_ptr(), SCB.data_ptr(), _stream(W_t)))
    return CB, SCB


def llmint8_quantize_act(X, threshold=6.0, Xq=None, row_absmax=None, outlier_idx=None,
                         n_outliers=None, ws=None):
    """X: fp16 [T,K].  Returns (Xq int8 [T,K], row_absmax f32 [T], outlier_idx int32 [K],
    n_outliers int32 [1]); outlier_idx[:n] is the ascending outlier column list."""
    lib = _load()
    _arg(X, "X", _H)
    T, K = X.shape
    d = X.device
    Xq = _new_or(Xq, "Xq", (torch.int8,), (T, K), d)
    row_absmax = _new_or(row_absmax, "row_absmax", (torch.float32,), (T,), d, min_numel=T)
    outlier_idx = _new_or(outlier_idx, "outlier_idx", (torch.int32,), (K,), d, min_numel=K)
    n_outliers = _new_or(n_outliers, "n_outliers", (torch.int32,), (1,), d, min_numel=1)
    ws = _ws(ws, llmint8_quantize_act_workspace_bytes(K), d)
    _on_device(X=X, Xq=Xq, row_absmax=row_absmax, outlier_idx=outlier_idx, n_outliers=n_outliers, ws=ws)
    _check("llmint8_quantize_act",
           lib.llmint8_quantize_act(X.data_ptr(), T, K, float(threshold), Xq.data_ptr(),
                                    row_absmax.data_ptr(), outlier_idx.data_ptr(),
                                    n_outliers.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                                    _stream(X)))
    return Xq, row_absmax, outlier_idx, n_outliers


def llmint8_matmul_path(X, CB, SCB, threshold=6.0, bias=None, out=None, ws=None, path=PATH_AUTO,
                        main_start=None, main_stop=None):
    """X fp16 [T,K], CB int8 [N,K], SCB f32 [N], bias fp16 [N] or None -> out fp16 [T,N].

    main_start / main_stop: optional raw hipEvent_t handles (ints) recorded
    around the main kernel's launch."""
    lib = _load()
    T, K, N = _matmul_operands(X, CB, SCB, bias, (torch.int8,))
    out = _new_or(out, "out", _H, (T, N), X.device)
    ws = _ws(ws, llmint8_workspace_bytes_path(T, K, N, path), X.device)
    _on_device(X=X, CB=CB, SCB=SCB, bias=bias, out=out, ws=ws)
    _check("llmint8_matmul_path",
           lib.llmint8_matmul_path(X.data_ptr(), T, K, N, CB.data_ptr(), SCB.data_ptr(), _ptr(bias),
                                   float(threshold), out.data_ptr(), ws.data_ptr(), _nbytes(ws),
                                   int(path), _ev(main_start), _ev(main_stop), _stream(X)))
    return out


def llmint8_matmul(X, CB, SCB, threshold=6.0, bias=None, out=None, ws=None):
    """The LLM.int8() decomposition matmul; see llmint8_matmul_path."""
    lib = _load()
    T, K, N = _matmul_operands(X, CB, SCB, bias, (torch.int8,))
    out = _new_or(out, "out", _H, (T, N), X.device)
    ws = _ws(ws, llmint8_workspace_bytes(T, K, N), X.device)
    _on_device(X=X, CB=CB, SCB=SCB, bias=bias, out=out, ws=ws)
    _check("llmint8_matmul",
           lib.llmint8_matmul(X.data_ptr(), T, K, N, CB.data_ptr(), SCB.data_ptr(), _ptr(bias),
                              float(threshold), out.data_ptr(), ws.data_ptr(), _nbytes(ws),
                              _stream(X)))
    return out


def llmint8_matmul_act(X, CB, SCB, threshold=6.0, activation=ACT_NONE, bias=None, out=None,
                       ws=None):
    """llmint8_matmul with the output activation (ACT_NONE or ACT_RELU) fused."""
    lib = _load()
    T, K, N = _matmul_operands(X, CB, SCB, bias, (torch.int8,))
    out = _new_or(out, "out", _H, (T, N), X.device)
    ws = _ws(ws, llmint8_workspace_bytes(T, K, N), X.device)
    _on_device(X=X, CB=CB, SCB=SCB, bias=bias, out=out, ws=ws)
    _check("llmint8_matmul_act",
           lib.llmint8_matmul_act(X.data_ptr(), T, K, N, CB.data_ptr(), SCB.data_ptr(), _ptr(bias),
                                  float(threshold), int(activation), out.data_ptr(), ws.data_ptr(),
                                  _nbytes(ws), _stream(X)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20   # LLMINT8_NOALLOC_SCRATCH_BYTES


def llmint8_matmul_noalloc(X, CB, SCB, out, threshold=6.0, bias=None):
    """llmint8_matmul on the library's static device scratch instead of a
    workspace (for callers that cannot allocate; calls that overlap on one
    device race).  `out` [T,N] fp16 is required: nothing is allocated here
    either.  Calls whose workspace query exceeds NOALLOC_SCRATCH_BYTES raise
    LLMInt8Error (LLMINT8_ERR_SCRATCH)."""
    lib = _load()
    T, K, N = _matmul_operands(X, CB, SCB, bias, (torch.int8,))
    _arg(out, "out", _H, shape=(T, N))
    _on_device(X=X, CB=CB, SCB=SCB, bias=bias, out=out)
    _check("llmint8_matmul_noalloc",
           lib.llmint8_matmul_noalloc(X.data_ptr(), T, K, N, CB.data_ptr(), SCB.data_ptr(),
                                      _ptr(bias), float(threshold), out.data_ptr(), _stream(X)))
    return out


def llmint8_mfma_ceiling(A, B, blocks, iters, start=None, stop=None):
    """The MFMA rate on the operands' own bits (benchmark hook): A [T,K] and
    B [N,K], both int8 (v_mfma_i32_32x32x32_i8) or both fp16
    (v_mfma_f32_32x32x16_f16); `blocks` workgroups of 4 wavefronts, each
    issuing iters * 32 MFMAs from registers, with optional timing events
    around the launch.  Returns (the per-lane checksums, the ops or flops
    issued)."""
    lib = _load()
    _arg(A, "A", (torch.int8, torch.float16))
    _arg(B, "B", (A.dtype,))
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[1]:
        raise ValueError("shape mismatch: A %s, B %s" % (tuple(A.shape), tuple(B.shape)))
    kind = 1 if A.dtype == torch.float16 else 0
    out = torch.empty((int(blocks) * 256,), dtype=torch.int32, device=A.device)
    _on_device(A=A, B=B, out=out)
    _check("llmint8_mfma_ceiling",
           lib.llmint8_mfma_ceiling(A.data_ptr(), A.shape[0], B.data_ptr(), B.shape[0], A.shape[1],
                                    kind, int(blocks), int(iters), out.data_ptr(), _ev(start),
                                    _ev(stop), _stream(A)))
    per_mfma = 32768 if kind else 65536
    return out, float(blocks) * 4 * iters * 32 * per_mfma


def llmint8_igemm_i32(Xq, CB, C=None, path=PATH_AUTO):
    """C int32 [T,N] = Xq int8 [T,K] @ CB int8 [N,K]^T, exact."""
    lib = _load()
    _arg(Xq, "Xq", (torch.int8,))
    _arg(CB, "CB", (torch.int8,))
    T, K = Xq.shape
    N = CB.shape[0]
    if CB.dim() != 2 or CB.shape[1] != K:
        raise ValueError("shape mismatch: Xq %s, CB %s" % (tuple(Xq.shape), tuple(CB.shape)))
    C = _new_or(C, "C", (torch.int32,), (T, N), Xq.device)
    _on_device(Xq=Xq, CB=CB, C=C)
    _check("llmint8_igemm_i32",
           lib.llmint8_igemm_i32(Xq.data_ptr(), T, K, N, CB.data_ptr(), C.data_ptr(), int(path),
                                 _stream(Xq)))
    return C


# ---------------------------------------------------------------------------
# Zero-point (asymmetric) variant.
# ---------------------------------------------------------------------------
def llmint8_quantize_weight_zp(W_t, CB=None, ND=None, ZP=None, RS=None):
    """W_t: fp16 [N,K].  Returns (CB int8 [N,K], ND f32 [N], ZP int32 [N], RS int32 [N])."""
    lib = _load()
    _arg(W_t, "W_t", _H)
    N, K = W_t.shape
    d = W_t.device
    CB = _new_or(CB, "CB", (torch.int8,), (N, K), d)
    ND = _new_or(ND, "ND", (torch.float32,), (N,), d)
    ZP = _new_or(ZP, "ZP", (torch.int32,), (N,), d)
    RS = _new_or(RS, "RS", (torch.int32,), (N,), d)
    _on_device(W_t=W_t, CB=CB, ND=ND, ZP=ZP, RS=RS)
    _check("llmint8_quantize_weight_zp",
           lib.llmint8_quantize_weight_zp(W_t.data_ptr(), K, N, CB.data_ptr(), ND.data_ptr(),
                                          ZP.data_ptr(), RS.data_ptr(), _stream(W_t)))
    return CB, ND, ZP, RS


def llmint8_quantize_act_zp(X, threshold=6.0, Xq=None, nd=None, row_zp=None, outlier_idx=None,
                            n_outliers=None, ws=None):
    """X: fp16 [T,K].  Returns (Xq int8 [T,K], nd f32 [T], row_zp int32 [T,2] = {zp, code sum},
    outlier_idx int32 [K], n_outliers int32 [1])."""
    lib = _load()
    _arg(X, "X", _H)
    T, K = X.shape
    d = X.device
    Xq = _new_or(Xq, "Xq", (torch.int8,), (T, K), d)
    nd = _new_or(nd, "nd", (torch.float32,), (T,), d, min_numel=T)
    row_zp = _new_or(row_zp, "row_zp", (torch.int32,), (T, 2), d, min_numel=2 * T)
    outlier_idx = _new_or(outlier_idx, "outlier_idx", (torch.int32,), (K,), d, min_numel=K)
    n_outliers = _new_or(n_outliers, "n_outliers", (torch.int32,), (1,), d, min_numel=1)
    ws = _ws(ws, llmint8_quantize_act_workspace_bytes(K), d)
    _on_device(X=X, Xq=Xq, nd=nd, row_zp=row_zp, outlier_idx=outlier_idx, n_outliers=n_outliers, ws=ws)
    _check("llmint8_quantize_act_zp",
           lib.llmint8_quantize_act_zp(X.data_ptr(), T, K, float(threshold), Xq.data_ptr(),
                                       nd.data_ptr(), row_zp.data_ptr(), outlier_idx.data_ptr(),
                                       n_outliers.data_ptr(), ws.data_ptr(),
                                       ws.numel() * ws.element_size(), _stream(X)))
    return Xq, nd, row_zp, outlier_idx, n_outliers


def _zp_operands(X, CB, ND, ZP, RS, bias):
    T, K, N = _matmul_operands(X, CB, ND, bias, (torch.int8,), scb_name="ND")
    _arg(ZP, "ZP", (torch.int32,), shape=(N,))
    _arg(RS, "RS", (torch.int32,), shape=(N,))
    return T, K, N


def llmint8_matmul_zp_path(X, CB, ND, ZP, RS, threshold=6.0, bias=None, out=None, ws=None,
                           path=PATH_AUTO, main_start=None, main_stop=None):
    """The zero-point decomposition: X fp16 [T,K] with the output of
    llmint8_quantize_weight_zp -> out fp16 [T,N].  path / events as
    llmint8_matmul_path."""
    lib = _load()
    T, K, N = _zp_operands(X, CB, ND, ZP, RS, bias)
    out = _new_or(out, "out", _H, (T, N), X.device)
    ws = _ws(ws, llmint8_workspace_bytes_path(T, K, N, path), X.device)
    _on_device(X=X, CB=CB, ND=ND, ZP=ZP, RS=RS, bias=bias, out=out, ws=ws)
    _check("llmint8_matmul_zp_path",
           lib.llmint8_matmul_zp_path(X.data_ptr(), T, K, N, CB.data_ptr(), ND.data_ptr(),
                                      ZP.data_ptr(), RS.data_ptr(), _ptr(bias), float(threshold),
                                      out.data_ptr(), ws.data_ptr(), _nbytes(ws), int(path),
                                      _ev(main_start), _ev(main_stop), _stream(X)))
    return out


def llmint8_matmul_zp(X, CB, ND, ZP, RS, threshold=6.0, bias=None, out=None, ws=None):
    """The zero-point decomposition (automatic kernel choice)."""
    lib = _load()
    T, K, N = _zp_operands(X, CB, ND, ZP, RS, bias)
    out = _new_or(out, "out", _H, (T, N), X.device)
    ws = _ws(ws, llmint8_workspace_bytes(T, K, N), X.device)
    _on_device(X=X, CB=CB, ND=ND, ZP=ZP, RS=RS, bias=bias, out=out, ws=ws)
    _check("llmint8_matmul_zp",
           lib.llmint8_matmul_zp(X.data_ptr(), T, K, N, CB.data_ptr(), ND.data_ptr(), ZP.data_ptr(),
                                 RS.data_ptr(), _ptr(bias), float(threshold), out.data_ptr(),
                                 ws.data_ptr(), _nbytes(ws), _stream(X)))
    return out


# ---------------------------------------------------------------------------
# FP8 variant: E5M2 (the _f8 functions) and E4M3 (the _e4m3 functions), the
# same arguments; the format only changes which library symbols are called.
# ---------------------------------------------------------------------------
def _quantize_weight_fp8(fmt, W_t, CB8, SC8):
    lib = _load()
    _arg(W_t, "W_t", _H)
    N, K = W_t.shape
    d = W_t.device
    CB8 = _new_or(CB8, "CB8", (torch.uint8,), (N, K), d)
    SC8 = _new_or(SC8, "SC8", (torch.float32,), (N,), d)
    _on_device(W_t=W_t, CB8=CB8, SC8=SC8)
    fn = "llmint8_quantize_weight_" + fmt
    _check(fn, getattr(lib, fn)(W_t.data_ptr(), K, N, CB8.data_ptr(), SC8.data_ptr(),
                                _stream(W_t)))
    return CB8, SC8


def _quantize_act_fp8(fmt, X, threshold, Xq8, row_scale, outlier_idx, n_outliers, ws):
    lib = _load()
    _arg(X, "X", _H)
    T, K = X.shape
    d = X.device
    Xq8 = _new_or(Xq8, "Xq8", (torch.uint8,), (T, K), d)
    row_scale = _new_or(row_scale, "row_scale", (torch.float32,), (T,), d, min_numel=T)
    outlier_idx = _new_or(outlier_idx, "outlier_idx", (torch.int32,), (K,), d, min_numel=K)
    n_outliers = _new_or(n_outliers, "n_outliers", (torch.int32,), (1,), d, min_numel=1)
    ws = _ws(ws, llmint8_quantize_act_workspace_bytes(K), d)
    _on_device(X=X, Xq8=Xq8, row_scale=row_scale, outlier_idx=outlier_idx, n_outliers=n_outliers, ws=ws)
    fn = "llmint8_quantize_act_" + fmt
    _check(fn, getattr(lib, fn)(X.data_ptr(), T, K, float(threshold), Xq8.data_ptr(),
                                row_scale.data_ptr(), outlier_idx.data_ptr(),
                                n_outliers.data_ptr(), ws.data_ptr(),
                                ws.numel() * ws.element_size(), _stream(X)))
    return Xq8, row_scale, outlier_idx, n_outliers


def _f8_operands(X, CB8, SC8, bias, out, ws, path=PATH_AUTO):
    T, K, N = _matmul_operands(X, CB8, SC8, bias, (torch.uint8,), scb_name="SC8")
    out = _new_or(out, "out", _H, (T, N), X.device)
    ws = _ws(ws, llmint8_workspace_bytes_path(T, K, N, path), X.device)
    return T, K, N, out, ws


def _matmul_fp8_path(fmt, X, CB8, SC8, threshold, bias, out, ws, path, main_start, main_stop):
    lib = _load()
    T, K, N, out, ws = _f8_operands(X, CB8, SC8, bias, out, ws, path)
    _on_device(X=X, CB8=CB8, SC8=SC8, bias=bias, out=out, ws=ws)
    fn = "llmint8_matmul_%s_path" % fmt
    _check(fn, getattr(lib, fn)(X.data_ptr(), T, K, N, CB8.data_ptr(), SC8.data_ptr(),
                                _ptr(bias), float(threshold), out.data_ptr(), ws.data_ptr(),
                                _nbytes(ws), int(path), _ev(main_start), _ev(main_stop),
                                _stream(X)))
    return out


def _matmul_fp8(fmt, X, CB8, SC8, threshold, bias, out, ws):
    lib = _load()
    T, K, N, out, ws = _f8_operands(X, CB8, SC8, bias, out, ws)
    _on_device(X=X, CB8=CB8, SC8=SC8, bias=bias, out=out, ws=ws)
    fn = "llmint8_matmul_" + fmt
    _check(fn, getattr(lib, fn)(X.data_ptr(), T, K, N, CB8.data_ptr(), SC8.data_ptr(),
                                _ptr(bias), float(threshold), out.data_ptr(), ws.data_ptr(),
                                _nbytes(ws), _stream(X)))
    return out


def llmint8_quantize_weight_f8(W_t, CB8=None, SC8=None):
    """W_t: fp16 [N,K].  Returns (CB8 uint8 [N,K] E5M2 codes, SC8 f32 [N] scales 2^-e)."""
    return _quantize_weight_fp8("f8", W_t, CB8, SC8)


def llmint8_quantize_act_f8(X, threshold=6.0, Xq8=None, row_scale=None, outlier_idx=None,
                            n_outliers=None, ws=None):
    """X: fp16 [T,K].  Returns (Xq8 uint8 [T,K] E5M2 codes, row_scale f32 [T], outlier_idx
    int32 [K], n_outliers int32 [1])."""
    return _quantize_act_fp8("f8", X, threshold, Xq8, row_scale, outlier_idx, n_outliers, ws)


def llmint8_matmul_f8_path(X, CB8, SC8, threshold=6.0, bias=None, out=None, ws=None,
                           path=PATH_AUTO, main_start=None, main_stop=None):
    """The FP8 decomposition: X fp16 [T,K] with the output of
    llmint8_quantize_weight_f8 -> out fp16 [T,N]; path / events as llmint8_matmul_path."""
    return _matmul_fp8_path("f8", X, CB8, SC8, threshold, bias, out, ws, path, main_start,
                            main_stop)


def llmint8_matmul_f8(X, CB8, SC8, threshold=6.0, bias=None, out=None, ws=None):
    """The FP8 decomposition (automatic kernel choice)."""
    return _matmul_fp8("f8", X, CB8, SC8, threshold, bias, out, ws)


def llmint8_quantize_weight_e4m3(W_t, CB8=None, SC8=None):
    """W_t: fp16 [N,K].  Returns (CB8 uint8 [N,K] E4M3 codes, SC8 f32 [N] scales 2^-e)."""
    return _quantize_weight_fp8("e4m3", W_t, CB8, SC8)


def llmint8_quantize_act_e4m3(X, threshold=6.0, Xq8=None, row_scale=None, outlier_idx=None,
                              n_outliers=None, ws=None):
    """X: fp16 [T,K].  Returns (Xq8 uint8 [T,K] E4M3 codes, row_scale f32 [T], outlier_idx
    int32 [K], n_outliers int32 [1])."""
    return _quantize_act_fp8("e4m3", X, threshold, Xq8, row_scale, outlier_idx, n_outliers, ws)


def llmint8_matmul_e4m3_path(X, CB8, SC8, threshold=6.0, bias=None, out=None, ws=None,
                             path=PATH_AUTO, main_start=None, main_stop=None):
    """The E4M3 decomposition: X fp16 [T,K] with the output of
    llmint8_quantize_weight_e4m3 -> out fp16 [T,N]; path / events as llmint8_matmul_path."""
    return _matmul_fp8_path("e4m3", X, CB8, SC8, threshold, bias, out, ws, path, main_start,
                            main_stop)


def llmint8_matmul_e4m3(X, CB8, SC8, threshold=6.0, bias=None, out=None, ws=None):
    """The E4M3 decomposition (automatic kernel choice)."""
    return _matmul_fp8("e4m3", X, CB8, SC8, threshold, bias, out, ws)
