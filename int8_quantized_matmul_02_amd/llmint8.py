"""Python binding of libllmint8.so: argument marshalling only.

Each function has the name of the C entry point it calls (see
include/llmint8.h for the operation, layouts, ownership and errors).  Every
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
PATH_AUTO, PATH_GEMM, PATH_DECODE = 0, 1, 2
ACT_NONE, ACT_RELU = 0, 1

EXPORTS = (
    "llmint8_status_string",
    "llmint8_workspace_bytes",
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
    lib.llmint8_quantize_weight_f8.argtypes = [P, I64, I64, P, P, P]
    lib.llmint8_quantize_act_f8.argtypes = [P, I64, I64, F, P, P, P, P, P, SZ, P]
    lib.llmint8_matmul_f8.argtypes = [P, I64, I64, I64, P, P, P, F, P, P, SZ, P]
    lib.llmint8_matmul_f8_path.argtypes = [P, I64, I64, I64, P, P, P, F, P, P, SZ, I, P, P, P]
    for fn in ("llmint8_quantize_weight", "llmint8_quantize_act", "llmint8_matmul",
               "llmint8_matmul_act", "llmint8_matmul_path", "llmint8_igemm_i32",
               "llmint8_quantize_weight_zp", "llmint8_quantize_act_zp", "llmint8_matmul_zp",
               "llmint8_matmul_zp_path", "llmint8_quantize_weight_f8", "llmint8_quantize_act_f8",
               "llmint8_matmul_f8", "llmint8_matmul_f8_path"):
        getattr(lib, fn).restype = I
    _lib = lib
    return lib


def _check(fn, rc):
    if rc != LLMINT8_OK:
        raise LLMInt8Error(fn, rc)


def _dev(t, name, dtypes):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device (cuda) tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


_H = (torch.float16, torch.int16)


def llmint8_status_string(status):
    return _load().llmint8_status_string(int(status)).decode()


def llmint8_workspace_bytes(T, K, N):
    return int(_load().llmint8_workspace_bytes(T, K, N))


def llmint8_quantize_act_workspace_bytes(K):
    return int(_load().llmint8_quantize_act_workspace_bytes(K))


def llmint8_quantize_weight(W_t, CB=None, SCB=None):
    """W_t: fp16 [N,K] (the nn.Linear weight layout).  Returns (CB int8 [N,K], SCB f32 [N])."""
    lib = _load()
    _dev(W_t, "W_t", _H)
    N, K = W_t.shape
    CB = torch.empty((N, K), dtype=torch.int8, device=W_t.device) if CB is None else _dev(CB, "CB", (torch.int8,))
    SCB = torch.empty((N,), dtype=torch.float32, device=W_t.device) if SCB is None else _dev(SCB, "SCB", (torch.float32,))
    _check("llmint8_quantize_weight",
           lib.llmint8_quantize_weight(W_t.data_ptr(), K, N, CB.data_ptr(), SCB.data_ptr(), _stream(W_t)))
    return CB, SCB


def llmint8_quantize_act(X, threshold=6.0, Xq=None, row_absmax=None, outlier_idx=None,
                         n_outliers=None, ws=None):
    """X: fp16 [T,K].  Returns (Xq int8 [T,K], row_absmax f32 [T], outlier_idx int32 [K],
    n_outliers int32 [1]); outlier_idx[:n] is the ascending outlier column list."""
    lib = _load()
    _dev(X, "X", _H)
    T, K = X.shape
    d = X.device
    Xq = torch.empty((T, K), dtype=torch.int8, device=d) if Xq is None else _dev(Xq, "Xq", (torch.int8,))
    row_absmax = torch.empty((T,), dtype=torch.float32, device=d) if row_absmax is None else row_absmax
    outlier_idx = torch.empty((K,), dtype=torch.int32, device=d) if outlier_idx is None else outlier_idx
    n_outliers = torch.empty((1,), dtype=torch.int32, device=d) if n_outliers is None else n_outliers
    need = llmint8_quantize_act_workspace_bytes(K)
    ws = torch.empty((need,), dtype=torch.uint8, device=d) if ws is None else ws
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
    _dev(X, "X", _H)
    _dev(CB, "CB", (torch.int8,))
    _dev(SCB, "SCB", (torch.float32,))
    T, K = X.shape
    N = CB.shape[0]
    if CB.shape[1] != K or SCB.shape != (N,):
        raise ValueError("shape mismatch: X %s, CB %s, SCB %s" % (tuple(X.shape), tuple(CB.shape), tuple(SCB.shape)))
    if bias is not None:
        _dev(bias, "bias", _H)
        if bias.shape != (N,):
            raise ValueError("bias must have shape (%d,)" % N)
    out = torch.empty((T, N), dtype=torch.float16, device=X.device) if out is None else _dev(out, "out", _H)
    if ws is None:
        ws = torch.empty((llmint8_workspace_bytes(T, K, N),), dtype=torch.uint8, device=X.device)
    _check("llmint8_matmul_path",
           lib.llmint8_matmul_path(X.data_ptr(), T, K, N, CB.data_ptr(), SCB.data_ptr(),
                                   bias.data_ptr() if bias is not None else None,
                                   float(threshold), out.data_ptr(), ws.data_ptr(),
                                   ws.numel() * ws.element_size(), int(path),
                                   ctypes.c_void_p(main_start) if main_start else None,
                                   ctypes.c_void_p(main_stop) if main_stop else None,
                                   _stream(X)))
    return out


def llmint8_matmul(X, CB, SCB, threshold=6.0, bias=None, out=None, ws=None):
    """The LLM.int8() decomposition matmul; see llmint8_matmul_path."""
    lib = _load()
    _dev(X, "X", _H)
    _dev(CB, "CB", (torch.int8,))
    _dev(SCB, "SCB", (torch.float32,))
    T, K = X.shape
    N = CB.shape[0]
    if CB.shape[1] != K or SCB.shape != (N,):
        raise ValueError("shape mismatch: X %s, CB %s, SCB %s" % (tuple(X.shape), tuple(CB.shape), tuple(SCB.shape)))
    if bias is not None:
        _dev(bias, "bias", _H)
    out = torch.empty((T, N), dtype=torch.float16, device=X.device) if out is None else _dev(out, "out", _H)
    if ws is None:
        ws = torch.empty((llmint8_workspace_bytes(T, K, N),), dtype=torch.uint8, device=X.device)
    _check("llmint8_matmul",
           lib.llmint8_matmul(X.data_ptr(), T, K, N, CB.data_ptr(), SCB.data_ptr(),
                              bias.data_ptr() if bias is not None else None, float(threshold),
                              out.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                              _stream(X)))
    return out


def llmint8_matmul_act(X, CB, SCB, threshold=6.0, activation=ACT_NONE, bias=None, out=None,
                       ws=None):
    """llmint8_matmul with the output activation (ACT_NONE or ACT_RELU) fused."""
    lib = _load()
    _dev(X, "X", _H)
    _dev(CB, "CB", (torch.int8,))
    _dev(SCB, "SCB", (torch.float32,))
    T, K = X.shape
    N = CB.shape[0]
    if CB.shape[1] != K or SCB.shape != (N,):
        raise ValueError("shape mismatch: X %s, CB %s, SCB %s" % (tuple(X.shape), tuple(CB.shape), tuple(SCB.shape)))
    if bias is not None:
        _dev(bias, "bias", _H)
    out = torch.empty((T, N), dtype=torch.float16, device=X.device) if out is None else _dev(out, "out", _H)
    if ws is None:
        ws = torch.empty((llmint8_workspace_bytes(T, K, N),), dtype=torch.uint8, device=X.device)
    _check("llmint8_matmul_act",
           lib.llmint8_matmul_act(X.data_ptr(), T, K, N, CB.data_ptr(), SCB.data_ptr(),
                                  bias.data_ptr() if bias is not None else None, float(threshold),
                                  int(activation), out.data_ptr(), ws.data_ptr(),
                                  ws.numel() * ws.element_size(), _stream(X)))
    return out


def llmint8_igemm_i32(Xq, CB, C=None, path=PATH_AUTO):
    """C int32 [T,N] = Xq int8 [T,K] @ CB int8 [N,K]^T, exact."""
    lib = _load()
    _dev(Xq, "Xq", (torch.int8,))
    _dev(CB, "CB", (torch.int8,))
    T, K = Xq.shape
    N = CB.shape[0]
    if CB.shape[1] != K:
        raise ValueError("shape mismatch: Xq %s, CB %s" % (tuple(Xq.shape), tuple(CB.shape)))
    C = torch.empty((T, N), dtype=torch.int32, device=Xq.device) if C is None else _dev(C, "C", (torch.int32,))
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
    _dev(W_t, "W_t", _H)
    N, K = W_t.shape
    d = W_t.device
    CB = torch.empty((N, K), dtype=torch.int8, device=d) if CB is None else _dev(CB, "CB", (torch.int8,))
    ND = torch.empty((N,), dtype=torch.float32, device=d) if ND is None else _dev(ND, "ND", (torch.float32,))
    ZP = torch.empty((N,), dtype=torch.int32, device=d) if ZP is None else _dev(ZP, "ZP", (torch.int32,))
    RS = torch.empty((N,), dtype=torch.int32, device=d) if RS is None else _dev(RS, "RS", (torch.int32,))
    _check("llmint8_quantize_weight_zp",
           lib.llmint8_quantize_weight_zp(W_t.data_ptr(), K, N, CB.data_ptr(), ND.data_ptr(),
                                          ZP.data_ptr(), RS.data_ptr(), _stream(W_t)))
    return CB, ND, ZP, RS


def llmint8_quantize_act_zp(X, threshold=6.0, Xq=None, nd=None, row_zp=None, outlier_idx=None,
                            n_outliers=None, ws=None):
    """X: fp16 [T,K].  Returns (Xq int8 [T,K], nd f32 [T], row_zp int32 [T,2] = {zp, code sum},
    outlier_idx int32 [K], n_outliers int32 [1])."""
    lib = _load()
    _dev(X, "X", _H)
    T, K = X.shape
    d = X.device
    Xq = torch.empty((T, K), dtype=torch.int8, device=d) if Xq is None else _dev(Xq, "Xq", (torch.int8,))
    nd = torch.empty((T,), dtype=torch.float32, device=d) if nd is None else _dev(nd, "nd", (torch.float32,))
    row_zp = (torch.empty((T, 2), dtype=torch.int32, device=d) if row_zp is None
              else _dev(row_zp, "row_zp", (torch.int32,)))
    outlier_idx = torch.empty((K,), dtype=torch.int32, device=d) if outlier_idx is None else outlier_idx
    n_outliers = torch.empty((1,), dtype=torch.int32, device=d) if n_outliers is None else n_outliers
    need = llmint8_quantize_act_workspace_bytes(K)
    ws = torch.empty((need,), dtype=torch.uint8, device=d) if ws is None else ws
    _check("llmint8_quantize_act_zp",
           lib.llmint8_quantize_act_zp(X.data_ptr(), T, K, float(threshold), Xq.data_ptr(),
                                       nd.data_ptr(), row_zp.data_ptr(), outlier_idx.data_ptr(),
                                       n_outliers.data_ptr(), ws.data_ptr(),
                                       ws.numel() * ws.element_size(), _stream(X)))
    return Xq, nd, row_zp, outlier_idx, n_outliers


def llmint8_matmul_zp_path(X, CB, ND, ZP, RS, threshold=6.0, bias=None, out=None, ws=None,
                           path=PATH_AUTO, main_start=None, main_stop=None):
    """The zero-point decomposition: X fp16 [T,K] with the output of
    llmint8_quantize_weight_zp -> out fp16 [T,N].  path / events as
    llmint8_matmul_path."""
    lib = _load()
    _dev(X, "X", _H)
    _dev(CB, "CB", (torch.int8,))
    _dev(ND, "ND", (torch.float32,))
    _dev(ZP, "ZP", (torch.int32,))
    _dev(RS, "RS", (torch.int32,))
    T, K = X.shape
    N = CB.shape[0]
    if CB.shape[1] != K or ND.shape != (N,) or ZP.shape != (N,) or RS.shape != (N,):
        raise ValueError("shape mismatch: X %s, CB %s, ND %s, ZP %s, RS %s"
                         % (tuple(X.shape), tuple(CB.shape), tuple(ND.shape), tuple(ZP.shape),
                            tuple(RS.shape)))
    if bias is not None:
        _dev(bias, "bias", _H)
        if bias.shape != (N,):
            raise ValueError("bias must have shape (%d,)" % N)
    out = torch.empty((T, N), dtype=torch.float16, device=X.device) if out is None else _dev(out, "out", _H)
    if ws is None:
        ws = torch.empty((llmint8_workspace_bytes(T, K, N),), dtype=torch.uint8, device=X.device)
    _check("llmint8_matmul_zp_path",
           lib.llmint8_matmul_zp_path(X.data_ptr(), T, K, N, CB.data_ptr(), ND.data_ptr(),
                                      ZP.data_ptr(), RS.data_ptr(),
                                      bias.data_ptr() if bias is not None else None,
                                      float(threshold), out.data_ptr(), ws.data_ptr(),
                                      ws.numel() * ws.element_size(), int(path),
                                      ctypes.c_void_p(main_start) if main_start else None,
                                      ctypes.c_void_p(main_stop) if main_stop else None,
                                      _stream(X)))
    return out


def llmint8_matmul_zp(X, CB, ND, ZP, RS, threshold=6.0, bias=None, out=None, ws=None):
    """The zero-point decomposition (automatic kernel choice)."""
    lib = _load()
    _dev(X, "X", _H)
    for t, name, dt in ((CB, "CB", torch.int8), (ND, "ND", torch.float32), (ZP, "ZP", torch.int32),
                        (RS, "RS", torch.int32)):
        _dev(t, name, (dt,))
    T, K = X.shape
    N = CB.shape[0]
    if CB.shape[1] != K or ND.shape != (N,) or ZP.shape != (N,) or RS.shape != (N,):
        raise ValueError("shape mismatch: X %s, CB %s" % (tuple(X.shape), tuple(CB.shape)))
    if bias is not None:
        _dev(bias, "bias", _H)
    out = torch.empty((T, N), dtype=torch.float16, device=X.device) if out is None else _dev(out, "out", _H)
    if ws is None:
        ws = torch.empty((llmint8_workspace_bytes(T, K, N),), dtype=torch.uint8, device=X.device)
    _check("llmint8_matmul_zp",
           lib.llmint8_matmul_zp(X.data_ptr(), T, K, N, CB.data_ptr(), ND.data_ptr(), ZP.data_ptr(),
                                 RS.data_ptr(), bias.data_ptr() if bias is not None else None,
                                 float(threshold), out.data_ptr(), ws.data_ptr(),
                                 ws.numel() * ws.element_size(), _stream(X)))
    return out


# ---------------------------------------------------------------------------
# FP8 (E5M2) variant.
# ---------------------------------------------------------------------------
def llmint8_quantize_weight_f8(W_t, CB8=None, SC8=None):
    """W_t: fp16 [N,K].  Returns (CB8 uint8 [N,K] E5M2 codes, SC8 f32 [N] scales 2^-e)."""
    lib = _load()
    _dev(W_t, "W_t", _H)
    N, K = W_t.shape
    d = W_t.device
    CB8 = torch.empty((N, K), dtype=torch.uint8, device=d) if CB8 is None else _dev(CB8, "CB8", (torch.uint8,))
    SC8 = torch.empty((N,), dtype=torch.float32, device=d) if SC8 is None else _dev(SC8, "SC8", (torch.float32,))
    _check("llmint8_quantize_weight_f8",
           lib.llmint8_quantize_weight_f8(W_t.data_ptr(), K, N, CB8.data_ptr(), SC8.data_ptr(),
                                          _stream(W_t)))
    return CB8, SC8


def llmint8_quantize_act_f8(X, threshold=6.0, Xq8=None, row_scale=None, outlier_idx=None,
                            n_outliers=None, ws=None):
    """X: fp16 [T,K].  Returns (Xq8 uint8 [T,K], row_scale f32 [T], outlier_idx int32 [K],
    n_outliers int32 [1])."""
    lib = _load()
    _dev(X, "X", _H)
    T, K = X.shape
    d = X.device
    Xq8 = torch.empty((T, K), dtype=torch.uint8, device=d) if Xq8 is None else _dev(Xq8, "Xq8", (torch.uint8,))
    row_scale = torch.empty((T,), dtype=torch.float32, device=d) if row_scale is None else row_scale
    outlier_idx = torch.empty((K,), dtype=torch.int32, device=d) if outlier_idx is None else outlier_idx
    n_outliers = torch.empty((1,), dtype=torch.int32, device=d) if n_outliers is None else n_outliers
    need = llmint8_quantize_act_workspace_bytes(K)
    ws = torch.empty((need,), dtype=torch.uint8, device=d) if ws is None else ws
    _check("llmint8_quantize_act_f8",
           lib.llmint8_quantize_act_f8(X.data_ptr(), T, K, float(threshold), Xq8.data_ptr(),
                                       row_scale.data_ptr(), outlier_idx.data_ptr(),
                                       n_outliers.data_ptr(), ws.data_ptr(),
                                       ws.numel() * ws.element_size(), _stream(X)))
    return Xq8, row_scale, outlier_idx, n_outliers


def _f8_operands(X, CB8, SC8, bias, out, ws):
    _dev(X, "X", _H)
    _dev(CB8, "CB8", (torch.uint8,))
    _dev(SC8, "SC8", (torch.float32,))
    T, K = X.shape
    N = CB8.shape[0]
    if CB8.shape[1] != K or SC8.shape != (N,):
        raise ValueError("shape mismatch: X %s, CB8 %s, SC8 %s"
                         % (tuple(X.shape), tuple(CB8.shape), tuple(SC8.shape)))
    if bias is not None:
        _dev(bias, "bias", _H)
        if bias.shape != (N,):
            raise ValueError("bias must have shape (%d,)" % N)
    out = torch.empty((T, N), dtype=torch.float16, device=X.device) if out is None else _dev(out, "out", _H)
    if ws is None:
        ws = torch.empty((llmint8_workspace_bytes(T, K, N),), dtype=torch.uint8, device=X.device)
    return T, K, N, out, ws


def llmint8_matmul_f8_path(X, CB8, SC8, threshold=6.0, bias=None, out=None, ws=None,
                           path=PATH_AUTO, main_start=None, main_stop=None):
    """The FP8 decomposition: X fp16 [T,K] with the output of
    llmint8_quantize_weight_f8 -> out fp16 [T,N]; path / events as llmint8_matmul_path."""
    lib = _load()
    T, K, N, out, ws = _f8_operands(X, CB8, SC8, bias, out, ws)
    _check("llmint8_matmul_f8_path",
           lib.llmint8_matmul_f8_path(X.data_ptr(), T, K, N, CB8.data_ptr(), SC8.data_ptr(),
                                      bias.data_ptr() if bias is not None else None,
                                      float(threshold), out.data_ptr(), ws.data_ptr(),
                                      ws.numel() * ws.element_size(), int(path),
                                      ctypes.c_void_p(main_start) if main_start else None,
                                      ctypes.c_void_p(main_stop) if main_stop else None,
                                      _stream(X)))
    return out


def llmint8_matmul_f8(X, CB8, SC8, threshold=6.0, bias=None, out=None, ws=None):
    """The FP8 decomposition (automatic kernel choice)."""
    lib = _load()
    T, K, N, out, ws = _f8_operands(X, CB8, SC8, bias, out, ws)
    _check("llmint8_matmul_f8",
           lib.llmint8_matmul_f8(X.data_ptr(), T, K, N, CB8.data_ptr(), SC8.data_ptr(),
                                 bias.data_ptr() if bias is not None else None, float(threshold),
                                 out.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                                 _stream(X)))
    return out
