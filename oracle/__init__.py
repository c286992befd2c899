"""Plain CPU oracle of the LLM.int8() mixed-precision decomposition matmul.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg are the only callers.  The HIP library never imports, links or
runs anything here, and this package never imports the HIP library.

The arithmetic lives in ``llmint8_oracle.c`` (plain C, one output element at
a time); this module only marshals numpy arrays through ctypes.  fp16 data is
passed as raw binary16 bit patterns (``uint16``); ``np.float16`` arrays are
accepted and reinterpreted.

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_*.py`` (worked examples printed on the pages, closed
forms, special cases and brute force); the zero-point variant's functions by
``tests/test_oracle_zeropoint.py``, the FP8 variant's by ``tests/test_oracle_fp8.py``.  The one part without a pin to an
independent value is the fp64 summation order of the fp16 outlier product,
which sits far below the fp16 output tolerance.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "llmint8_oracle.c")
_SO = os.path.join(_HERE, "libllmint8_oracle.so")

_lib = None


def build():
    """Compile the oracle shared library with gcc (IEEE arithmetic, OpenMP)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", "-shared", "-fPIC", _SRC, "-o", _SO + ".tmp",
           "-lm"]
    subprocess.check_call(cmd)
    os.replace(_SO + ".tmp", _SO)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO):
        build()
    lib = ctypes.CDLL(_SO)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_half_to_double_n.argtypes = [P, I64, P]
    lib.oracle_double_to_half_n.argtypes = [P, I64, P]
    lib.oracle_round_127x_over_a_n.argtypes = [P, P, I64, P]
    lib.oracle_dequant_weight_n.argtypes = [P, P, I64, P]
    lib.oracle_quantize_weight.argtypes = [P, I64, I64, P, P]
    lib.oracle_outlier_columns.argtypes = [P, I64, I64, ctypes.c_float, P]
    lib.oracle_outlier_columns.restype = I64
    lib.oracle_quantize_rows.argtypes = [P, I64, I64, P, I64, P, I64, P, P]
    lib.oracle_int_gemm.argtypes = [P, P, I64, I64, I64, P]
    lib.oracle_int_gemm.restype = I64
    lib.oracle_matmul.argtypes = [P, I64, I64, I64, P, P, P, ctypes.c_float,
                                  P, I64, P, I64, P, P, P, P]
    lib.oracle_matmul.restype = I64
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_dequant_weight_zp_n.argtypes = [P, P, P, I64, P]
    lib.oracle_quantize_weight_zp.argtypes = [P, I64, I64, P, P, P]
    lib.oracle_quantize_rows_zp.argtypes = [P, I64, I64, P, I64, P, I64, P, P, P]
    lib.oracle_matmul_zp.argtypes = [P, I64, I64, I64, P, P, P, P, ctypes.c_float,
                                     P, I64, P, I64, P, P, P, P, P]
    lib.oracle_matmul_zp.restype = I64
    lib.oracle_e5m2_to_double_n.argtypes = [P, I64, P]
    lib.oracle_double_to_e5m2_n.argtypes = [P, I64, P]
    lib.oracle_f8_scale_exp_n.argtypes = [P, I64, P]
    lib.oracle_quantize_weight_f8.argtypes = [P, I64, I64, P, P]
    lib.oracle_quantize_rows_f8.argtypes = [P, I64, I64, P, I64, P, I64, P, P]
    lib.oracle_matmul_f8.argtypes = [P, I64, I64, I64, P, P, P, ctypes.c_float,
                                     P, I64, P, I64, P, P, P, P]
    lib.oracle_e4m3_to_double_n.argtypes = [P, I64, P]
    lib.oracle_double_to_e4m3_n.argtypes = [P, I64, P]
    lib.oracle_f8_scale_exp_fmt_n.argtypes = [P, I64, P, ctypes.c_int]
    lib.oracle_quantize_weight_f8_fmt.argtypes = [P, I64, I64, P, P, ctypes.c_int]
    lib.oracle_quantize_rows_f8_fmt.argtypes = [P, I64, I64, P, I64, P, I64, P, P, ctypes.c_int]
    lib.oracle_matmul_f8_fmt.argtypes = [P, I64, I64, I64, P, P, P, ctypes.c_float,
                                         P, I64, P, I64, P, P, P, P, ctypes.c_int]
    _lib = lib
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _bits(a):
    """Binary16 bit patterns of an fp16 (or already uint16) array."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("expected float16 or uint16 bit patterns, got %s" % a.dtype)
    return a


def num_threads():
    return int(_load().oracle_num_threads())


def half_to_double(h):
    h = _bits(h)
    out = np.empty(h.shape, np.float64)
    _load().oracle_half_to_double_n(_ptr(h), h.size, _ptr(out))
    return out


def double_to_half(v):
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().oracle_double_to_half_n(_ptr(v), v.size, _ptr(out))
    return out


def round_127x_over_a(x, a):
    """Nearest integer (ties to even) to 127*x/a for binary16 x, a."""
    x, a = np.broadcast_arrays(_bits(x), _bits(a))
    x = np.ascontiguousarray(x)
    a = np.ascontiguousarray(a)
    out = np.empty(x.shape, np.int32)
    _load().oracle_round_127x_over_a_n(_ptr(x), _ptr(a), x.size, _ptr(out))
    return out


def dequant_weight(cb, scb):
    """Binary16 value nearest to cb*scb/127, element-wise."""
    cb, scb = np.broadcast_arrays(np.asarray(cb, np.int8), np.asarray(scb, np.float32))
    cb = np.ascontiguousarray(cb)
    scb = np.ascontiguousarray(scb)
    out = np.empty(cb.shape, np.uint16)
    _load().oracle_dequant_weight_n(_ptr(cb), _ptr(scb), cb.size, _ptr(out))
    return out


def quantize_weight(W_t):
    """W_t: [N,K] fp16 (row n = output column n).  Returns (CB [N,K] int8, SCB [N] f32)."""
    W_t = _bits(W_t)
    N, K = W_t.shape
    CB = np.empty((N, K), np.int8)
    SCB = np.empty((N,), np.float32)
    _load().oracle_quantize_weight(_ptr(W_t), K, N, _ptr(CB), _ptr(SCB))
    return CB, SCB


def outlier_columns(X, threshold):
    """Ascending int32 array of the columns whose max |x| exceeds threshold."""
    X = _bits(X)
    T, K = X.shape
    O = np.empty((max(K, 1),), np.int32)
    n = _load().oracle_outlier_columns(_ptr(X), T, K, float(threshold), _ptr(O))
    return O[:n].copy()


def quantize_rows(X, O, rows=None):
    """Returns (Xq [nrows,K] int8, a [nrows] f32) for the listed rows (all by default)."""
    X = _bits(X)
    T, K = X.shape
    O = np.ascontiguousarray(O, np.int32)
    if rows is None:
        nrows = T
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(rows, np.int64)
        nrows = rows_arr.size
    Xq = np.empty((nrows, K), np.int8)
    a = np.empty((nrows,), np.float32)
    _load().oracle_quantize_rows(_ptr(X), T, K, _ptr(O), O.size, _ptr(rows_arr),
                                 nrows, _ptr(Xq), _ptr(a))
    return Xq, a


def int_gemm(Xq, CB):
    """C[i,n] = sum_k Xq[i,k]*CB[n,k] (int64 sums, returned as int32)."""
    Xq = np.ascontiguousarray(Xq, np.int8)
    CB = np.ascontiguousarray(CB, np.int8)
    M, K = Xq.shape
    N, K2 = CB.shape
    assert K == K2
    C = np.empty((M, N), np.int32)
    bad = _load().oracle_int_gemm(_ptr(Xq), _ptr(CB), M, K, N, _ptr(C))
    if bad:
        raise OverflowError("%d int32 overflows in the integer product" % bad)
    return C


def relu_half(h):
    """ReLU on binary16 bit patterns: every value with the sign bit set
    (negative numbers, -0, -inf) becomes +0, the rest is unchanged.  Rounding
    to nearest is monotone and maps 0 to 0, so relu(fp16(v)) = fp16(max(v, 0))
    for every real v: applying it to the rounded output is the ReLU of the
    exact output, rounded once."""
    h = np.ascontiguousarray(h).view(np.uint16)
    return np.where(h & np.uint16(0x8000), np.uint16(0), h).astype(np.uint16)


def matmul(X, CB, SCB, threshold=6.0, bias=None, rows=None, cols=None, relu=False):
    """The decomposition for the listed output rows/columns (relu: followed
    by the layer's ReLU, as the feed-forward expansion layers have it).

    Returns (out [nrows,ncols] uint16 binary16 bits, O int32, a [nrows] f32).
    O is always found from all rows of X.
    """
    X = _bits(X)
    T, K = X.shape
    CB = np.ascontiguousarray(CB, np.int8)
    SCB = np.ascontiguousarray(SCB, np.float32)
    N = CB.shape[0]
    assert CB.shape == (N, K) and SCB.shape == (N,)
    b = _bits(bias) if bias is not None else None
    rows_arr = None if rows is None else np.ascontiguousarray(rows, np.int64)
    cols_arr = None if cols is None else np.ascontiguousarray(cols, np.int64)
    nrows = T if rows_arr is None else rows_arr.size
    ncols = N if cols_arr is None else cols_arr.size
    out = np.empty((nrows, ncols), np.uint16)
    O = np.empty((max(K, 1),), np.int32)
    n = np.zeros((1,), np.int64)
    a = np.empty((max(nrows, 1),), np.float32)
    bad = _load().oracle_matmul(_ptr(X), T, K, N, _ptr(CB), _ptr(SCB), _ptr(b),
                                float(threshold), _ptr(rows_arr), nrows,
                                _ptr(cols_arr), ncols, _ptr(out), _ptr(O),
                                _ptr(n), _ptr(a))
    if bad:
        raise OverflowError("%d int32 overflows in the integer product" % bad)
    if relu:
        out = relu_half(out)
    return out, O[: int(n[0])].copy(), a[:nrows].copy()


# ---------------------------------------------------------------------------
# Zero-point (asymmetric) vector-wise variant.  The readings of the page's
# garbled zero-point formulas are stated in llmint8_oracle.c; in short, per
# vector: range [min(min,0), max(max,0)], d = max' - min', nd = 254/d exact,
# zp = RNE(nd*min') + 127, code = RNE(nd*x) - zp (exact rationals rounded,
# ties to even), x ~= (code + zp) / nd; the stored nd is the nearest fp32.
# ---------------------------------------------------------------------------
def dequant_weight_zp(cb, zp, nd):
    """Binary16 value of fp32((cb + zp) / nd), element-wise (0 where nd = 0)."""
    cb, zp, nd = np.broadcast_arrays(np.asarray(cb, np.int8), np.asarray(zp, np.int32),
                                     np.asarray(nd, np.float32))
    cb, zp, nd = (np.ascontiguousarray(v) for v in (cb, zp, nd))
    out = np.empty(cb.shape, np.uint16)
    _load().oracle_dequant_weight_zp_n(_ptr(cb), _ptr(zp), _ptr(nd), cb.size, _ptr(out))
    return out


def quantize_weight_zp(W_t):
    """W_t: [N,K] fp16.  Returns (CB [N,K] int8, ND [N] f32, ZP [N] int32)."""
    W_t = _bits(W_t)
    N, K = W_t.shape
    CB = np.empty((N, K), np.int8)
    ND = np.empty((N,), np.float32)
    ZP = np.empty((N,), np.int32)
    _load().oracle_quantize_weight_zp(_ptr(W_t), K, N, _ptr(CB), _ptr(ND), _ptr(ZP))
    return CB, ND, ZP


def quantize_rows_zp(X, O, rows=None):
    """Returns (Xq [nrows,K] int8, nd [nrows] f32, zp [nrows] int32) for the
    listed rows (all by default); outlier columns hold -zp."""
    X = _bits(X)
    T, K = X.shape
    O = np.ascontiguousarray(O, np.int32)
    rows_arr = None if rows is None else np.ascontiguousarray(rows, np.int64)
    nrows = T if rows_arr is None else rows_arr.size
    Xq = np.empty((nrows, K), np.int8)
    nd = np.empty((nrows,), np.float32)
    zp = np.empty((nrows,), np.int32)
    _load().oracle_quantize_rows_zp(_ptr(X), T, K, _ptr(O), O.size, _ptr(rows_arr), nrows,
                                    _ptr(Xq), _ptr(nd), _ptr(zp))
    return Xq, nd, zp


def matmul_zp(X, CB, ND, ZP, threshold=6.0, bias=None, rows=None, cols=None):
    """The decomposition with zero-point quantization on both operands, for
    the listed output rows/columns.  Returns (out [nrows,ncols] uint16
    binary16 bits, O int32, nd [nrows] f32, zp [nrows] int32)."""
    X = _bits(X)
    T, K = X.shape
    CB = np.ascontiguousarray(CB, np.int8)
    ND = np.ascontiguousarray(ND, np.float32)
    ZP = np.ascontiguousarray(ZP, np.int32)
    N = CB.shape[0]
    assert CB.shape == (N, K) and ND.shape == (N,) and ZP.shape == (N,)
    b = _bits(bias) if bias is not None else None
    rows_arr = None if rows is None else np.ascontiguousarray(rows, np.int64)
    cols_arr = None if cols is None else np.ascontiguousarray(cols, np.int64)
    nrows = T if rows_arr is None else rows_arr.size
    ncols = N if cols_arr is None else cols_arr.size
    out = np.empty((nrows, ncols), np.uint16)
    O = np.empty((max(K, 1),), np.int32)
    n = np.zeros((1,), np.int64)
    nd = np.empty((max(nrows, 1),), np.float32)
    zp = np.empty((max(nrows, 1),), np.int32)
    bad = _load().oracle_matmul_zp(_ptr(X), T, K, N, _ptr(CB), _ptr(ND), _ptr(ZP), _ptr(b),
                                   float(threshold), _ptr(rows_arr), nrows, _ptr(cols_arr),
                                   ncols, _ptr(out), _ptr(O), _ptr(n), _ptr(nd), _ptr(zp))
    if bad:
        raise OverflowError("%d int32 overflows in the integer product" % bad)
    return out, O[: int(n[0])].copy(), nd[:nrows].copy(), zp[:nrows].copy()


# ---------------------------------------------------------------------------
# FP8 (E5M2) variant.  Readings in llmint8_oracle.c: per vector a power-of-two
# scale 2^e (the largest e with absmax * 2^e <= 57344), codes = E5M2 nearest
# to x * 2^e, stored scale 2^-e; outlier columns are +0.
# ---------------------------------------------------------------------------
def e5m2_to_double(c):
    c = np.ascontiguousarray(c, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().oracle_e5m2_to_double_n(_ptr(c), c.size, _ptr(out))
    return out


def double_to_e5m2(v):
    v = np.ascontiguousarray(v, np.float64)
    out = np.empty(v.shape, np.uint8)
    _load().oracle_double_to_e5m2_n(_ptr(v), v.size, _ptr(out))
    return out


def e4m3_to_double(c):
    c = np.ascontiguousarray(c, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().oracle_e4m3_to_double_n(_ptr(c), c.size, _ptr(out))
    return out


def double_to_e4m3(v):
    v = np.ascontiguousarray(v, np.float64)
    out = np.empty(v.shape, np.uint8)
    _load().oracle_double_to_e4m3_n(_ptr(v), v.size, _ptr(out))
    return out


# FP8 formats: E5M2 (the pages' kind) and E4M3 (largest finite 448)
F8_FORMATS = {"e5m2": 1, "e4m3": 2}


def f8_to_double(c, fmt="e5m2"):
    return e4m3_to_double(c) if fmt == "e4m3" else e5m2_to_double(c)


def f8_scale_exp(amax, fmt="e5m2"):
    a = np.ascontiguousarray(amax, np.float64)
    out = np.empty(a.shape, np.int32)
    if fmt == "e5m2":
        _load().oracle_f8_scale_exp_n(_ptr(a), a.size, _ptr(out))
    else:
        _load().oracle_f8_scale_exp_fmt_n(_ptr(a), a.size, _ptr(out), F8_FORMATS[fmt])
    return out


def quantize_weight_f8(W_t, fmt="e5m2"):
    """W_t: [N,K] fp16.  Returns (CB8 [N,K] uint8 codes of the format, SC8 [N] f32 scales 2^-e)."""
    W_t = _bits(W_t)
    N, K = W_t.shape
    CB8 = np.empty((N, K), np.uint8)
    SC8 = np.empty((N,), np.float32)
    _load().oracle_quantize_weight_f8_fmt(_ptr(W_t), K, N, _ptr(CB8), _ptr(SC8), F8_FORMATS[fmt])
    return CB8, SC8


def quantize_rows_f8(X, O, rows=None, fmt="e5m2"):
    """Returns (Xq8 [nrows,K] uint8, sc8 [nrows] f32) for the listed rows."""
    X = _bits(X)
    T, K = X.shape
    O = np.ascontiguousarray(O, np.int32)
    rows_arr = None if rows is None else np.ascontiguousarray(rows, np.int64)
    nrows = T if rows_arr is None else rows_arr.size
    Xq8 = np.empty((nrows, K), np.uint8)
    sc8 = np.empty((nrows,), np.float32)
    _load().oracle_quantize_rows_f8_fmt(_ptr(X), T, K, _ptr(O), O.size, _ptr(rows_arr), nrows,
                                        _ptr(Xq8), _ptr(sc8), F8_FORMATS[fmt])
    return Xq8, sc8


def matmul_f8(X, CB8, SC8, threshold=6.0, bias=None, rows=None, cols=None, fmt="e5m2"):
    """The decomposition with the non-outlier part in FP8 (E5M2, or E4M3 with
    fmt="e4m3").  Returns (out [nrows,ncols] uint16 binary16 bits, O int32,
    sc8 [nrows] f32)."""
    X = _bits(X)
    T, K = X.shape
    CB8 = np.ascontiguousarray(CB8, np.uint8)
    SC8 = np.ascontiguousarray(SC8, np.float32)
    N = CB8.shape[0]
    assert CB8.shape == (N, K) and SC8.shape == (N,)
    b = _bits(bias) if bias is not None else None
    rows_arr = None if rows is None else np.ascontiguousarray(rows, np.int64)
    cols_arr = None if cols is None else np.ascontiguousarray(cols, np.int64)
    nrows = T if rows_arr is None else rows_arr.size
    ncols = N if cols_arr is None else cols_arr.size
    out = np.empty((nrows, ncols), np.uint16)
    O = np.empty((max(K, 1),), np.int32)
    n = np.zeros((1,), np.int64)
    sc = np.empty((max(nrows, 1),), np.float32)
    _load().oracle_matmul_f8_fmt(_ptr(X), T, K, N, _ptr(CB8), _ptr(SC8), _ptr(b),
                                 float(threshold), _ptr(rows_arr), nrows, _ptr(cols_arr), ncols,
                                 _ptr(out), _ptr(O), _ptr(n), _ptr(sc), F8_FORMATS[fmt])
    return out, O[: int(n[0])].copy(), sc[:nrows].copy()
