"""GPU parity on the five workloads at their full sizes.

The oracle runs on the full tensors where that takes seconds (weight and
activation quantization, the outlier set) and on a seeded sample of output
rows (rows 0 and T-1 plus random rows) or output columns where the full
product would take minutes; the GPU computes everything, in the launch
configuration the benchmark times, and the sampled part is compared.
"""
import numpy as np
import pytest
import torch

import oracle
from int8_quantized_matmul_02_amd import llmint8 as L
from int8_quantized_matmul_02_amd import workloads
from tests.gpu_helpers import (assert_equal_exact, assert_fp16_close, d2h, h2d, sample_rows, say)

pytestmark = pytest.mark.gpu


def _check_act(Xd, X, thr, what):
    Xq, a, O, n = L.llmint8_quantize_act(Xd, thr)
    Or = oracle.outlier_columns(X, thr)
    Xqr, ar = oracle.quantize_rows(X, Or)
    n_g = int(d2h(n)[0])
    assert n_g == Or.size, "%s: n %d vs %d" % (what, n_g, Or.size)
    assert_equal_exact(d2h(O)[:n_g], Or, what + " O")
    assert_equal_exact(d2h(a), ar, what + " a")
    assert_equal_exact(d2h(Xq), Xqr, what + " Xq")
    return Xq, Xqr, Or


def _full_case(X, W_t, thr, rows, what, check_c=True):
    say("%s: T=%d K=%d N=%d thr=%s" % (what, X.shape[0], X.shape[1], W_t.shape[0], thr))
    Xd = h2d(X)
    CB, SCB = L.llmint8_quantize_weight(h2d(W_t))
    CBr, SCBr = oracle.quantize_weight(W_t)
    assert_equal_exact(d2h(CB), CBr, what + " CB")
    assert_equal_exact(d2h(SCB), SCBr, what + " SCB")
    Xq, Xqr, Or = _check_act(Xd, X, thr, what)
    if check_c:
        C = d2h(L.llmint8_igemm_i32(Xq, CB, path=L.PATH_AUTO))
        assert_equal_exact(C[rows], oracle.int_gemm(Xqr[rows], CBr), what + " C")
    out = d2h(L.llmint8_matmul(Xd, CB, SCB, thr))
    ref, O2, _ = oracle.matmul(X, CBr, SCBr, thr, rows=rows)
    assert_fp16_close(out[rows], ref, what + " out")
    return Or


def test_tiny_both_paths():
    d = workloads.tiny()
    X, W_t, thr = d["X"], d["W_t"], d["threshold"]
    Or = _full_case(X, W_t, thr, np.arange(16), "tiny")
    assert list(Or) == [7, 200]
    CB, SCB = L.llmint8_quantize_weight(h2d(W_t))
    CBr, SCBr = oracle.quantize_weight(W_t)
    ref, _, _ = oracle.matmul(X, CBr, SCBr, thr)
    Xq, _, _, _ = L.llmint8_quantize_act(h2d(X), thr)
    Xqr, _ = oracle.quantize_rows(X, Or)
    for p in (L.PATH_GEMM, L.PATH_DECODE):
        assert_equal_exact(d2h(L.llmint8_igemm_i32(Xq, CB, path=p)), oracle.int_gemm(Xqr, CBr), "tiny C path %d" % p)
        assert_fp16_close(d2h(L.llmint8_matmul_path(h2d(X), CB, SCB, thr, path=p)), ref, "tiny out path %d" % p)


def test_up_proj_1p3b():
    d = workloads.up_proj_1p3b()
    Or = _full_case(d["X"], d["W_t"], d["threshold"], sample_rows(2048, 126), "1.3B up-proj")
    assert Or.size == 3


def test_ffn_6p7b_fc1():
    d = workloads.ffn_6p7b(with_fc2=False)
    Or = _full_case(d["X"], d["W_t"], d["threshold"], sample_rows(4096, 62), "6.7B fc1")
    assert Or.size == 6


def test_ffn_6p7b_fc2():
    W2_t = workloads.ffn_6p7b(with_fc2=True)["W2_t"]
    d = workloads.ffn_6p7b_fc2_input()
    Or = _full_case(d["X"], W2_t, d["threshold"], sample_rows(4096, 14), "6.7B fc2", check_c=False)
    say("fc2 outlier columns: %d of 16384" % Or.size)


@pytest.mark.parametrize("T", [1, 4, 16])
def test_decode_175b(T):
    d = workloads.decode_175b(T, with_weight=True)
    X, W_t, thr = d["X"], d["W_t"], d["threshold"]
    say("decode T=%d K=12288 N=49152" % T)
    cols = np.unique(np.concatenate([[0, 49151], np.random.default_rng(5).choice(49152, 254, replace=False)]))
    CB, SCB = L.llmint8_quantize_weight(h2d(W_t))
    CBr, SCBr = oracle.quantize_weight(W_t[cols])
    assert_equal_exact(d2h(CB)[cols], CBr, "decode CB")
    assert_equal_exact(d2h(SCB)[cols], SCBr, "decode SCB")
    Xd = h2d(X)
    Xq, Xqr, Or = _check_act(Xd, X, thr, "decode T=%d" % T)
    assert Or.size == 6
    C = d2h(L.llmint8_igemm_i32(Xq, CB))
    assert_equal_exact(C[:, cols], oracle.int_gemm(Xqr, CBr), "decode C")
    out = d2h(L.llmint8_matmul(Xd, CB, SCB, thr))
    ref, _, _ = oracle.matmul(X, CBr, SCBr, thr)
    assert_fp16_close(out[:, cols], ref, "decode out")


_SWEEP_W = {}


def _sweep_weight():
    if "W" not in _SWEEP_W:
        W_t = workloads.attn_proj_sweep(with_weight=True)["W_t"]
        _SWEEP_W["W"] = W_t
        _SWEEP_W["ref"] = oracle.quantize_weight(W_t)
    return _SWEEP_W["W"], _SWEEP_W["ref"]


@pytest.mark.parametrize("n_dims,thr,T", [(6, 6.0, 4096), (0, 6.0, 4096), (32, 6.0, 4096),
                                          (128, 6.0, 4096), (6, 0.0, 4096), (6, np.inf, 4096),
                                          (6, 6.0, 4095)])
def test_attn_proj_sweep(n_dims, thr, T):
    W_t, (CBr, SCBr) = _sweep_weight()
    X = workloads.attn_proj_sweep(n_dims=n_dims, T=T, with_weight=False)["X"]
    what = "sweep n=%d thr=%s T=%d" % (n_dims, thr, T)
    say(what)
    Xd = h2d(X)
    CB, SCB = L.llmint8_quantize_weight(h2d(W_t))
    assert_equal_exact(d2h(CB), CBr, what + " CB")
    Xq, Xqr, Or = _check_act(Xd, X, thr, what)
    if thr == 6.0:
        assert Or.size == n_dims
    rows = sample_rows(T, 14 if thr == 0.0 else 30)
    C = d2h(L.llmint8_igemm_i32(Xq, CB))
    assert_equal_exact(C[rows], oracle.int_gemm(Xqr[rows], CBr), what + " C")
    out = d2h(L.llmint8_matmul(Xd, CB, SCB, thr))
    cols = None if thr != 0.0 else np.arange(0, 12288, 3)
    ref, _, _ = oracle.matmul(X, CBr, SCBr, thr, rows=rows, cols=cols)
    got = out[rows] if cols is None else out[np.ix_(rows, cols)]
    assert_fp16_close(got, ref, what + " out")
