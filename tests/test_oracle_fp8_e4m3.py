"""Pins of the oracle's E4M3 form of the FP8 variant of the decomposition.

The LLM.int8() summary (kurtkim.github.io, "LLM.int8()", section "Related
work", 8-bit data types; "Discussion and Limitations") expects the Int8
findings to carry over to 8-bit floating-point formats.  It names the kind
with a 5-bit exponent; E4M3 (4 exponent bits, 3 fraction bits, the "fn"
layout with no infinities and a largest finite value of 448) is the other
8-bit float format that MFMA units compute in, and the oracle's E4M3 form
takes every reading of the E5M2 one with this format in its place (the
per-vector power-of-two scale targets 448).  Each test checks the oracle
against something other than its own formula: torch's float8_e4m3fn type,
the binary16 bit layout, brute force, exact products, error bounds, sign
and power-of-two symmetries.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

NO_O = np.zeros(0, np.int32)
FMT = "e4m3"


def f16(v):
    return np.asarray(v, np.float16)


def torch_e4m3_codes(v):
    """torch's conversion of float64 values to float8_e4m3fn, as code bytes."""
    return torch.from_numpy(np.ascontiguousarray(v, np.float64)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_codec_matches_torch_float8_e4m3fn():
    c = np.arange(256, dtype=np.uint8)
    d = oracle.e4m3_to_double(c)
    t = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(d), np.isnan(t))
    assert np.flatnonzero(np.isnan(d)).tolist() == [0x7F, 0xFF]          # the only NaNs
    ok = ~np.isnan(d)
    assert np.array_equal(d[ok], t[ok])
    assert d[0x7E] == 448.0                     # largest finite
    assert d[0x01] == 2.0 ** -9                 # smallest subnormal
    assert d[0x08] == 2.0 ** -6                 # smallest normal
    assert d[0x38] == 1.0                       # exponent bias 7
    assert np.all(np.diff(d[:0x7F]) > 0)        # codes are ordered like their values
    assert np.array_equal(oracle.f8_to_double(c, "e4m3")[ok], d[ok])


def test_rounding_of_every_fp16_value_in_range():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = h.view(np.float16).astype(np.float64)
    keep = np.isfinite(v) & (np.abs(v) <= 464.0)
    got = oracle.double_to_e4m3(v[keep])
    # torch's own conversion
    assert np.array_equal(got, torch_e4m3_codes(v[keep]))
    a = np.abs(v[keep])
    sign = np.where(np.signbit(v[keep]), 0x80, 0).astype(np.uint8)
    # normal range: binary16 rebiased by 15 - 7 and its fraction rounded
    # from 10 to 3 bits (ties to even, the carry running into the exponent)
    hb = (h[keep] & 0x7FFF).astype(np.int64)
    nrm = a >= 2.0 ** -6
    bitwise = ((hb - (8 << 10) + 0x3F + ((hb >> 7) & 1)) >> 7)
    assert np.array_equal(got[nrm], (bitwise[nrm].astype(np.uint8) | sign[nrm]))
    # subnormal range: the nearest multiple of 2^-9 (ties to even), whose
    # count is the code itself, 8 being the smallest normal
    sub = ~nrm
    r = np.round(a[sub] * 2.0 ** 9)             # numpy rounds halves to even
    assert np.array_equal(got[sub], r.astype(np.uint8) | sign[sub])
    # the tie at 464 between 448 and the NaN position goes to the even 448;
    # anything above it has no finite code
    assert oracle.double_to_e4m3(np.array([464.0, -464.0, 460.0]))[:].tolist() == [0x7E, 0xFE,
                                                                                   0x7E]
    assert np.isnan(oracle.e4m3_to_double(oracle.double_to_e4m3(np.array([464.5, 480.0, 1e6]))))\
        .all()


def test_scale_exponent_is_the_largest_that_fits():
    h = np.arange(1, 0x7C00, 7, dtype=np.uint32).astype(np.uint16)   # positive finite fp16
    a = np.concatenate([h.view(np.float16).astype(np.float64),
                        [448.0, 448.25, 1.0, 1.75, 1.875, 65504.0, 2.0 ** -24]])
    e = oracle.f8_scale_exp(a, FMT)
    for ai, ei in zip(a, e):
        x = Fraction(ai)
        assert x * Fraction(2) ** int(ei) <= 448 < x * Fraction(2) ** (int(ei) + 1), (ai, ei)
    assert oracle.f8_scale_exp(np.array([0.0]), FMT)[0] == 0
    assert list(oracle.f8_scale_exp(np.array([448.0, 448.25, 1.0, 1.75, 1.875]), FMT)) == [
        0, -1, 8, 8, 7]


def test_row_codes_match_torch_and_fill_the_top_binade():
    rng = np.random.default_rng(13)
    X = rng.standard_normal((6, 192))
    X[1] *= 1e-4
    X[2] = rng.uniform(-60000, 60000, 192)
    X[3] = 0.0
    X[4] = np.abs(X[4])
    X = f16(X)
    q, sc = oracle.quantize_rows_f8(X, NO_O, fmt=FMT)
    for t in range(X.shape[0]):
        x = X[t].astype(np.float64)
        amax = np.abs(x).max()
        if amax == 0:
            assert sc[t] == 1.0 and not q[t].any()
            continue
        scale = 1.0 / np.float64(sc[t])
        assert scale == 2.0 ** np.round(np.log2(scale))                  # a power of two
        assert 224.0 < amax * scale <= 448.0                              # top binade of E4M3
        assert np.array_equal(q[t], torch_e4m3_codes(x * scale))
        assert not np.isnan(oracle.e4m3_to_double(q[t])).any()           # never past 448


def test_outlier_columns_are_zero_and_do_not_set_the_scale():
    rng = np.random.default_rng(14)
    X = rng.standard_normal((5, 128))
    X[:, [9, 70]] = rng.uniform(20, 60, (5, 2))
    X = f16(X)
    O = oracle.outlier_columns(X, 6.0)
    assert O.tolist() == [9, 70]
    q, sc = oracle.quantize_rows_f8(X, O, fmt=FMT)
    assert not q[:, O].any()
    X0 = X.copy()
    X0[:, O] = 0
    q0, sc0 = oracle.quantize_rows_f8(X0, NO_O, fmt=FMT)
    assert np.array_equal(q, q0) and np.array_equal(sc, sc0)


def test_weight_quantization_is_per_output_column():
    rng = np.random.default_rng(15)
    W = f16(rng.standard_normal((64, 96)) * 0.05)
    CB8, SC8 = oracle.quantize_weight_f8(W, FMT)
    q, sc = oracle.quantize_rows_f8(W, NO_O, fmt=FMT)
    assert np.array_equal(CB8, q) and np.array_equal(SC8, sc)
    # the E4M3 codes differ from the E5M2 ones (a wrong format code would
    # pass every other test of this file that only compares the two paths)
    CB5, _ = oracle.quantize_weight_f8(W, "e5m2")
    assert not np.array_equal(CB8, CB5)


def test_representable_inputs_give_the_exact_product():
    # entries with at most 4 significant bits stay exact under E4M3 (the
    # power-of-two scale keeps them in its normal range), so the
    # decomposition is the exact product rounded once to fp16, outliers and
    # bias included; 1.875 and 0.9375 need the fourth bit, which E5M2 lacks
    rng = np.random.default_rng(16)
    T, K, N = 12, 256, 96
    X = rng.choice([-3.0, -1.875, -1.0, -0.5, 0.0, 0.25, 0.9375, 1.0, 2.0, 3.5], (T, K))
    X[::2, 17] = 24.0                 # an outlier column (exact in fp16 too)
    W = rng.choice([-0.375, -0.25, -0.234375, 0.0, 0.0625, 0.125, 0.1875, 0.25], (N, K))
    bias = rng.choice([-1.0, 0.5, 2.0], N)
    CB8, SC8 = oracle.quantize_weight_f8(f16(W), FMT)
    out, O, _ = oracle.matmul_f8(f16(X), CB8, SC8, 6.0, bias=f16(bias), fmt=FMT)
    assert O.tolist() == [17]
    exact = X @ W.T + bias
    assert np.array_equal(out, exact.astype(np.float16).view(np.uint16))
    out5, _, _ = oracle.matmul_f8(f16(X), *oracle.quantize_weight_f8(f16(W), "e5m2"), 6.0,
                                  bias=f16(bias))
    assert not np.array_equal(out5, out)


@pytest.mark.parametrize("thr", [np.inf, 6.0])
def test_output_is_within_the_quantization_error_of_the_true_product(thr):
    rng = np.random.default_rng(17)
    T, K, N = 16, 256, 64
    X = rng.standard_normal((T, K))
    if np.isfinite(thr):
        X[::2, 40] = rng.uniform(20, 60, T // 2)
    X = f16(X)
    W = f16(rng.standard_normal((N, K)) * 0.05)
    CB8, SC8 = oracle.quantize_weight_f8(W, FMT)
    out, O, sc = oracle.matmul_f8(X, CB8, SC8, thr, fmt=FMT)
    Xq8, _ = oracle.quantize_rows_f8(X, O, fmt=FMT)
    isout = np.zeros(K, bool)
    isout[O] = True
    Xd, Wd = X.astype(np.float64), W.astype(np.float64)
    xhat = oracle.e4m3_to_double(Xq8) * sc.astype(np.float64)[:, None]
    what = oracle.e4m3_to_double(CB8) * SC8.astype(np.float64)[:, None]
    # E4M3 rounding: relative 2^-4 for normal values, absolute 2^-10 * scale below
    dx = np.maximum(np.abs(Xd) * 2.0 ** -4, 2.0 ** -10 * sc.astype(np.float64)[:, None])
    dw = np.maximum(np.abs(Wd) * 2.0 ** -4, 2.0 ** -10 * SC8.astype(np.float64)[:, None])
    assert np.all(np.abs(xhat - Xd)[:, ~isout] <= dx[:, ~isout])
    assert np.all(np.abs(what - Wd) <= dw)
    got = out.view(np.float16).astype(np.float64)
    true = Xd @ Wd.T
    ax = np.abs(Xd)
    bound = (ax * ~isout) @ dw.T + (dx * ~isout) @ np.abs(what).T
    bound += (ax * isout) @ (dw + 2.0 ** -11 * np.abs(what)).T
    bound += 2.0 ** -11 * np.abs(got) + 1e-6
    assert np.all(np.abs(got - true) <= bound)


def test_threshold_zero_is_the_fp16_gemm_with_dequantized_weights():
    rng = np.random.default_rng(18)
    X = f16(rng.standard_normal((8, 128)))
    W = f16(rng.standard_normal((64, 128)) * 0.05)
    CB8, SC8 = oracle.quantize_weight_f8(W, FMT)
    out, O, _ = oracle.matmul_f8(X, CB8, SC8, 0.0, fmt=FMT)
    assert len(O) == 128
    wdq = (oracle.e4m3_to_double(CB8) * SC8.astype(np.float64)[:, None]).astype(np.float16)
    ref = (X.astype(np.float64) @ wdq.astype(np.float64).T).astype(np.float16)
    assert np.array_equal(out, ref.view(np.uint16))


def test_negation_and_power_of_two_row_scaling():
    rng = np.random.default_rng(19)
    X = f16(rng.standard_normal((10, 192)))
    W = f16(rng.standard_normal((64, 192)) * 0.05)
    CB8, SC8 = oracle.quantize_weight_f8(W, FMT)
    out, _, sc = oracle.matmul_f8(X, CB8, SC8, np.inf, fmt=FMT)
    out_n, _, _ = oracle.matmul_f8(-X, CB8, SC8, np.inf, fmt=FMT)
    assert np.array_equal(out_n, out ^ np.uint16(0x8000))
    # a row times 2^j keeps its codes (the scale absorbs it) and its output
    # row is the old one times 2^j, exactly
    X2 = X.copy()
    X2[3] *= np.float16(8.0)
    X2[7] *= np.float16(0.25)
    out2, _, sc2 = oracle.matmul_f8(X2, CB8, SC8, np.inf, fmt=FMT)
    q, _ = oracle.quantize_rows_f8(X, NO_O, fmt=FMT)
    q2, _ = oracle.quantize_rows_f8(X2, NO_O, fmt=FMT)
    assert np.array_equal(q, q2)
    assert sc2[3] == sc[3] * 8 and sc2[7] == sc[7] / 4
    o = out.view(np.float16).astype(np.float64)
    o2 = out2.view(np.float16).astype(np.float64)
    assert np.array_equal(o2[3], o[3] * 8) and np.array_equal(o2[7], o[7] / 4)
    keep = [r for r in range(10) if r not in (3, 7)]
    assert np.array_equal(out2[keep], out[keep])
