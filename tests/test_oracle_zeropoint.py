"""Pins of the oracle's zero-point (asymmetric) vector-wise variant.

The LLM.int8() summary (kurtkim.github.io, "LLM.int8()", section "8-bit Data
Types and Quantization") defines zeropoint quantization: scale by the
normalized dynamic range nd = 2*127/(max - min), shift by an integer zero
point so the values fill [-127, 127], multiply (A_i8 + zp_a)(B_i8 + zp_b) in
integers and dequantize by dividing by nd_a*nd_b.  The printed formulas are
garbled; the readings the oracle takes are stated in oracle/llmint8_oracle.c.
Each test checks the oracle against something other than its own formula:
the page's ReLU remark, the absmax oracle (pinned on its own), exact
rational arithmetic, error bounds against the true product, the textbook
fp16 GEMM, and sign symmetry.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle

NO_O = np.zeros(0, np.int32)


def f16(v):
    return np.asarray(v, np.float16)


def widened(X):
    return np.asarray(X, np.float16).astype(np.float64)


def exact_params(row):
    """(d, nd, zp) of one vector from exact rationals: the range with 0 added,
    nd = 254/d, zp = RNE(nd*min') + 127 (round() on a Fraction: ties to even)."""
    xs = widened(row)
    mn, mx = min(xs.min(), 0.0), max(xs.max(), 0.0)
    d = Fraction(mx) - Fraction(mn)
    if d == 0:
        return d, Fraction(0), 0
    nd = 254 / d
    return d, nd, round(nd * Fraction(mn)) + 127


def nearest_f32(v):
    """The fp32 value nearest to the positive rational v, ties to even: the
    best of numpy's float32 of float(v) and its two neighbours."""
    c = np.float32(float(v))
    cands = [c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(0))]
    return min(cands, key=lambda f: (abs(Fraction(float(f)) - v),
                                     int(np.float32(f).view(np.uint32)) & 1))


def test_relu_row_uses_the_whole_code_range():
    # the page: on a ReLU output absmax leaves [-127, 0) unused, zeropoint
    # quantization uses the full range
    x = f16([[0.0, 0.5, 1.0, 2.0, 3.5, 5.25, 0.125, 4.0]])
    q, nd, zp = oracle.quantize_rows_zp(x, NO_O)
    assert q.min() == -127 and q.max() == 127
    assert q[0, 0] == -127                     # the minimum, 0, takes the lowest code
    assert zp[0] == 127
    q_abs = oracle.round_127x_over_a(x.view(np.uint16), np.full(x.shape, f16(5.25).view(np.uint16)))
    assert q_abs.min() >= 0 and q_abs.max() == 127   # absmax: only the upper half


@pytest.mark.parametrize("j", [-3, 0, 2, 5])
def test_symmetric_power_of_two_row_equals_absmax(j):
    # a row holding +a and -a, a = 2^j: the zero point is 0 and nd = 127/a
    # exactly, so the codes are the absmax codes round(127 x / a)
    rng = np.random.default_rng(100 + j)
    a = 2.0 ** j
    x = f16(rng.uniform(-a, a, (3, 96)))
    x[:, 7] = a
    x[:, 50] = -a
    q, nd, zp = oracle.quantize_rows_zp(x, NO_O)
    assert np.all(zp == 0)
    assert np.all(nd == np.float32(127.0 / a))
    ref = oracle.round_127x_over_a(x.view(np.uint16), np.full(x.shape, f16(a).view(np.uint16)))
    assert np.array_equal(q.astype(np.int32), ref)


def test_ties_round_to_even():
    # min -63.5, max 63.5: d = 127, nd = 2 exactly, zp = 0; 0.25, 0.75, 1.25
    # scale to the ties 0.5, 1.5, 2.5 -> 0, 2, 2 (half away from zero would give 1, 2, 3)
    x = f16([[-63.5, 63.5, 0.25, 0.75, 1.25, -0.25, -0.75, -1.25]])
    q, nd, zp = oracle.quantize_rows_zp(x, NO_O)
    assert nd[0] == np.float32(2.0) and zp[0] == 0
    assert q[0, 2:].tolist() == [0, 2, 2, 0, -2, -2]


def _rows_mixed(seed, T=12, K=192):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, K))
    X[1] = np.abs(X[1]) + 0.5            # all positive (0 still joins the range)
    X[2] = -np.abs(X[2]) * 3 - 1.0       # all negative
    X[3] = np.maximum(X[3], 0)           # ReLU-like
    X[4] *= 1e-3                         # small magnitudes
    X[5] = rng.exponential(2.0, K)       # skewed
    X[6] = 0.0                           # all zero
    X[7] = rng.uniform(-1, 60000, K)     # near the fp16 limit
    return f16(X)


@pytest.mark.parametrize("seed", [1, 2])
def test_codes_are_exact_rational_roundings(seed):
    X = _rows_mixed(seed)
    q, nd, zp = oracle.quantize_rows_zp(X, NO_O)
    Xd = widened(X)
    for t in range(X.shape[0]):
        d, ndx, zpx = exact_params(X[t])
        if d == 0:
            assert nd[t] == 0 and zp[t] == 0 and not q[t].any()
            continue
        assert nd[t] == nearest_f32(ndx)
        assert zp[t] == zpx
        for k in range(X.shape[1]):
            assert q[t, k] == round(ndx * Fraction(Xd[t, k])) - zpx, (t, k)
    assert np.abs(q.astype(np.int32)).max() <= 127


# Ranges [-lo, hi] (binary16 values) whose 254/d, rounded to fp64 first, lands
# exactly on the midpoint between two fp32 values while the exact quotient
# lies above it, so that rounding the fp64 quotient to fp32 gives the lower
# neighbour instead of the nearest; found by a search over binary16 pairs.
MIDPOINT_RANGES = [(7112.0, 889), (14224.0, 1778)]     # (hi, bits of lo)


def test_stored_nd_is_not_a_double_rounding():
    for hi, lo_bits in MIDPOINT_RANGES:
        lo = float(np.array([lo_bits], np.uint16).view(np.float16)[0])
        row = f16([hi, -lo, 1.0])
        q, nd, zp = oracle.quantize_rows_zp(row[None, :], NO_O)
        d, ndx, zpx = exact_params(row)
        via_fp64 = np.float32(254.0 / (hi + lo))
        assert nd[0] == nearest_f32(ndx) and nd[0] != via_fp64


def _random_rows(seed, rows=120, K=256):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((rows, K)) * rng.uniform(0.01, 100, (rows, 1))
    X[::3] = np.abs(X[::3])
    return f16(X)


def test_codes_follow_the_exact_nd_not_a_rounded_one():
    # rounding nd to fp32 before the products (the natural fp32 shortcut)
    # moves some codes by one; the oracle must give the exact-rational code
    # there too.  The seeded rows hold such cases, and the test requires them.
    X = _random_rows(1)
    q, nd, zp = oracle.quantize_rows_zp(X, NO_O)
    Xd = widened(X)
    moved = 0
    for t in range(X.shape[0]):
        d, ndx, zpx = exact_params(X[t])
        mn, mx = min(Xd[t].min(), 0.0), max(Xd[t].max(), 0.0)
        nd32 = Fraction(float(np.float32(254.0) / (np.float32(mx) - np.float32(mn))))
        zp32 = round(nd32 * Fraction(mn)) + 127
        for k in range(X.shape[1]):
            exact = round(ndx * Fraction(Xd[t, k])) - zpx
            shortcut = min(round(nd32 * Fraction(Xd[t, k])) - zp32, 127)
            assert q[t, k] == exact, (t, k)
            moved += shortcut != exact
    assert moved >= 1


def test_stored_nd_is_the_nearest_fp32():
    # vectors whose range d has many significant bits (a large and a tiny
    # end), so 254/d is far from any short binary fraction
    rng = np.random.default_rng(7)
    for _ in range(300):
        hi = float(np.float16(rng.uniform(1, 60000)))
        lo = -float(np.float16(rng.uniform(0, 1) * 2.0 ** -int(rng.integers(0, 24))))
        row = f16([hi, lo, 0.5 * hi])
        q, nd, zp = oracle.quantize_rows_zp(row[None, :], NO_O)
        d, ndx, zpx = exact_params(row)
        assert nd[0] == nearest_f32(ndx) and zp[0] == zpx
        assert q[0, 0] == 127 and q[0, 1] == -127


@pytest.mark.parametrize("seed", [3, 4])
def test_reconstruction_error_is_half_a_step(seed):
    X = _rows_mixed(seed)
    q, nd, zp = oracle.quantize_rows_zp(X, NO_O)
    Xd = widened(X)
    for t in range(X.shape[0]):
        d, ndx, zpx = exact_params(X[t])
        if d == 0:
            continue
        step = 1 / ndx
        for k in range(X.shape[1]):
            # x is within half a step of its dequantized value, exactly
            assert abs(Fraction(Xd[t, k]) - (int(q[t, k]) + zpx) * step) <= step / 2, (t, k)
        # the range is covered: its ends take the extreme codes
        assert q[t].min() == -127 or Xd[t].min() > 0
        assert q[t].max() == 127 or Xd[t].max() < 0


def test_outlier_columns_hold_the_code_of_zero():
    rng = np.random.default_rng(9)
    X = rng.standard_normal((6, 128))
    X[:, [3, 77, 100]] = rng.uniform(20, 60, (6, 3)) * rng.choice([-1, 1], (6, 3))
    X = f16(X)
    O = oracle.outlier_columns(X, 6.0)
    assert O.tolist() == [3, 77, 100]
    q, nd, zp = oracle.quantize_rows_zp(X, O)
    assert np.array_equal(q[:, O].astype(np.int32), -zp[:, None] * np.ones((1, 3), np.int32))
    # with 0 always in the range, dropping the outlier columns is the same as
    # zeroing them: the row parameters and the other codes agree
    X0 = X.copy()
    X0[:, O] = 0
    q0, nd0, zp0 = oracle.quantize_rows_zp(X0, NO_O)
    assert np.array_equal(nd, nd0) and np.array_equal(zp, zp0) and np.array_equal(q, q0)


def test_weight_quantization_matches_row_quantization():
    # vector-wise on the weight: each row of W_t is one vector over all of K
    rng = np.random.default_rng(5)
    W = f16(rng.standard_normal((64, 128)) * 0.05 + 0.01)
    CB, ND, ZP = oracle.quantize_weight_zp(W)
    q, nd, zp = oracle.quantize_rows_zp(W, NO_O)
    assert np.array_equal(CB, q) and np.array_equal(ND, nd) and np.array_equal(ZP, zp)


def test_dequantized_weight_is_fp32_quotient_rounded_to_fp16():
    rng = np.random.default_rng(6)
    cb = rng.integers(-127, 128, 4000).astype(np.int8)
    zp = rng.integers(-127, 128, 4000).astype(np.int32)
    nd = (rng.uniform(0.5, 3000, 4000)).astype(np.float32)
    nd[:10] = 0
    got = oracle.dequant_weight_zp(cb, zp, nd)
    with np.errstate(divide="ignore", invalid="ignore"):
        want = ((cb.astype(np.int32) + zp).astype(np.float32) / nd).astype(np.float16)
    want[:10] = 0
    assert np.array_equal(got, want.view(np.uint16))


def _shifted(q, zp):
    return q.astype(np.int64) + zp.astype(np.int64)[:, None]


@pytest.mark.parametrize("thr", [np.inf, 6.0])
def test_output_is_within_the_quantization_error_of_the_true_product(thr):
    rng = np.random.default_rng(11)
    T, K, N = 16, 256, 64
    X = rng.standard_normal((T, K))
    X[:, 3:6] = np.maximum(X[:, 3:6], 0) * 3          # skewed columns
    if np.isfinite(thr):
        X[::2, 40] = rng.uniform(20, 60, T // 2)
        X[1::3, 200] = -rng.uniform(20, 60, len(range(1, T, 3)))
    X = f16(X)
    W = f16(rng.standard_normal((N, K)) * 0.05 + 0.02)
    CB, ND, ZP = oracle.quantize_weight_zp(W)
    out, O, nd, zp = oracle.matmul_zp(X, CB, ND, ZP, threshold=thr)
    assert (len(O) > 0) == bool(np.isfinite(thr))
    Xq, _, _ = oracle.quantize_rows_zp(X, O)
    Xd, Wd = widened(X), widened(W)
    true = Xd @ Wd.T
    got = out.view(np.float16).astype(np.float64)
    isout = np.zeros(K, bool)
    isout[O] = True
    xhat = _shifted(Xq, zp) / nd.astype(np.float64)[:, None]
    what = _shifted(CB, ZP) / ND.astype(np.float64)[:, None]
    # per element: half a step (1.5 where a code was clamped)
    dx = np.where(_shifted(Xq, zp) == np.rint(nd.astype(np.float64)[:, None] * Xd), 0.5, 1.5) \
        / nd.astype(np.float64)[:, None]
    dw = np.where(_shifted(CB, ZP) == np.rint(ND.astype(np.float64)[:, None] * Wd), 0.5, 1.5) \
        / ND.astype(np.float64)[:, None]
    ax = np.abs(Xd)
    bound = (ax * ~isout) @ dw.T + (dx * ~isout) @ np.abs(what).T
    wdq = widened(oracle.dequant_weight_zp(CB, ZP[:, None], ND[:, None]).view(np.float16))
    bound += (ax * isout) @ (dw + 2.0 ** -11 * np.abs(wdq)).T
    bound += 2.0 ** -11 * np.abs(got) + 1e-6
    assert np.all(np.abs(got - true) <= bound)
    # and the quantized operands themselves, multiplied exactly, give the output
    approx = (xhat * ~isout) @ what.T + (Xd * isout) @ wdq.T
    assert np.all(np.abs(got - approx) <= 2.0 ** -11 * np.abs(approx) + 1e-7)


def test_threshold_zero_is_the_fp16_gemm_with_dequantized_weights():
    rng = np.random.default_rng(12)
    T, K, N = 8, 128, 64
    X = f16(rng.standard_normal((T, K)))
    W = f16(rng.standard_normal((N, K)) * 0.05 - 0.01)
    CB, ND, ZP = oracle.quantize_weight_zp(W)
    out, O, nd, zp = oracle.matmul_zp(X, CB, ND, ZP, threshold=0.0)
    assert len(O) == K and np.all(nd == 0) and np.all(zp == 0)
    wdq = ((CB.astype(np.int32) + ZP[:, None]).astype(np.float32) / ND[:, None]).astype(np.float16)
    ref = (widened(X) @ widened(wdq).T).astype(np.float16)
    assert np.array_equal(out, ref.view(np.uint16))


def test_negating_the_input_negates_the_output():
    rng = np.random.default_rng(13)
    T, K, N = 12, 192, 64
    X = rng.standard_normal((T, K))
    X[:, 10] = rng.uniform(10, 30, T)                   # one outlier column
    X[2] = np.abs(X[2])
    X = f16(X)
    W = f16(rng.standard_normal((N, K)) * 0.05)
    CB, ND, ZP = oracle.quantize_weight_zp(W)
    out_p, O_p, nd_p, zp_p = oracle.matmul_zp(X, CB, ND, ZP, threshold=6.0)
    out_n, O_n, nd_n, zp_n = oracle.matmul_zp(-X, CB, ND, ZP, threshold=6.0)
    # the range of -x is the range of x mirrored (same d), and rounding to
    # nearest even is odd-symmetric, so the shifted codes negate exactly
    Xq_p, _, _ = oracle.quantize_rows_zp(X, O_p)
    Xq_n, _, _ = oracle.quantize_rows_zp(-X, O_n)
    assert np.array_equal(_shifted(Xq_n, zp_n), -_shifted(Xq_p, zp_p))
    assert np.array_equal(O_p, O_n) and np.array_equal(nd_p, nd_n)
    assert np.array_equal(out_n, out_p ^ np.uint16(0x8000))


def test_symmetric_operands_reproduce_the_absmax_decomposition():
    # rows holding +-2^j and weight rows holding +-2^i (and no larger value):
    # zero points are 0 and nd = 127/absmax exactly, so the whole output must
    # equal the absmax oracle's, bit for bit, outliers included
    rng = np.random.default_rng(14)
    T, K, N = 16, 256, 128
    X = rng.uniform(-3.9, 3.9, (T, K))
    X[:, 0] = 4.0
    X[:, 1] = -4.0
    X[::3, 30] = rng.uniform(8, 40, len(range(0, T, 3)))
    X[1::2, 31] = -rng.uniform(8, 40, T // 2)
    X = f16(X)
    W = rng.uniform(-0.124, 0.124, (N, K))
    W[:, 5] = 0.125
    W[:, 6] = -0.125
    W = f16(W)
    CB, ND, ZP = oracle.quantize_weight_zp(W)
    CBa, SCB = oracle.quantize_weight(W)
    assert np.all(ZP == 0) and np.array_equal(CB, CBa)
    bias = f16(rng.standard_normal(N))
    out_z, O_z, _, zp = oracle.matmul_zp(X, CB, ND, ZP, threshold=6.0, bias=bias)
    out_a, O_a, _ = oracle.matmul(X, CBa, SCB, threshold=6.0, bias=bias)
    assert np.all(zp == 0) and O_z.tolist() == [30, 31] and np.array_equal(O_z, O_a)
    assert np.array_equal(out_z, out_a)


def test_sampled_rows_and_columns_match_the_full_call():
    rng = np.random.default_rng(15)
    X = f16(rng.standard_normal((20, 128)) + 0.3)
    X[4, 9] = 30.0
    W = f16(rng.standard_normal((64, 128)) * 0.05)
    CB, ND, ZP = oracle.quantize_weight_zp(W)
    full, O, nd, zp = oracle.matmul_zp(X, CB, ND, ZP)
    rows, cols = [19, 0, 4], [63, 1, 2, 40]
    part, O2, nd2, zp2 = oracle.matmul_zp(X, CB, ND, ZP, rows=rows, cols=cols)
    assert np.array_equal(part, full[np.ix_(rows, cols)])
    assert np.array_equal(O, O2) and np.array_equal(nd2, nd[rows]) and np.array_equal(zp2, zp[rows])
