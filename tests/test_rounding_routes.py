"""The two fp32 routes the HIP kernels use for round(127*x/a), checked on the
CPU against the oracle's exact rational rounding (ties to even).

* the division route rint((127x)/a) with one correctly rounded fp32 division;
* the reciprocal route r = 127/a, y = x*r, q = rint(y), taken only where
  |y - q| < 0.5 - 2^-15 (the kernels fall back to the division elsewhere);
* the same route with the product fused into the rounding and the residual
  (hipcc contracts x*r + 1.5*2^23 and x*r - q into fused multiply-adds):
  q = rint of the exact product p = x*r, accepted where fp32(p - q) is below
  the same margin.

numpy's float32 arithmetic is IEEE round-to-nearest-even, as the GPU's is, so
these are the kernels' results.  Every binary16 x with |x| <= a is tried for
a spread of a (special values and a seeded random sample)."""
import numpy as np
import pytest

import oracle

HALF_MARGIN = np.float32(0.5 - 2.0 ** -15)


def all_x_up_to(a_bits):
    """Every binary16 bit pattern x with |x| <= a (both signs)."""
    mag = np.arange(0, int(a_bits) + 1, dtype=np.uint16)
    return np.concatenate([mag, mag | np.uint16(0x8000)])


def special_a():
    vals = [6.0, 5.3984375, 1.0, 2.0, 0.5, 127.0, 254.0, 3.19921875, 65504.0, 6.1035156e-05,
            5.9604645e-08, 1.0009766, 0.99951172, 3.0, 255.0, 100.0]
    return np.array(vals, np.float16).view(np.uint16)


def random_a(n, seed=11):
    rng = np.random.default_rng(seed)
    bits = rng.integers(1, 0x7c00, n).astype(np.uint16)   # positive finite, nonzero
    return bits


def routes(xb, ab):
    x = xb.view(np.float16).astype(np.float32)
    a = np.float32(np.array(ab, np.uint16).view(np.float16))
    q_div = np.rint((np.float32(127.0) * x) / a)
    r = np.float32(127.0) / a
    y = x * r
    q_rec = np.rint(y)
    ok = np.abs(y - q_rec) < HALF_MARGIN
    # fused: the product is exact in fp64 (11 + 24 bits), so are its rounding
    # to an integer and the residual; only the residual is rounded to fp32
    p = x.astype(np.float64) * np.float64(r)
    q_fus = np.rint(p)
    ok_fus = np.abs((p - q_fus).astype(np.float32)) < HALF_MARGIN
    return (q_div.astype(np.int32), q_rec.astype(np.int32), ok, q_fus.astype(np.int32), ok_fus)


@pytest.mark.parametrize("which", ["special", "random"])
def test_reciprocal_and_division_routes_are_exact(which):
    a_list = special_a() if which == "special" else random_a(1500)
    fallback = 0
    total = 0
    for ab in a_list:
        xb = all_x_up_to(ab)
        exact = oracle.round_127x_over_a(xb, np.full(xb.shape, ab, np.uint16))
        q_div, q_rec, ok, q_fus, ok_fus = routes(xb, ab)
        assert np.array_equal(q_div, exact), "division route, a bits %#x" % ab
        assert np.array_equal(q_rec[ok], exact[ok]), "reciprocal route, a bits %#x" % ab
        assert np.array_equal(q_fus[ok_fus], exact[ok_fus]), "fused route, a bits %#x" % ab
        fallback += int((~ok).sum()) + int((~ok_fus).sum())
        total += xb.size
    # the fallback is rare on these inputs (ties and near-ties only)
    assert fallback < 0.02 * total


def test_reciprocal_route_declines_exact_ties():
    # 127 * x / a = k + 1/2 exactly: a = 254, x = 1 (0.5), x = 3 (1.5); a = 2, x = 1/127-ish
    # is not representable, so use a = 254 * 2^j
    for j in range(-6, 7):
        a = np.float16(254.0 * 2.0 ** j)
        xs = np.array([1.0, 3.0, 5.0, 253.0], np.float16) * np.float16(2.0 ** j)
        xb = xs.view(np.uint16)
        ab = np.uint16(np.array(a).view(np.uint16))
        exact = oracle.round_127x_over_a(xb, np.full(xb.shape, ab, np.uint16))
        q_div, q_rec, ok, q_fus, ok_fus = routes(xb, ab)
        assert not ok.any() and not ok_fus.any(), "a tie must take the division route"
        assert np.array_equal(q_div, exact)
        assert np.array_equal(exact % 2, np.zeros_like(exact)), "ties go to even"


# ---------------------------------------------------------------------------
# Zero-point variant: the kernels compute the code of x from one fused
# multiply-add, fma(x, nd, 1.5*2^23) (the exact product rounded to an integer,
# ties to even, since 1.5*2^23 is even), minus zp (exact), clamped by an fp32
# min at 1.5*2^23 + 127, and take it as bits - bits(1.5*2^23); the zero point
# as fma(min', nd, 1.5*2^23) - 1.5*2^23 + 127.  (Folding zp into the addend
# would be wrong: with an odd addend the ties go to odd.)  A fused
# multiply-add rounds the exact x*nd + c once; that rounding is done here
# with exact rationals.
# ---------------------------------------------------------------------------
from fractions import Fraction  # noqa: E402

MAGIC = 12582912.0


def fp32_round(v):
    """Nearest fp32 value to the rational v (ties to even); v within the
    normal range."""
    if v == 0:
        return 0.0
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = Fraction(2) ** (e - 23)          # 24 significant bits
    q = a / ulp
    r = round(q)                           # ties to even
    return sign * float(r * ulp)


def fma32(x, y, c):
    return fp32_round(Fraction(float(x)) * Fraction(float(y)) + Fraction(float(c)))


@pytest.mark.parametrize("seed", [21, 22, 23])
def test_zero_point_fused_route_matches_the_oracle(seed):
    rng = np.random.default_rng(seed)
    kinds = [rng.standard_normal(64), np.abs(rng.standard_normal(64)) + 0.25,
             -rng.exponential(3.0, 64), rng.uniform(-1e-3, 5e-3, 64),
             rng.uniform(-60000, 900, 64), np.r_[[-63.5, 63.5], rng.choice([0.25, 0.75, 1.25, -0.75], 62)],
             # nd = 2 with an odd zero point (1): the ties 0.5, 1.5, 2.5 must
             # still go to even before the zero point is subtracted
             np.r_[[-63.0, 64.0], rng.choice([0.25, 0.75, 1.25, -0.75, -1.25, 3.25], 62)]]
    X = np.stack(kinds).astype(np.float16)
    q_or, nd_or, zp_or = oracle.quantize_rows_zp(X, np.zeros(0, np.int32))
    for t in range(X.shape[0]):
        xs = X[t].astype(np.float32)
        mn = np.float32(min(xs.min(), 0.0))
        mx = np.float32(max(xs.max(), 0.0))
        d = np.float32(mx - mn)
        nd = np.float32(254.0) / d
        zp = int(fma32(mn, nd, MAGIC) - MAGIC) + 127
        assert nd == nd_or[t] and zp == zp_or[t]
        for k in range(X.shape[1]):
            s = min(fma32(xs[k], nd, MAGIC) - zp, MAGIC + 127.0)
            bits = int(np.float32(s).view(np.uint32)) - int(np.float32(MAGIC).view(np.uint32))
            assert bits == q_or[t, k], (t, k)
