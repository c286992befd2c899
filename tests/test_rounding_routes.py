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
# Zero-point variant: the kernels round the exact rational 254 x / d
# (d = max' - min', exact in fp64) as floor(y) + (frac(y) > 1/2) with
# y = x * fp64(254/d), and decide a fraction within 2^-40 of 1/2 by the sign
# of 508 x - (2k + 1) d (one exact fused multiply-add on the GPU, exact
# integers here).  The stored nd is fp32(fp64(254/d)) unless fp64(254/d) lies
# within 2^-52 of the midpoint between two fp32 values, where the sign of
# mid * d - 254 picks the side.  numpy's float64 and float32 arithmetic is
# IEEE round-to-nearest-even, as the GPU's is.
# ---------------------------------------------------------------------------
from fractions import Fraction  # noqa: E402

NEAR_HALF = 2.0 ** -40


def rne254_route(x, d, r, hits):
    xd = np.float64(x)
    y = xd * r
    k = np.floor(y)
    f = y - k
    q = int(k) + (1 if f > 0.5 else 0)
    if abs(f - 0.5) < NEAR_HALF:
        hits.append(1)
        e = Fraction(508) * Fraction(float(xd)) - (2 * int(k) + 1) * Fraction(float(d))
        q = int(k) + (1 if e > 0 else 0 if e < 0 else (int(k) & 1))
    return q


def nearest_nd_route(d, r):
    f = np.float32(r)
    fd = np.float64(f)
    if fd == r:
        return f
    fb = int(f.view(np.uint32))
    g = np.array([fb + 1 if r > fd else fb - 1], np.uint32).view(np.float32)[0]
    mid = 0.5 * (fd + np.float64(g))
    if abs(r - mid) > 2.0 ** -52 * r:
        return f
    lo, hi = min(f, g), max(f, g)
    e = Fraction(float(mid)) * Fraction(float(d)) - 254
    if e > 0:
        return lo
    if e < 0:
        return hi
    return hi if int(lo.view(np.uint32)) & 1 else lo


def zp_route(row, hits):
    xs = row.astype(np.float32)
    mn, mx = min(xs.min(), np.float32(0)), max(xs.max(), np.float32(0))
    d = np.float64(mx) - np.float64(mn)
    if d == 0:
        return np.float32(0), 0, [0] * len(xs)
    r = np.float64(254.0) / d
    zp = rne254_route(mn, d, r, hits) + 127
    return nearest_nd_route(d, r), zp, [rne254_route(x, d, r, hits) - zp for x in xs]


@pytest.mark.parametrize("seed", [21, 22, 23])
def test_zero_point_route_matches_the_oracle(seed):
    rng = np.random.default_rng(seed)
    kinds = [rng.standard_normal(64), np.abs(rng.standard_normal(64)) + 0.25,
             -rng.exponential(3.0, 64), rng.uniform(-1e-3, 5e-3, 64),
             rng.uniform(-60000, 900, 64), rng.uniform(-2.0 ** -20, 3.0, 64),
             # exact ties: d = 127 gives nd = 2, so 0.25, 0.75, 1.25 scale to
             # 0.5, 1.5, 2.5; with the zero point odd (min' = -63) as well
             np.r_[[-63.5, 63.5], rng.choice([0.25, 0.75, 1.25, -0.75], 62)],
             np.r_[[-63.0, 64.0], rng.choice([0.25, 0.75, 1.25, -0.75, -1.25, 3.25], 62)]]
    kinds += [rng.standard_normal(64) * rng.uniform(0.01, 100) for _ in range(24)]
    X = np.stack(kinds).astype(np.float16)
    q_or, nd_or, zp_or = oracle.quantize_rows_zp(X, np.zeros(0, np.int32))
    hits = []
    for t in range(X.shape[0]):
        nd, zp, codes = zp_route(X[t], hits)
        assert nd == nd_or[t] and zp == zp_or[t], t
        assert codes == q_or[t].astype(int).tolist(), t
    assert len(hits) >= 60          # the exact tie branch ran (the tie rows)


def test_nearest_nd_route_at_fp32_midpoints():
    # fp64 values d for which fp64(254/d) lands on, or next to, the midpoint
    # between two fp32 values: there fp32(fp64(254/d)) can be a double
    # rounding, and the route must still give the fp32 value nearest to the
    # exact quotient
    rng = np.random.default_rng(31)
    checked = 0
    for _ in range(400):
        f = np.float32(rng.uniform(0.002, 2.0 ** 31))
        g = np.nextafter(f, np.float32(np.inf))
        mid = 0.5 * (np.float64(f) + np.float64(g))
        d0 = np.float64(254.0) / mid
        for step in range(-3, 4):
            d = d0
            for _ in range(abs(step)):
                d = np.nextafter(d, np.inf if step > 0 else 0.0)
            r = np.float64(254.0) / d
            exact = Fraction(254) / Fraction(float(d))
            cands = [np.float32(r), np.nextafter(np.float32(r), np.float32(np.inf)),
                     np.nextafter(np.float32(r), np.float32(0))]
            want = min(cands, key=lambda v: (abs(Fraction(float(v)) - exact),
                                             int(v.view(np.uint32)) & 1))
            assert nearest_nd_route(d, r) == want
            checked += abs(r - mid) <= 2.0 ** -52 * r
    assert checked >= 100           # the midpoint branch ran
