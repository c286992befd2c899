"""Pins of the oracle's absmax quantization (weights and activations).

Pins, each against something other than the oracle itself:
  * the worked absmax example printed on the Hugging Face LLM.int8() write-up
    (agentlenshq.com, section on zero-point vs absmax quantization);
  * the reciprocal-scale example printed in the quantization basics page
    (techblog.paldyn.com, PTQ scale snippet);
  * exhaustive / random agreement of the exact-rational rounding with numpy's
    fp64 and fp32 routes (np.rint, ties to even) -- the fp32 route is the one
    the GPU kernels take;
  * hand-derived ties (x/a giving exactly k + 1/2);
  * the round-trip bound |x - q*a/127| <= a/254 and the range/structure
    invariants of the absmax map.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
f16 = np.float16


def test_worked_absmax_example():
    g = json.load(open(os.path.join(GOLDEN, "absmax_worked_example.json")))
    x = np.array([g["vector_shown"]], f16)
    Xq, a = oracle.quantize_rows(x, np.zeros(0, np.int32))
    assert a[0] == float(f16(5.4))          # absmax of the fp16 vector
    scale = 127.0 / a[0]
    assert round(scale, g["printed_scale_decimals"]) == g["printed_scale"]
    lo, hi = g["int8_range"]
    assert Xq.min() >= lo and Xq.max() <= hi
    # the absmax element maps to the end of the range, the others inside it
    assert Xq[0, 3] == 127
    assert list(Xq[0]) == [28, -12, -101, 127]


def test_reciprocal_scale_example():
    g = json.load(open(os.path.join(GOLDEN, "reciprocal_scale_example.json")))
    W_t = np.array([[g["weight_max"], -1.0, 0.5, 0.0]], f16)
    CB, SCB = oracle.quantize_weight(W_t)
    assert SCB[0] == float(f16(g["weight_max"]))
    assert round(SCB[0] / g["int8_max"], g["printed_scale_decimals"]) == g["printed_scale"]
    assert CB[0, 0] == 127
    # recovering q*scale lands within half a step of the original
    rec = CB[0].astype(np.float64) * SCB[0] / 127.0
    assert np.all(np.abs(rec - W_t[0].astype(np.float64)) <= 0.5 * SCB[0] / 127.0 * (1 + 1e-12))


def _nonneg_halves_upto(a_bits):
    return np.arange(0, int(a_bits) + 1, dtype=np.uint32).astype(np.uint16)


@pytest.mark.parametrize("a_val", [1.0, 5.3984375, 6.0, 0.0999, 127.0, 254.0,
                                   65504.0, 2.0 ** -14, 3 * 2.0 ** -24, 1.7e-3])
def test_rounding_exhaustive_in_x(a_val):
    a = np.array([a_val], f16).view(np.uint16)[0]
    xs = _nonneg_halves_upto(a)
    xs = np.concatenate([xs, xs | np.uint16(0x8000)])
    got = oracle.round_127x_over_a(xs, np.full(xs.shape, a, np.uint16))
    x64 = xs.view(f16).astype(np.float64)
    a64 = float(np.array([a], np.uint16).view(f16)[0])
    ref64 = np.rint((127.0 * x64) / a64)
    assert np.array_equal(got, ref64.astype(np.int32))
    x32 = xs.view(f16).astype(np.float32)
    ref32 = np.rint((np.float32(127.0) * x32) / np.float32(a64))
    assert np.array_equal(got, ref32.astype(np.int32))


def test_rounding_random_pairs():
    rng = np.random.default_rng(2)
    a = rng.integers(1, 0x7C00, 3_000_000).astype(np.uint16)
    frac = rng.random(a.size)
    x = (frac * a.astype(np.float64)).astype(np.uint16)   # bit patterns <= a's pattern
    x = x | np.where(rng.random(a.size) < 0.5, 0x8000, 0).astype(np.uint16)
    got = oracle.round_127x_over_a(x, a)
    x32 = x.view(f16).astype(np.float32)
    a32 = a.view(f16).astype(np.float32)
    ref = np.rint((np.float32(127.0) * x32) / a32).astype(np.int32)
    assert np.array_equal(got, ref)


def test_ties_round_to_even():
    # a = 254: 127*x/a = x/2, so odd integers x give exact halves
    a = np.array([254.0], f16).view(np.uint16)
    x = np.array([1, 3, 5, 7, -1, -3, -5, 2, 9], f16).view(np.uint16)
    got = oracle.round_127x_over_a(x, np.repeat(a, x.size))
    assert list(got) == [0, 2, 2, 4, 0, -2, -2, 1, 4]


def test_round_trip_bound_and_invariants():
    rng = np.random.default_rng(3)
    X = (rng.standard_normal((64, 96)) * np.exp(rng.uniform(-6, 4, (64, 1)))).astype(f16)
    X[5] = 0.0                                  # an all-zero row
    Xq, a = oracle.quantize_rows(X, np.zeros(0, np.int32))
    x64 = X.astype(np.float64)
    assert np.all(np.abs(Xq.astype(np.int32)) <= 127)
    err = np.abs(x64 - Xq.astype(np.float64) * a[:, None].astype(np.float64) / 127.0)
    # fp64 slack: the bound is reached exactly at ties
    assert np.all(err <= 0.5 * a[:, None].astype(np.float64) / 127.0 * (1 + 1e-12))
    assert np.array_equal(a, np.abs(x64).max(1).astype(np.float32))
    nz = a > 0
    assert np.all(np.abs(Xq[nz].astype(np.int32)).max(1) == 127)
    assert a[5] == 0 and not Xq[5].any()


def test_weight_round_trip_and_invariants():
    rng = np.random.default_rng(4)
    W_t = (rng.standard_normal((40, 128)) * 0.02).astype(f16)
    W_t[7] = 0.0
    CB, SCB = oracle.quantize_weight(W_t)
    w64 = W_t.astype(np.float64)
    assert np.array_equal(SCB, np.abs(w64).max(1).astype(np.float32))
    rec = CB.astype(np.float64) * SCB[:, None].astype(np.float64) / 127.0
    assert np.all(np.abs(rec - w64) <= 0.5 * SCB[:, None].astype(np.float64) / 127.0 * (1 + 1e-12))
    assert np.all(np.abs(CB.astype(np.int32)).max(1)[SCB > 0] == 127)
    assert SCB[7] == 0 and not CB[7].any()
    assert CB.min() >= -127


def test_dequant_weight_all_pairs():
    """fp16 nearest to cb*scb/127 for every cb in [-127,127] and a spread of scb."""
    scb_bits = np.arange(1, 0x7C00, 7, dtype=np.uint32).astype(np.uint16)
    scb = scb_bits.view(f16).astype(np.float32)
    cb = np.arange(-127, 128, dtype=np.int8)
    CBm, SCm = np.meshgrid(cb, scb, indexing="ij")
    got = oracle.dequant_weight(CBm, SCm)
    ref = ((CBm.astype(np.float64) * SCm.astype(np.float64)) / 127.0).astype(f16).view(np.uint16)
    assert np.array_equal(got, ref)
    # the GPU route: exact fp32 product, one fp32 division, then fp32 -> fp16
    ref32 = ((CBm.astype(np.float32) * SCm) / np.float32(127.0)).astype(f16).view(np.uint16)
    assert np.array_equal(got, ref32)
