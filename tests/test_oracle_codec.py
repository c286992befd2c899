"""Pins of the oracle's binary16 codec against numpy's independent float16.

The codec is written from the bit layout (1 sign, 5 exponent, 10 fraction
bits; techblog.paldyn.com quantization basics, section on FP16).  numpy's
float16 conversions are a separate implementation of IEEE-754 binary16 with
round-to-nearest-even, so agreement on every bit pattern and on every
midpoint pins both directions.
"""
import json
import os

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_half_to_double_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.half_to_double(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_fp16_max_matches_page():
    g = json.load(open(os.path.join(GOLDEN, "decomposition_constants.json")))["fp16_max"]
    assert oracle.half_to_double(np.array([0x7BFF], np.uint16))[0] == g["value"]
    assert oracle.double_to_half(np.array([g["value"]]))[0] == 0x7BFF
    # just past the largest finite value: the midpoint 65520 rounds (to even) to inf
    assert oracle.double_to_half(np.array([65519.99]))[0] == 0x7BFF
    assert oracle.double_to_half(np.array([65520.0]))[0] == 0x7C00
    assert oracle.double_to_half(np.array([-1e6]))[0] == 0xFC00


def _all_finite_halves():
    bits = np.arange(0, 0x7C00, dtype=np.uint16)  # +0 .. 65504
    return bits.view(np.float16).astype(np.float64)


def test_double_to_half_midpoints_and_neighbours():
    v = _all_finite_halves()
    mids = (v[:-1] + v[1:]) / 2.0             # exact in fp64: ties
    eps = np.abs(mids) * 2.0 ** -40 + 2.0 ** -70
    cand = np.concatenate([v, mids, mids + eps, mids - eps, [65520.0, 65520.0 - 1e-9, 70000.0]])
    cand = np.concatenate([cand, -cand])
    got = oracle.double_to_half(cand)
    ref = cand.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_double_to_half_random():
    rng = np.random.default_rng(1)
    mag = np.exp(rng.uniform(np.log(1e-9), np.log(1e6), 2_000_000))
    v = mag * np.where(rng.random(mag.size) < 0.5, -1.0, 1.0)
    got = oracle.double_to_half(v)
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
