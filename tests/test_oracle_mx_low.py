"""Pins of the oracle's lower-precision MX element formats (oracle/mx.py):
FP4 E2M1, FP6 E2M3, FP6 E3M2 with one E8M0 scale per 32 values.

Checked against: the formats' value sets as the OCP MX specification defines
them (E2M1's eight magnitudes listed outright; the extremes of the FP6
formats), hand-computed blocks (tests/golden/mx_low_blocks.json), a brute
force that picks the nearest value of each format's full code table (ties to
the even code), round trips of every code, the generic encoder against the
torch-pinned E4M3 encoder on the E4M3 format, and the quantisation error
bound.  (torch has no fp6 type and cannot cast to its fp4 type.)
"""
import json
import os

import numpy as np
import pytest

from oracle.mx import FORMATS, e4m3_encode, mx_dequantize, mx_quantize, mx_roundtrip

GOLD = os.path.join(os.path.dirname(__file__), "golden", "mx_low_blocks.json")
LOW = ("e2m1", "e2m3", "e3m2")


def test_value_sets_as_the_specification_defines_them():
    e2m1 = FORMATS["e2m1"].table
    assert sorted(set(np.abs(e2m1))) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert e2m1.size == 16 and np.all(np.isfinite(e2m1))
    e2m3 = np.abs(FORMATS["e2m3"].table)
    assert e2m3.max() == 7.5 and sorted(set(e2m3))[1] == 0.125 and e2m3.size == 64
    e3m2 = np.abs(FORMATS["e3m2"].table)
    assert e3m2.max() == 28.0 and sorted(set(e3m2))[1] == 0.0625 and e3m2.size == 64
    # the binade ladder: smallest normal 1 (E2M1, E2M3) and 0.25 (E3M2)
    assert FORMATS["e2m3"].decode(np.uint8(8)) == 1.0
    assert FORMATS["e3m2"].decode(np.uint8(4)) == 0.25
    for f in LOW:
        assert FORMATS[f].emax == {"e2m1": 2, "e2m3": 2, "e3m2": 4}[f]


@pytest.mark.parametrize("fmt", LOW)
def test_every_code_round_trips(fmt):
    F = FORMATS[fmt]
    neg_zero = 1 << (F.ebits + F.mbits)
    codes = np.array([c for c in range(F.ncodes) if c != neg_zero], np.uint8)
    assert np.array_equal(F.encode(F.decode(codes)), codes)
    assert F.encode(np.array([-0.0]))[0] == 0


def _brute_force(F, v):
    """Nearest value of the code table; ties to the code with an even
    mantissa; the sign bit set exactly for v < 0."""
    mags = F.table[: F.ncodes // 2]            # non-negative codes, ascending
    out = np.empty(v.shape, np.int64)
    for i, x in np.ndenumerate(v):
        d = np.abs(mags - abs(x))
        best = np.flatnonzero(d == d.min())
        c = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        out[i] = c | ((x < 0) << (F.ebits + F.mbits))
    return out.astype(np.uint8)


@pytest.mark.parametrize("fmt", LOW)
def test_encoder_matches_brute_force_nearest(fmt):
    F = FORMATS[fmt]
    rng = np.random.default_rng(11)
    lo = np.log2(F.table[1]) - 2
    mag = np.exp2(rng.uniform(lo, np.log2(F.max), 3000))
    mags = F.table[: F.ncodes // 2]
    mids = (mags[:-1] + mags[1:]) / 2                # exact ties
    v = np.concatenate([mag, mids, np.nextafter(mids, 0), np.nextafter(mids, 9), [F.max, 0.0]])
    v = v * rng.choice([-1.0, 1.0], v.size)
    assert np.array_equal(F.encode(v), _brute_force(F, v))


def test_generic_encoder_is_the_e4m3_encoder_on_e4m3():
    rng = np.random.default_rng(3)
    v = np.exp2(rng.uniform(-12, np.log2(448.0), 20000)) * rng.choice([-1.0, 1.0], 20000)
    assert np.array_equal(FORMATS["e4m3"].encode(v), e4m3_encode(v))


def test_golden_blocks():
    for case in json.load(open(GOLD))["blocks"]:
        v = np.array(case["values"], np.float64)[None, :]
        codes, scales = mx_quantize(v, axis=1, fmt=case["fmt"])
        assert int(scales[0, 0]) == case["scale"], case["why"]
        assert codes[0].tolist() == case["codes"], case["why"]


@pytest.mark.parametrize("fmt", LOW)
def test_scale_and_error_bound(fmt):
    F = FORMATS[fmt]
    rng = np.random.default_rng(5)
    v = rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    c, s = mx_quantize(v, axis=1, fmt=fmt)
    amax = np.abs(v).reshape(64, 8, 32).max(axis=2)
    assert np.array_equal(s.astype(np.int64) - 127, np.floor(np.log2(amax)).astype(np.int64) - F.emax)
    q = mx_dequantize(c, s, axis=1, fmt=fmt)
    assert np.array_equal(mx_roundtrip(v, axis=1, fmt=fmt), q)
    scale = np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)
    # half a spacing of the value's binade (floored at the smallest normal),
    # plus what saturation at the format's maximum removes
    e = np.maximum(np.floor(np.log2(np.maximum(np.abs(v) / scale, 1e-300))), F.emin)
    bound = np.exp2(e - F.mbits - 1) * scale + np.maximum(0, np.abs(v) - F.max * scale)
    assert np.all(np.abs(q - v) <= bound * (1 + 1e-12))
    assert np.abs(q - v).max() > 0
