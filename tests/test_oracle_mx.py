"""Pins of the oracle's MXFP8 quantiser (oracle/mx.py).

Checked against: hand-computed blocks (tests/golden/mx_blocks.json, from the
OCP MX conversion rule), torch's float8_e4m3fn cast (an independent library
encoder: nearest-even, subnormals), the exhaustive code table, and the
format's error bound.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle.mx import (e4m3_decode, e4m3_encode, e8m0_decode, mx_dequantize,
                       mx_quantize, mx_roundtrip)

GOLD = os.path.join(os.path.dirname(__file__), "golden", "mx_blocks.json")


def torch_e4m3(v):
    """torch's encoder on values already clamped to [-448, 448]."""
    t = torch.tensor(np.asarray(v, np.float64)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_golden_blocks():
    for case in json.load(open(GOLD))["blocks"]:
        v = np.array(case["values"], np.float64)[None, :]
        codes, scales = mx_quantize(v, axis=1)
        assert int(scales[0, 0]) == case["scale"], case["why"]
        assert codes[0].tolist() == case["codes"], case["why"]


def test_decode_matches_torch_table():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]


def test_every_finite_code_roundtrips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)
    # -0 encodes as +0: the sign bit is set only for values < 0
    assert e4m3_encode(np.array([-0.0]))[0] == 0


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_encode_matches_torch_cast(seed):
    rng = np.random.default_rng(seed)
    # log-uniform magnitudes across the whole range, subnormals included
    mag = np.exp2(rng.uniform(-12, np.log2(448.0), 200_000))
    v = mag * rng.choice([-1.0, 1.0], mag.size)
    # exact midpoints between neighbouring codes (ties to even)
    vals = e4m3_decode(np.arange(0, 0x7E, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    v = np.concatenate([v, mids, -mids, [448.0, -448.0, 2.0 ** -10, -2.0 ** -10]])
    assert np.array_equal(e4m3_encode(v), torch_e4m3(v))


def test_clamp_and_ties_at_the_top():
    assert e4m3_encode(np.array([448.0]))[0] == 0x7E
    # 432 is the midpoint of 416 (mantissa 5) and 448 (mantissa 6): even wins
    assert e4m3_encode(np.array([432.0, 431.0]))[0:2].tolist() == [0x7E, 0x7D]
    # values above 448 reach the encoder only after the block clamp
    c, s = mx_quantize(np.array([[449.0, 464.0, 480.0, 511.0] + [0.0] * 28]), axis=1)
    assert s[0, 0] == 127 and c[0, :4].tolist() == [0x7E] * 4
    with pytest.raises(ValueError):
        e4m3_encode(np.array([449.0]))


def test_subnormal_and_zero_rounding():
    got = e4m3_encode(np.array([2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -9, 7.5 * 2.0 ** -9]))
    assert got.tolist() == [0x00, 0x02, 0x01, 0x08]


@pytest.mark.parametrize("n", [-20, -3, 0, 5, 17])
@pytest.mark.parametrize("frac", [1.0, 1.75, 1.99])
def test_scale_code_is_floor_log2_amax_minus_8(n, frac):
    rng = np.random.default_rng(n + 100)
    amax = frac * 2.0 ** n
    b = rng.uniform(-amax, amax, 32)
    b[7] = -amax
    _, s = mx_quantize(b[None, :], axis=1)
    assert int(s[0, 0]) == n - 8 + 127
    assert e8m0_decode(s)[0, 0] == 2.0 ** (n - 8)


def test_error_bound_and_axis_handling():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((6, 64, 96))
    for axis in (0, 1, 2) if False else (1, 2):
        c, s = mx_quantize(v, axis=axis)
        assert c.shape == v.shape
        assert s.shape[axis] == v.shape[axis] // 32
        d = mx_dequantize(c, s, axis=axis)
        assert np.array_equal(d, mx_roundtrip(v, axis=axis))
        # per-element bound for values the block scale keeps in the normal range
        amax = np.max(np.abs(np.moveaxis(v, axis, -1).reshape(-1, 32)), axis=1)
        scale = np.exp2(np.floor(np.log2(amax)) - 8)
        vv = np.moveaxis(v, axis, -1).reshape(-1, 32)
        dd = np.moveaxis(d, axis, -1).reshape(-1, 32)
        scaled = np.abs(vv) / scale[:, None]
        ok = (scaled >= 2.0 ** -6) & (scaled <= 448)
        bound = np.exp2(np.floor(np.log2(np.abs(vv))) - 4)
        assert np.all(np.abs(vv - dd)[ok] <= bound[ok])
        # subnormal region: absolute error at most half the subnormal step
        sub = scaled < 2.0 ** -6
        assert np.all((np.abs(vv - dd) / scale[:, None])[sub] <= 2.0 ** -10)


def test_zero_block():
    c, s = mx_quantize(np.zeros((2, 64)), axis=1)
    assert not c.any() and not s.any()
    assert not mx_dequantize(c, s, axis=1).any()


def test_non_multiple_of_32_rejected():
    with pytest.raises(ValueError):
        mx_quantize(np.zeros((1, 48)), axis=1)


# --- quantisation down the rows (the MX weight-gradient recipe) -------------

def _representable_rows(n, m, seed):
    """An n x m matrix whose 32-row blocks (per column) are exactly
    representable: each block gets its own scale 2^s, one element of E4M3
    exponent 8 (so the block maximum selects exactly s) and the rest E4M3
    values that include subnormals (which a wrong block grouping, choosing a
    larger scale, would round away)."""
    rng = np.random.default_rng(seed)
    v = np.zeros((n, m))
    top = 256.0 + 32.0 * np.arange(7)          # E4M3 values with exponent 8: 256 .. 448
    small = np.ldexp(np.arange(1, 8), -9)       # E4M3 subnormals
    mid = np.ldexp(8.0 + np.arange(8), -3)      # normals in [1, 2)
    for b0 in range(0, n, 32):
        rows = min(32, n - b0)
        for c in range(m):
            s = int(rng.integers(-20, 20))
            blk = rng.choice(np.concatenate([small, mid, -small, -mid]), rows)
            blk[rng.integers(rows)] = rng.choice(top) * rng.choice([-1.0, 1.0])
            v[b0:b0 + rows, c] = np.ldexp(blk, s)
    return v


def test_rows_roundtrip_identity_on_representable_blocks():
    from oracle.mx import mx_roundtrip, mx_rows_roundtrip
    v = _representable_rows(96, 32, seed=1)
    assert np.array_equal(mx_rows_roundtrip(v), v)
    # quantising along the other axis instead loses the per-row-block scales
    assert not np.array_equal(mx_roundtrip(v, axis=1), v)


def test_rows_roundtrip_ragged_segment_zero_padded():
    from oracle.mx import mx_rows_roundtrip
    v = _representable_rows(37, 4, seed=2)      # last block holds 5 real rows
    assert np.array_equal(mx_rows_roundtrip(v), v)
    r = np.random.default_rng(3).standard_normal((37, 6))
    padded = np.vstack([r, np.zeros((27, 6))])
    assert np.array_equal(mx_rows_roundtrip(r), mx_rows_roundtrip(padded)[:37])


def test_rows_roundtrip_matches_column_quantiser_transposed():
    from oracle.mx import mx_roundtrip, mx_rows_roundtrip
    r = np.random.default_rng(4).standard_normal((64, 7)) * 3.0
    # blocks down the rows of r are blocks along the columns of r^T
    assert np.array_equal(mx_rows_roundtrip(r), mx_roundtrip(r.T, axis=1).T)
    assert not np.array_equal(mx_rows_roundtrip(r[:, :32 * 0 + 7]), r)


def test_rows_roundtrip_product_within_e4m3_bound():
    """|Q(A)^T Q(B) - A^T B| within the bound E4M3/E8M0 rounding allows:
    per value |q - v| <= 2^-4 |v| + 2^-18 amax(block) + max(0, |v| - 448 2^s)
    with 2^s = 2^(floor(log2 amax) - 8): half an ulp with 3 mantissa bits;
    below the normals half the 2^-9 quantum of 2^s (2^s <= amax / 256); and
    the saturation of block values between 448 and 512 times 2^s."""
    from oracle.mx import mx_rows_roundtrip
    rng = np.random.default_rng(5)
    A = rng.standard_normal((70, 9)) * np.exp(rng.standard_normal((70, 1)))
    B = rng.standard_normal((70, 11))

    def err_bound(M):
        pad = np.vstack([np.abs(M), np.zeros(((-len(M)) % 32, M.shape[1]))])
        amax = pad.reshape(-1, 32, M.shape[1]).max(axis=1)
        amax_rows = np.repeat(amax, 32, axis=0)[:len(M)]
        scale = np.ldexp(1.0, np.frexp(amax_rows)[1] - 1 - 8)
        return (2.0 ** -4 * np.abs(M) + 2.0 ** -18 * amax_rows
                + np.maximum(0.0, np.abs(M) - 448.0 * scale))

    eA, eB = err_bound(A), err_bound(B)
    qA, qB = mx_rows_roundtrip(A), mx_rows_roundtrip(B)
    assert np.all(np.abs(qA - A) <= eA) and np.all(np.abs(qB - B) <= eB)
    bound = eA.T @ np.abs(B) + np.abs(A).T @ eB + eA.T @ eB
    assert np.all(np.abs(qA.T @ qB - A.T @ B) <= bound * (1 + 1e-12))
    # and the quantisation is not the identity on these inputs
    assert np.abs(qA - A).max() > 0


def test_backward_mx_wgrad_recipe():
    """With MXFP8 and mx_wgrad the weight gradients move by at most the MX
    error of their operands; the data gradients do not move at all."""
    import oracle
    import synth
    w = synth.custom(T=48, H=128, E=3, k=2, I=64, routing="supplied", mx=True, seed=9)
    inp = synth.make_inputs(w)
    fw = oracle.forward(inp, w.k, mx=True)
    b0 = oracle.backward(inp, fw)
    b1 = oracle.backward(inp, fw, mx_wgrad=True)
    assert np.array_equal(b0["dx"], b1["dx"]) and np.array_equal(b0["dX"], b1["dX"])
    for key in ("dWg", "dWu", "dWd"):
        d = np.abs(b1[key] - b0[key]).max() / np.abs(b0[key]).max()
        assert 0 < d < 0.1, (key, d)
