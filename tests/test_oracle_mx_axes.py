"""Pins of the axis along which the oracle quantises each expert weight (MXFP8).

Each GEMM's MX operands carry one E8M0 scale per 32 values along that GEMM's
contraction axis.  The forward contracts W_gate, W_up [H, I] over H and
W_down [I, H] over I; the backward data gradients contract W_gate, W_up over
I (dX = dg W_gate^T + du W_up^T) and W_down over H (dA = dY W_down^T).

The weights here are built so that every 32-block along one chosen axis is
exactly representable in MXFP8 (its own power-of-two scale, one element in
the top binade, the rest E4M3 values down to the subnormals) while the
32-blocks across that axis are not (they mix scales, so the larger scale
rounds the small values away).  Quantising along the right axis is then the
identity and along the other axis is not, which the checks below observe
through the layer's own outputs.  A mutated oracle that swaps any axis fails
them (``test_swapped_axis_is_caught``).
"""
import numpy as np
import pytest

import oracle
from oracle import layer as L
from oracle.mx import FORMATS, mx_roundtrip
from oracle.numerics import bf16, bf16_to_f64, f32
from synth import f32_to_bf16_bits

FMTS = ("e4m3", "e2m1", "e2m3", "e3m2")


def _levels(fmt):
    """(values of the format's top binade, its other nonzero values, the
    smallest ones included)."""
    F = FORMATS[fmt]
    mags = F.table[: F.ncodes // 2]
    mags = mags[np.isfinite(mags) & (mags > 0)]
    top = mags[np.floor(np.log2(mags)) == F.emax]
    return top, mags[np.floor(np.log2(mags)) < F.emax]


def representable(shape, axis, seed, s_lo=-14, s_hi=-9, fmt="e4m3"):
    """bf16 bits of a 2-D matrix whose 32-blocks along ``axis`` are exactly
    representable in MX format ``fmt``, each with its own scale 2^s, s in
    [s_lo, s_hi] (shifted by the format's emax relative to E4M3's)."""
    TOP, VALS = _levels(fmt)
    shift = 8 - FORMATS[fmt].emax
    s_lo, s_hi = s_lo + shift, s_hi + shift
    rng = np.random.default_rng(seed)
    v = np.moveaxis(np.zeros(shape), axis, -1)
    nb = v.shape[-1] // 32
    blk = rng.choice(np.concatenate([VALS, -VALS]), v.shape[:-1] + (nb, 32))
    top = rng.integers(32, size=v.shape[:-1] + (nb,))
    np.put_along_axis(blk, top[..., None],
                      (rng.choice(TOP, top.shape) * rng.choice([-1.0, 1.0], top.shape))[..., None],
                      axis=-1)
    s = rng.integers(s_lo, s_hi + 1, size=v.shape[:-1] + (nb, 1))
    v = np.moveaxis(np.ldexp(blk, s).reshape(v.shape), -1, axis)
    bits = f32_to_bf16_bits(v.astype(np.float32))
    assert np.array_equal(bf16_to_f64(bits), v)          # exact in bf16
    return bits


def _inputs(T, H, E, I, w_axis, seed, fmt="e4m3"):
    """A top-1 layer (weight 1.0 per token, so dY is dOut itself) whose x and
    dOut rows are representable along H in MXFP8 and whose expert weights are
    representable in ``fmt`` along axis ``w_axis`` of each [rows, cols]
    matrix."""
    rng = np.random.default_rng(seed)

    def w(shape, sd):
        return representable(shape, w_axis, sd, fmt=fmt)
    inp = dict(x=representable((T, H), 1, seed + 1, -8, -6),
               dout=representable((T, H), 1, seed + 2, -8, -6),
               w_gate=np.stack([w((H, I), seed + 10 + e) for e in range(E)]),
               w_up=np.stack([w((H, I), seed + 20 + e) for e in range(E)]),
               w_down=np.stack([w((I, H), seed + 30 + e) for e in range(E)]),
               topk_idx=rng.integers(E, size=(T, 1)).astype(np.int32),
               topk_w=np.ones((T, 1), np.float32))
    return inp


T, H, E, I = 96, 128, 3, 64


def check_forward_axes(inp, fmt="e4m3"):
    """With weights representable along the forward contraction axis (-2),
    the MX forward's g, u are the unquantised products and Y is the product of
    its quantised activation with the raw W_down."""
    fx = oracle.forward(inp, 1, mx=True, wfmt=fmt)
    fb = oracle.forward(inp, 1, mx=False)
    assert np.array_equal(fx["Xhat"], fb["Xhat"])           # x rows representable
    assert np.array_equal(fx["g"], fb["g"]), "gate weights quantised across H"
    assert np.array_equal(fx["u"], fb["u"]), "up weights quantised across H"
    for e in range(E):
        rs = slice(int(fx["offsets"][e]), int(fx["offsets"][e + 1]))
        Wd = bf16_to_f64(inp["w_down"][e])
        assert np.array_equal(fx["Y"][rs], bf16(fx["ahat"][rs] @ Wd)), \
            "down weights quantised across I"


def check_backward_axes(inp, fmt="e4m3"):
    """With weights representable along the backward contraction axis (-1),
    the MX backward's dg, du equal those of the unquantised backward over the
    same forward state (dY = dOut is representable along H), and dX is the
    product of the quantised dg, du with the raw W_gate, W_up."""
    fx = oracle.forward(inp, 1, mx=True, wfmt=fmt)
    bx = oracle.backward(inp, fx)
    fb = dict(fx, mx=False, W=L.ExpertWeights(inp, False))
    bb = oracle.backward(inp, fb)
    assert np.array_equal(bx["dY"], bf16_to_f64(inp["dout"])[fx["perm"]])
    assert np.array_equal(bx["dg"], bb["dg"]), "down weights quantised across H"
    assert np.array_equal(bx["du"], bb["du"]), "down weights quantised across H"
    for e in range(E):
        rs = slice(int(fx["offsets"][e]), int(fx["offsets"][e + 1]))
        Wg, Wu = bf16_to_f64(inp["w_gate"][e]), bf16_to_f64(inp["w_up"][e])
        ref = bf16(mx_roundtrip(bx["dg"][rs], axis=1) @ Wg.T
                   + mx_roundtrip(bx["du"][rs], axis=1) @ Wu.T)
        assert np.array_equal(bx["dX"][rs], ref), "gate/up weights quantised across I"


@pytest.mark.parametrize("fmt", FMTS)
def test_construction_is_one_sided(fmt):
    for axis in (0, 1):
        v = bf16_to_f64(representable((128, 64), axis, 3, fmt=fmt))
        assert np.array_equal(mx_roundtrip(v, axis=axis, fmt=fmt), v)
        assert not np.array_equal(mx_roundtrip(v, axis=1 - axis, fmt=fmt), v)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("backward", [False, True])
def test_expert_weights_quantise_along_the_contraction_axis(backward, fmt):
    axis = -1 if backward else -2
    inp = _inputs(T, H, E, I, axis, seed=5, fmt=fmt)
    W = L.ExpertWeights(inp, mx=True, wfmt=fmt)
    for e in range(E):
        got = W.bwd(e) if backward else W.fwd(e)
        other = W.fwd(e) if backward else W.bwd(e)
        for key, src in (("g", "w_gate"), ("u", "w_up"), ("d", "w_down")):
            raw = bf16_to_f64(inp[src][e])
            assert np.array_equal(got[key], raw), (key, e)
            assert not np.array_equal(other[key], raw), (key, e)


@pytest.mark.parametrize("fmt", FMTS)
def test_mx_forward_quantises_weights_along_h_for_gate_up_and_i_for_down(fmt):
    check_forward_axes(_inputs(T, H, E, I, -2, seed=7, fmt=fmt), fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_mx_backward_quantises_weights_along_i_for_gate_up_and_h_for_down(fmt):
    check_backward_axes(_inputs(T, H, E, I, -1, seed=9, fmt=fmt), fmt)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("which", ["gate", "up", "down"])
@pytest.mark.parametrize("backward", [False, True])
def test_swapped_axis_is_caught(monkeypatch, which, backward, fmt):
    """Swap the axis of one weight in one direction: the matching check fails."""
    orig = L.expert_weights
    mutate_backward = backward

    def mutant(w_gate, w_up, w_down, mx, backward=False, wfmt="e4m3"):
        W = orig(w_gate, w_up, w_down, mx, backward, wfmt)
        bwd = backward
        if mx and bwd == mutate_backward:
            key = dict(gate="g", up="u", down="d")[which]
            raw = dict(g=w_gate, u=w_up, d=w_down)[key]
            W[key] = mx_roundtrip(L._val(raw), axis=-2 if bwd else -1, fmt=wfmt)
        return W

    monkeypatch.setattr(L, "expert_weights", mutant)
    if backward:
        inp = _inputs(T, H, E, I, -1, seed=9, fmt=fmt)
        with pytest.raises(AssertionError):
            check_backward_axes(inp, fmt)
    else:
        inp = _inputs(T, H, E, I, -2, seed=7, fmt=fmt)
        with pytest.raises(AssertionError):
            check_forward_axes(inp, fmt)


def test_exact_weights_give_f32_products():
    """Sanity of the construction: f32 of the products is what g holds."""
    inp = _inputs(T, H, E, I, -2, seed=7)
    fx = oracle.forward(inp, 1, mx=True)
    e = int(inp["topk_idx"][0, 0])
    r = int(fx["inv"][0])
    x0 = bf16_to_f64(inp["x"][0])
    assert np.array_equal(fx["g"][r], f32(x0 @ bf16_to_f64(inp["w_gate"][e])))
