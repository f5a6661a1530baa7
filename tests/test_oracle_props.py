"""Randomised properties of the oracle over small shapes (hypothesis).

Shapes: T in 1..64, E in 1..16, k in 1..8 (k > E allowed with supplied
routing, which then repeats experts), skewed expert probabilities that leave
experts without rows or put every row on one expert, bf16 and MXFP8.  For
each drawn layer:
* the layout is a stable counting sort (counts sum to T*k, segments hold only
  their expert in ascending flat order, inv is perm's inverse);
* dispatch then scatter-back by inv returns every token k times;
* the layer's forward output and its dx and dw equal the per-token brute
  force (no layout, no permutation) bit for bit.
"""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import synth
from oracle.layer import TokenEvaluator, dispatch, layout
from oracle.numerics import bf16_to_f64


@st.composite
def layers(draw):
    T = draw(st.integers(1, 64))
    E = draw(st.integers(1, 16))
    k = draw(st.integers(1, 8))
    skew = draw(st.sampled_from(["uniform", "zero-load", "one-expert", "zipf"]))
    mx = draw(st.booleans())
    seed = draw(st.integers(0, 2 ** 16))
    probs = None
    if skew == "zero-load" and E > 1:
        probs = tuple(float(i % 2) for i in range(E))   # odd experts only
    elif skew == "one-expert":
        probs = (1.0,) + (0.0,) * (E - 1)
    zipf = 1.2 if skew == "zipf" else 0.0
    w = synth.custom(T=T, H=64, E=E, k=k, I=32, routing="supplied", zipf_s=zipf,
                     expert_probs=probs, mx=mx, seed=seed)
    return w


@settings(max_examples=25, deadline=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(layers())
def test_layout_and_permutation_properties(w):
    inp = synth.make_inputs(w, only={"x", "topk_idx", "topk_w"})
    idx = inp["topk_idx"]
    counts, offsets, perm, inv = layout(idx, w.E)
    flat = idx.reshape(-1)
    R = w.T * w.k
    assert counts.sum() == R and offsets[0] == 0 and offsets[-1] == R
    assert np.array_equal(inv[perm], np.arange(R))
    for e in range(w.E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)
    xp = dispatch(inp["x"], perm, w.k)
    assert np.array_equal(xp[inv].reshape(w.T, w.k, -1),
                          np.repeat(inp["x"][:, None, :], w.k, axis=1))


@settings(max_examples=12, deadline=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(layers())
def test_layer_equals_per_token_brute_force(w):
    inp = synth.make_inputs(w)
    fw = oracle.forward(inp, w.k, mx=w.mx)
    bw = oracle.backward(inp, fw)
    ev = TokenEvaluator(inp, w.k, mx=w.mx)
    dout = bf16_to_f64(inp["dout"])
    for t in range(w.T):
        tk = ev.token(t)
        assert np.array_equal(tk["out"], fw["out"][t])
        tg = ev.token_grad(t, dout[t])
        assert np.array_equal(tg["dw"], bw["dw"][t])
        assert np.array_equal(tg["dx"], bw["dx"][t])
