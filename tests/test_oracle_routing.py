"""Pins of the oracle's router, top-k selection and layout (oracle/layer.py).

Checked against: hand-worked fixtures (tests/golden/topk_cases.json,
layout_cases.json), Python's own stable ``sorted`` on the ordering key,
closed forms (one-hot tokens, k = 1, k = E), the full-softmax formulation,
layout invariants, and the synthetic hot-expert share of the skewed workload.
"""
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import layout, router_logits, topk_softmax
from oracle.numerics import bf16_bits

G = os.path.join(os.path.dirname(__file__), "golden")


def test_topk_golden():
    for c in json.load(open(os.path.join(G, "topk_cases.json")))["cases"]:
        L = np.array([c["logits"]], np.float32)
        idx, w = topk_softmax(L, c["k"])
        assert idx[0].tolist() == c["idx"], c["why"]
        assert np.allclose(w[0], c["w"], rtol=0, atol=2e-7), c["why"]


@pytest.mark.parametrize("ties", [False, True])
@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (50, 64, 6), (20, 256, 8), (9, 5, 5)])
def test_topk_equals_python_sorted(T, E, k, ties):
    L = synth.router_logits_inputs(T, E, seed=3, ties=ties)
    idx, w = topk_softmax(L, k)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(L[t, e]), e))
        assert idx[t].tolist() == order[:k]
    # renormalised top-k == full softmax, restricted to the selection, renormalised
    p = np.exp(L.astype(np.float64) - L.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    sel = np.take_along_axis(p, idx, axis=1)
    assert np.allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-6, atol=0)
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)   # slot order follows descending logit


def test_topk_k1_and_kE():
    L = synth.router_logits_inputs(40, 16, seed=9)
    _, w1 = topk_softmax(L, 1)
    assert np.all(w1 == 1.0)
    idx, _ = topk_softmax(L, 16)
    assert all(sorted(r) == list(range(16)) for r in idx.tolist())
    assert np.all(np.diff(np.take_along_axis(L, idx, 1), axis=1) <= 0)


def test_router_logits_closed_form():
    # one-hot tokens pick out rows of W_r; the bias is added to every token
    H, E = 16, 5
    rng = np.random.default_rng(0)
    Wr = bf16_bits(rng.standard_normal((H, E)))
    bias = rng.standard_normal(E).astype(np.float32)
    x = np.zeros((H, H), np.uint16)
    x[np.arange(H), np.arange(H)] = 0x3F80          # bf16 1.0
    from oracle.numerics import bf16_to_f64
    L = router_logits(x, Wr, bias)
    assert np.array_equal(L, (bf16_to_f64(Wr) + bias.astype(np.float64)).astype(np.float32)
                          .astype(np.float64))
    L2 = router_logits(x[:3] * 0, Wr)                # zero tokens -> zero logits
    assert not L2.any()


def test_layout_golden():
    for c in json.load(open(os.path.join(G, "layout_cases.json")))["cases"]:
        counts, offsets, perm, inv = layout(np.array(c["idx"]), c["E"])
        assert counts.tolist() == c["counts"], c["why"]
        assert offsets.tolist() == c["offsets"], c["why"]
        assert perm.tolist() == c["perm"], c["why"]
        assert inv.tolist() == c["inv"], c["why"]


def _check_layout(idx, E):
    counts, offsets, perm, inv = layout(idx, E)
    flat = np.asarray(idx).reshape(-1)
    R = flat.size
    assert counts.sum() == R and offsets[0] == 0 and offsets[-1] == R
    assert np.all(np.diff(offsets) == counts)
    assert sorted(perm.tolist()) == list(range(R))
    assert np.array_equal(inv[perm], np.arange(R))
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)
    brute = sorted(range(R), key=lambda f: (int(flat[f]), f))
    assert perm.tolist() == brute


@pytest.mark.parametrize("T,E,k,probs", [
    (1, 1, 1, None), (1, 8, 2, None), (37, 8, 2, None), (300, 64, 6, None),
    (128, 6, 8, (1, 0, 0, 3, 0, 2)),        # zero-load experts, duplicates (k > E)
    (64, 16, 4, (1,) + (0,) * 15),           # every row on one expert
])
def test_layout_invariants(T, E, k, probs):
    idx, _ = synth.supplied_routing(T, E, k, seed=T + E, probs=probs)
    _check_layout(idx, E)


def test_layout_rejects_bad_expert():
    with pytest.raises(ValueError):
        layout(np.array([[0, 4]]), 4)


@pytest.mark.slow
def test_dsv3_hot_expert_share():
    """The skewed workload's bias sends about half the routed rows to 10 % of experts."""
    w = synth.workload("dsv3-bf16")
    # only x, the router and the bias are needed: draw them alone
    inp = synth.make_inputs(w, only={"x", "w_router", "bias"})
    L = router_logits(inp["x"], inp["w_router"], inp["bias"])
    idx, _ = topk_softmax(L, w.k)
    share = np.isin(idx, inp["hot"]).mean()
    assert math.ceil(0.1 * w.E) == w.hot_experts == len(inp["hot"])
    assert 0.49 <= share <= 0.51, share


def test_forward_routes_from_given_logits():
    """forward(logits=L) with the router's own fp32 logits reproduces the
    router-routed layer bit for bit (backward included); other logits change
    the selection exactly as topk_softmax of them does."""
    import oracle
    w = synth.custom(T=40, H=64, E=8, k=3, I=32, routing="router", router_std=0.3, seed=4)
    inp = synth.make_inputs(w)
    a = oracle.forward(inp, w.k)
    b = oracle.forward(inp, w.k, logits=a["logits"])
    for key in ("idx", "w", "perm", "out", "Y"):
        assert np.array_equal(a[key], b[key]), key
    ga, gb = oracle.backward(inp, a), oracle.backward(inp, b)
    for key in ("dx", "dWr", "dWg", "dw"):
        assert np.array_equal(ga[key], gb[key]), key
    L2 = a["logits"][:, ::-1].copy()
    c = oracle.forward(inp, w.k, logits=L2)
    idx, wts = oracle.topk_softmax(L2, w.k)
    assert np.array_equal(c["idx"], idx) and np.array_equal(c["w"], wts)
    with np.testing.assert_raises(ValueError):
        oracle.forward(inp, w.k, logits=a["logits"] + 1e-12)
