"""Pins of the oracle's whole layer (oracle/layer.py), forward and backward.

Checked against:
* brute force per token (no layout, no permutation) -- bit-exact;
* one expert, top-1 == a dense SwiGLU FFN computed with torch's own silu,
  matmul and bf16 cast -- bit-exact;
* permute then unpermute is the identity (k = 1 exact; k > 1 up to fp32);
* counts sum to tokens x top-k on every workload;
* central finite differences of the rounding-free oracle (fp64), for every
  parameter, router included;
* torch fp64 autograd of an independent index_add formulation.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.layer import TokenEvaluator, combine, dispatch, layout
from oracle.numerics import bf16_to_f64


def small(**kw):
    base = dict(T=48, H=64, E=4, k=2, I=32, routing="router", router_std=0.3, seed=1)
    base.update(kw)
    return synth.custom(**base)


CASES = {
    "router": small(),
    "supplied-dup": small(routing="supplied", k=5, E=3, zipf_s=1.0),
    "shared": small(shared_I=64, hot_experts=1, hot_bias=0.5),
    "router-mx": small(mx=True),
    "supplied-mx-shared": small(routing="supplied", mx=True, shared_I=32, k=3),
}


@pytest.mark.parametrize("name", list(CASES))
def test_brute_force_per_token_matches_layer(name):
    w = CASES[name]
    inp = synth.make_inputs(w)
    fw = oracle.forward(inp, w.k, mx=w.mx)
    bw = oracle.backward(inp, fw)
    ev = TokenEvaluator(inp, w.k, mx=w.mx)
    dout = bf16_to_f64(inp["dout"])
    for t in range(w.T):
        tk = ev.token(t)
        assert np.array_equal(tk["idx"], fw["idx"][t])
        assert np.array_equal(tk["out"], fw["out"][t])
        tg = ev.token_grad(t, dout[t])
        assert np.array_equal(tg["dw"], bw["dw"][t])
        assert np.array_equal(tg["dx"], bw["dx"][t])


def test_tiny_brute_force():
    w = synth.workload("tiny")
    inp = synth.make_inputs(w)
    fw = oracle.forward(inp, w.k)
    ev = TokenEvaluator(inp, w.k)
    for t in range(0, w.T, 17):
        assert np.array_equal(ev.token(t)["out"], fw["out"][t])


def _bf16_torch(t):
    return t.to(torch.float32).to(torch.bfloat16).to(torch.float64)


def test_one_expert_top1_is_dense_swiglu():
    w = small(E=1, k=1, routing="supplied")
    inp = synth.make_inputs(w)
    fw = oracle.forward(inp, 1)
    assert np.all(fw["w"] == 1.0)
    x = torch.from_numpy(inp["x"].astype(np.int16)).view(torch.bfloat16).to(torch.float64)
    Wg, Wu, Wd = (torch.from_numpy(inp[n][0].astype(np.int16)).view(torch.bfloat16)
                  .to(torch.float64) for n in ("w_gate", "w_up", "w_down"))
    g = (x @ Wg).to(torch.float32).to(torch.float64)
    u = (x @ Wu).to(torch.float32).to(torch.float64)
    a = _bf16_torch(torch.nn.functional.silu(g) * u)
    y = _bf16_torch(a @ Wd)
    assert np.array_equal(fw["out"], y.numpy())


def test_one_expert_top1_backward_is_dense_swiglu_backward():
    """The backward of one expert with top-1 routing against a dense SwiGLU
    backward written with torch: silu's derivative from torch's autograd, the
    bf16 and fp32 rounding points by torch's casts (saved g, u as bf16
    activations; dg, du, dX, dx stored as bf16; weight gradients in fp32)."""
    w = small(E=1, k=1, routing="supplied")
    inp = synth.make_inputs(w)
    fw = oracle.forward(inp, 1)
    bw = oracle.backward(inp, fw)

    def t(name, e=None):
        a = inp[name] if e is None else inp[name][e]
        return torch.from_numpy(a.astype(np.int16)).view(torch.bfloat16).to(torch.float64)
    x, dout = t("x"), t("dout")
    Wg, Wu, Wd = t("w_gate", 0), t("w_up", 0), t("w_down", 0)
    f32 = lambda v: v.to(torch.float32).to(torch.float64)           # noqa: E731
    g = _bf16_torch(f32(x @ Wg)).requires_grad_()
    u = _bf16_torch(f32(x @ Wu)).requires_grad_()
    a = _bf16_torch(f32(torch.nn.functional.silu(f32(x @ Wg)) * f32(x @ Wu)))
    dA = f32(dout @ Wd.T)
    (torch.nn.functional.silu(g) * u).backward(dA)
    dg, du = _bf16_torch(g.grad), _bf16_torch(u.grad)
    dX = _bf16_torch(dg @ Wg.T + du @ Wu.T)
    assert np.array_equal(bw["dx"], dX.numpy())
    assert np.array_equal(bw["dWd"][0], f32(a.T @ dout).numpy())
    assert np.array_equal(bw["dWg"][0], f32(x.T @ dg).numpy())
    assert np.array_equal(bw["dWu"][0], f32(x.T @ du).numpy())
    # g, u enter the backward as bf16: with fp32 g, u the gradients differ
    g32 = f32(x @ Wg).requires_grad_()
    u32 = f32(x @ Wu).requires_grad_()
    (torch.nn.functional.silu(g32) * u32).backward(dA)
    assert not np.array_equal(_bf16_torch(g32.grad).numpy(), dg.numpy())


@pytest.mark.parametrize("k", [1, 3])
def test_permute_unpermute_identity(k):
    T, E, H = 40, 5, 16
    idx, wts = synth.supplied_routing(T, E, k, seed=4)
    rng = np.random.default_rng(0)
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    counts, offsets, perm, inv = layout(idx, E)
    assert counts.sum() == T * k
    xp = dispatch(x, perm, k)
    # scatter by inv_perm gives x repeated k times
    assert np.array_equal(xp[inv].reshape(T, k, H), np.repeat(x[:, None, :], k, axis=1))
    # identity FFN then combine with the routing weights returns x
    out = combine(bf16_to_f64(xp), wts, inv, k)
    ref = bf16_to_f64(x)
    if k == 1:
        assert np.array_equal(out, ref)
    else:
        assert np.allclose(out, ref * wts.astype(np.float64).sum(1, keepdims=True),
                           rtol=2 ** -8, atol=0)


@pytest.mark.parametrize("name", ["tiny", "mid", "kimi-bf16", "kimi-mx"])
def test_counts_sum_to_rows(name):
    w = synth.workload(name)
    if w.routing == "supplied":
        inp = synth.make_inputs(w, only={"x"})
        idx = inp["topk_idx"]
    else:
        inp = synth.make_inputs(w, only={"x", "w_router", "bias"})
        idx, _ = oracle.topk_softmax(oracle.router_logits(inp["x"], inp["w_router"],
                                                          inp["bias"]), w.k)
    counts, offsets, perm, inv = layout(idx, w.E)
    assert counts.sum() == w.T * w.k == offsets[-1]


# ----------------------------------------------------------------------------
# gradients


def _exact_inputs(seed, T=4, H=8, E=4, k=2, I=8, Is=0, router=True):
    rng = np.random.default_rng(seed)
    inp = dict(x=rng.standard_normal((T, H)),
               w_gate=rng.standard_normal((E, H, I)) / np.sqrt(H),
               w_up=rng.standard_normal((E, H, I)) / np.sqrt(H),
               w_down=rng.standard_normal((E, I, H)) / np.sqrt(I),
               dout=rng.standard_normal((T, H)))
    if router:
        inp["w_router"] = rng.standard_normal((H, E))
        inp["bias"] = None
    else:
        inp["topk_idx"] = rng.integers(0, E, (T, k)).astype(np.int32)
        inp["topk_w"] = rng.dirichlet(np.ones(k), T)
    if Is:
        inp["ws_gate"] = rng.standard_normal((H, Is)) / np.sqrt(H)
        inp["ws_up"] = rng.standard_normal((H, Is)) / np.sqrt(H)
        inp["ws_down"] = rng.standard_normal((Is, H)) / np.sqrt(Is)
    return inp


def _loss(inp, k, routing):
    fw = oracle.forward(inp, k, exact=True, routing=routing)
    return float(np.sum(fw["out"] * inp["dout"]))


@pytest.mark.parametrize("router,Is", [(True, 0), (True, 8), (False, 8)])
def test_finite_differences(router, Is):
    k = 2
    inp = _exact_inputs(11, Is=Is, router=router)
    fw = oracle.forward(inp, k, exact=True)
    bw = oracle.backward(inp, fw)
    routing = None if router else (inp["topk_idx"], inp["topk_w"])
    grads = dict(x=bw["dx"], w_gate=bw["dWg"], w_up=bw["dWu"], w_down=bw["dWd"])
    if router:
        grads["w_router"] = bw["dWr"]
    else:
        grads["topk_w"] = bw["dw"]
    if Is:
        grads.update(ws_gate=bw["dWsg"], ws_up=bw["dWsu"], ws_down=bw["dWsd"])
    eps = 1e-6
    rng = np.random.default_rng(3)
    for name, g in grads.items():
        base = inp[name]
        flat = base.reshape(-1)
        picks = rng.choice(flat.size, min(flat.size, 24), replace=False)
        for p in picks:
            old = flat[p]
            flat[p] = old + eps
            r = None if routing is None else (routing[0], inp["topk_w"])
            lp = _loss(inp, k, r)
            flat[p] = old - eps
            r = None if routing is None else (routing[0], inp["topk_w"])
            lm = _loss(inp, k, r)
            flat[p] = old
            fd = (lp - lm) / (2 * eps)
            an = g.reshape(-1)[p]
            scale = max(1.0, np.abs(g).max())
            assert abs(fd - an) <= 1e-6 * scale, (name, p, fd, an)


def _torch_layer(inp, k, idx, router):
    """Independent formulation: per-slot gather of expert weights, index_add."""
    T64 = torch.float64
    P = {n: torch.tensor(v, dtype=T64, requires_grad=True) for n, v in inp.items()
         if n not in ("topk_idx", "dout", "bias") and v is not None}
    x = P["x"]
    if router:
        logits = x @ P["w_router"]
        sel = torch.gather(logits, 1, torch.tensor(idx, dtype=torch.int64))
        wts = torch.softmax(sel, dim=1)
    else:
        wts = P["topk_w"]
    out = torch.zeros_like(x)
    T = x.shape[0]
    for j in range(k):
        e = torch.tensor(idx[:, j], dtype=torch.int64)
        g = torch.einsum("th,thi->ti", x, P["w_gate"][e])
        u = torch.einsum("th,thi->ti", x, P["w_up"][e])
        y = torch.einsum("ti,tih->th", torch.nn.functional.silu(g) * u, P["w_down"][e])
        out = out.index_add(0, torch.arange(T), wts[:, j:j + 1] * y)
    if "ws_gate" in P:
        g = x @ P["ws_gate"]
        u = x @ P["ws_up"]
        out = out + (torch.nn.functional.silu(g) * u) @ P["ws_down"]
    (out * torch.tensor(inp["dout"])).sum().backward()
    return {n: p.grad.numpy() for n, p in P.items()}


@pytest.mark.parametrize("router,Is", [(True, 0), (False, 16), (True, 16)])
def test_torch_autograd_cross_check(router, Is):
    k = 3
    inp = _exact_inputs(21, T=16, H=32, E=5, k=k, I=16, Is=Is, router=router)
    fw = oracle.forward(inp, k, exact=True)
    bw = oracle.backward(inp, fw)
    tg = _torch_layer(inp, k, fw["idx"], router)
    pairs = dict(x="dx", w_gate="dWg", w_up="dWu", w_down="dWd")
    if router:
        pairs["w_router"] = "dWr"
    else:
        pairs["topk_w"] = "dw"
    if Is:
        pairs.update(ws_gate="dWsg", ws_up="dWsu", ws_down="dWsd")
    for tn, on in pairs.items():
        assert np.allclose(bw[on], tg[tn], rtol=1e-10, atol=1e-10), tn


def test_mx_mode_close_to_bf16_mode():
    w = small(T=64, H=128, I=64)
    inp = synth.make_inputs(w)
    a = oracle.forward(inp, w.k, mx=False)
    b = oracle.forward(inp, w.k, mx=True)
    assert np.array_equal(a["idx"], b["idx"])
    rel = np.abs(a["out"] - b["out"]).max() / np.abs(a["out"]).max()
    assert 0 < rel < 0.1
    ga = oracle.backward(inp, a)
    gb = oracle.backward(inp, b)
    for n in ("dx", "dWg", "dWu", "dWd"):
        rel = np.abs(ga[n] - gb[n]).max() / np.abs(ga[n]).max()
        assert 0 < rel < 0.15, n


@pytest.mark.parametrize("name", ["router", "supplied-dup", "router-mx"])
def test_sampled_weight_gradient_columns_match_full_backward(name):
    from oracle.layer import expert_weight_grad_columns
    w = CASES[name]
    inp = synth.make_inputs(w)
    fw = oracle.forward(inp, w.k, mx=w.mx)
    bw = oracle.backward(inp, fw)
    for e in range(w.E):
        cols = np.array([0, 5, w.I - 1])
        got = expert_weight_grad_columns(inp, w.k, w.mx, e, cols)
        assert np.array_equal(got["dWd"], bw["dWd"][e][cols, :])
        assert np.array_equal(got["dWg"], bw["dWg"][e][:, cols].T)
        assert np.array_equal(got["dWu"], bw["dWu"][e][:, cols].T)
        assert got["rows"] == fw["counts"][e]


def test_sampled_shared_expert_columns_match_full_backward():
    from oracle.layer import expert_weight_grad_columns
    w = CASES["shared"]
    inp = synth.make_inputs(w)
    fw = oracle.forward(inp, w.k)
    bw = oracle.backward(inp, fw)
    cols = np.array([1, 33, w.shared_I - 1])
    got = expert_weight_grad_columns(inp, w.k, False, 0, cols, shared=True)
    assert np.array_equal(got["dWd"], bw["dWsd"][cols, :])
    assert np.array_equal(got["dWg"], bw["dWsg"][:, cols].T)
    assert np.array_equal(got["dWu"], bw["dWsu"][:, cols].T)
