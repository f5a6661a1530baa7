"""GPU parity at the full benchmark sizes, in the launch configuration
bench.py times (one moe_layer_fwd + moe_layer_bwd through the C ABI).

The oracle cannot run these layers whole, so it evaluates samples one by one:
routing and layout in full (bit-exact), the dispatched rows (bit-exact: in
full for bf16; seeded rows of codes, scales and round trip for MXFP8), and
for seeded samples of tokens the output, dx and the routing weight gradient
(brute force per token), and for seeded columns of chosen experts the three
weight gradients.  Tolerance: max|gpu - oracle| / max|oracle| <= 2e-2 (bf16)
or 4e-2 (MXFP8) over each sampled tensor.

The router weight gradient is not sampled at the DeepSeek-shaped size (each
of its columns needs the full forward of every token routed to that expert);
it is checked in full on the mid-sized layers in test_gpu_parity.py and
test_gpu_mx.py.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import TOL_BF16, TOL_MX, Run, bf, check_rel, host, note, unblock_scales
from oracle.layer import TokenEvaluator, expert_weight_grad_columns
from oracle.numerics import bf16_bits, bf16_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    import os
    from mixture_experts_layer_offsets_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from mixture_experts_layer_offsets_amd import build
        build.build(verbose=False)


def _check_dispatch_mx(run, perm, k, H, rng, n_rows=512):
    R = perm.size
    rows = np.sort(rng.choice(R, min(n_rows, R), replace=False))
    codes, scales = oracle.dispatch(run.inp["x"], perm[rows], k, mx=True)
    rt = torch.as_tensor(rows, device="cuda")
    xq = run.saved("x_perm", torch.uint8, (R, H)).index_select(0, rt)
    xs = unblock_scales(host(run.saved("x_scale", torch.uint8, (R, H // 32))), R, H)[rows]
    xh = run.saved("x_hat", torch.int16, (R, H)).index_select(0, rt)
    assert np.array_equal(host(xq), codes)
    assert np.array_equal(xs, scales)
    ref_hat = oracle.mx.mx_dequantize(codes, scales, axis=1)
    assert np.array_equal(host(xh).view(np.uint16), bf16_bits(ref_hat))


def _check_fullsize(name, n_tok, experts, n_cols, seed=123, token_experts=False):
    """``experts``: the experts whose weight-gradient columns are sampled; with
    ``token_experts`` they are drawn from the sampled tokens' experts instead
    (their decoded weights are then shared with the token checks)."""
    w = synth.workload(name)
    tol = TOL_MX if w.mx else TOL_BF16
    note(f"full-size {name}: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I} shared={w.shared_I} "
         f"mx={w.mx}")
    inp = synth.make_inputs(w, threads=16)
    run = Run(w, inp)
    T, k, E, H, I = w.T, w.k, w.E, w.H, w.I
    R = T * k
    rng = np.random.default_rng(seed)

    # routing and layout, in full
    flips = np.zeros(T, bool)
    if w.routing == "router":
        L = oracle.router_logits(inp["x"], inp["w_router"], inp["bias"])
        Lg = host(run.saved("logits", torch.float32, (T, E)))
        check_rel("logits", Lg, L, 1e-4)
        ref_idx, ref_w = oracle.topk_softmax(L, k)
        idx = host(run.saved("topk_idx", torch.int32, (T, k)))
        flips = np.any(idx != ref_idx, axis=1)
        d = np.abs(Lg - L).max()
        for t in np.flatnonzero(flips):
            sel = L[t, idx[t]]
            assert sel.min() >= np.sort(L[t])[-k] - 2 * d
        assert flips.mean() < 0.001, flips.sum()
        wts = host(run.saved("topk_w", torch.float32, (T, k)))
        assert np.abs(wts[~flips] - ref_w[~flips]).max() <= 1e-5
    else:
        ref_idx = inp["topk_idx"]
    perm_g = host(run.saved("perm", torch.int32, (R,)))
    if not flips.any():
        counts, offsets, perm, inv = oracle.layout(ref_idx, E)
        assert np.array_equal(host(run.saved("counts", torch.int32, (E,))), counts)
        assert np.array_equal(host(run.saved("offsets", torch.int32, (E + 1,))), offsets)
        assert np.array_equal(perm_g, perm)
        assert np.array_equal(host(run.saved("inv_perm", torch.int32, (R,))), inv)
        if not w.mx:
            xp = host(run.saved("x_perm", torch.int16, (R, H))).view(np.uint16)
            assert np.array_equal(xp, oracle.dispatch(inp["x"], perm, k))
    if w.mx:   # rows as the GPU laid them out (valid even after a near-tie flip)
        _check_dispatch_mx(run, perm_g, k, H, rng)

    # sampled tokens: out, routed rows' Y, dx, dtopk_w
    ev = TokenEvaluator(inp, k, mx=w.mx)
    dout = bf16_to_f64(inp["dout"])
    ts = rng.choice(np.flatnonzero(~flips), n_tok, replace=False)
    idx_g = host(run.saved("topk_idx", torch.int32, (T, k)))
    if token_experts:
        pool = np.unique(idx_g[ts])
        experts = rng.choice(pool, min(len(experts), pool.size), replace=False)
    need = np.unique(np.concatenate([idx_g[ts].reshape(-1), np.asarray(experts, np.int64)]))
    note(f"  decoding weights of {need.size} experts")
    ev.W.prefetch(need, threads=16)
    inv_g = host(run.saved("inv_perm", torch.int32, (R,)))
    Yg = run.saved("y", torch.int16, (R, H))
    out_g, out_r, dx_g, dx_r, dw_g, dw_r, y_g, y_r = [], [], [], [], [], [], [], []
    for t in ts:
        tk = ev.token(int(t))
        out_g.append(bf(run.out[t])); out_r.append(tk["out"])
        for j, s in enumerate(tk["slots"]):
            y_g.append(bf(Yg[int(inv_g[t * k + j])])); y_r.append(s["Y"])
        tg = ev.token_grad(int(t), dout[t])
        dx_g.append(bf(run.grads["dx"][t])); dx_r.append(tg["dx"])
        dw_g.append(host(run.grads["dtopk_w"][t])); dw_r.append(tg["dw"])
    check_rel("out (sampled)", np.array(out_g), np.array(out_r), tol)
    check_rel("Y (sampled rows)", np.array(y_g), np.array(y_r), tol)
    check_rel("dx (sampled)", np.array(dx_g), np.array(dx_r), tol)
    check_rel("dtopk_w (sampled)", np.array(dw_g), np.array(dw_r), tol)

    # sampled weight-gradient columns
    g = run.grads
    for e in experts:
        cols = np.sort(rng.choice(I, n_cols, replace=False))
        ref = expert_weight_grad_columns(inp, k, w.mx, int(e), cols, weights=ev.W[int(e)])
        ct = torch.as_tensor(cols, device="cuda")
        check_rel(f"dW_down[{e}]", host(g["dw_down"][e].index_select(0, ct)), ref["dWd"], tol)
        check_rel(f"dW_gate[{e}]", host(g["dw_gate"][e].index_select(1, ct)).T, ref["dWg"], tol)
        check_rel(f"dW_up[{e}]", host(g["dw_up"][e].index_select(1, ct)).T, ref["dWu"], tol)
    if w.shared_I:
        Is = w.shared_I
        cols = np.sort(rng.choice(Is, n_cols, replace=False))
        ref = expert_weight_grad_columns(inp, k, w.mx, 0, cols, shared=True, weights=ev.WS)
        ct = torch.as_tensor(cols, device="cuda")
        dws = g["dws"]
        dWsg = dws[:H * Is].view(H, Is)
        dWsu = dws[H * Is:2 * H * Is].view(H, Is)
        dWsd = dws[2 * H * Is:].view(Is, H)
        check_rel("dWs_down", host(dWsd.index_select(0, ct)), ref["dWd"], tol)
        check_rel("dWs_gate", host(dWsg.index_select(1, ct)).T, ref["dWg"], tol)
        check_rel("dWs_up", host(dWsu.index_select(1, ct)).T, ref["dWu"], tol)
    return run


def test_kimi_bf16_full_size():
    w = synth.workload("kimi-bf16")
    _check_fullsize("kimi-bf16", n_tok=12, experts=range(w.E), n_cols=4)


def test_dsv3_bf16_full_size():
    rng = np.random.default_rng(7)
    experts = rng.choice(256, 4, replace=False)
    _check_fullsize("dsv3-bf16", n_tok=8, experts=experts, n_cols=3)


def test_kimi_mx_full_size():
    w = synth.workload("kimi-mx")
    _check_fullsize("kimi-mx", n_tok=12, experts=range(w.E), n_cols=4)


def test_dsv3_mx_full_size():
    # MX weights take seconds per expert to decode on the host: the sampled
    # tokens' experts are decoded once and reused for the weight gradients
    _check_fullsize("dsv3-mx", n_tok=3, experts=range(2), n_cols=3, token_experts=True)
