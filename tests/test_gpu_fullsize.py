"""GPU parity at the full benchmark sizes, through the C ABI.

Kimi-shaped expert share (bf16 and MXFP8: 2048 tokens x top-8 = 16,384
routed rows, hidden 7168, six experts of intermediate 2048): one forward and
backward in the pipelined schedule bench.py times, against the whole oracle
forward and backward; every saved tensor, output and gradient is compared in
full (routing and layout bit-exact, dispatched rows bit-exact -- codes and
scales for MXFP8 --, the rest within 2e-2 (bf16) or 4e-2 (MXFP8) of each
tensor's maximum).

DeepSeek-V3-shaped layer (8192 tokens, 256 routed experts + one shared,
top-8, hidden 7168, intermediate 2048): the oracle cannot hold the whole
layer (45 GB of weight gradients in fp64 twice over), so
- routing and layout are checked in full, bit-exact, the oracle's top-k and
  layout running on the GPU's fp32 logits;
- the dispatched rows in full (bf16 copies, or MXFP8 codes, scales and round
  trips, bit-exact);
- a seeded sample of 256 tokens goes through the oracle's forward and
  backward (every per-token result -- out, dx, dtopk_w, the tokens' rows of
  Y and a, the shared expert's y -- is independent of the other tokens);
- 16 experts (8 of the hot ones, 8 others) have 16 seeded columns of each
  weight gradient recomputed over all their rows, as does the shared expert.
dW_router is not checked at this size (each of its columns needs every token
routed to that expert, i.e. most of the layer); the mid-sized router layers
check it in full.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_offsets_amd as m
import oracle
import synth
from gpu_util import (TOL_BF16, TOL_MX, Run, bf, check_layer, check_layer_mx, check_rel,
                      check_routing_layout, host, logits_of, note, oracle_forward,
                      unblock_scales)
from oracle.layer import _LazyWeights, _each, expert_weight_grad_columns
from oracle.mx import mx_dequantize, mx_quantize
from oracle.numerics import bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    import os
    from mixture_experts_layer_offsets_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from mixture_experts_layer_offsets_amd import build
        build.build(verbose=False)


def _pipelined():
    s = m.MoeSched()
    s.schedule = m.MOE_SCHED_PIPELINED
    return s


@pytest.mark.parametrize("name", ["kimi-bf16", "kimi-mx"])
def test_kimi_full_size_in_full(name):
    w = synth.workload(name)
    note(f"full-size {name}: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I} mx={w.mx}, "
         f"pipelined schedule")
    inp = synth.make_inputs(w, threads=16)
    run = Run(w, inp, sched=_pipelined())
    note("  oracle forward + backward over the whole layer")
    fw = oracle_forward(inp, w, logits_of(run))
    bw = oracle.backward(inp, fw)
    note("  comparing")
    (check_layer_mx if w.mx else check_layer)(run, fw, bw)


def _check_dsv3(name, n_tok=256, n_hot=8, n_cold=8, n_cols=16, seed=123):
    w = synth.workload(name)
    tol = TOL_MX if w.mx else TOL_BF16
    note(f"full-size {name}: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I} shared={w.shared_I} "
         f"mx={w.mx}")
    inp = synth.make_inputs(w, threads=16)
    run = Run(w, inp)
    T, k, E, H, I = w.T, w.k, w.E, w.H, w.I
    R = T * k
    rng = np.random.default_rng(seed)

    # routing and layout in full, from the GPU's fp32 logits
    Lg = logits_of(run)
    own = oracle.router_logits(inp["x"], inp["w_router"], inp["bias"])
    check_rel("logits", Lg, own, 1e-4)
    idx, wts = oracle.topk_softmax(Lg, k)
    counts, offsets, perm, inv = oracle.layout(idx, E)
    full = dict(idx=idx, w=wts, counts=counts, offsets=offsets, perm=perm, inv=inv)
    check_routing_layout(run.layer, w, full)
    own_idx, _ = oracle.topk_softmax(own, k)
    note(f"  {int(np.any(own_idx != idx, axis=1).sum())} of {T} tokens would route "
         f"differently from the oracle's own fp64 logits (near-ties)")

    # the dispatched rows in full: a row is a copy (or the per-row MX
    # conversion) of its token, so the tokens are converted once and gathered
    src = perm.astype(np.int64) // k
    if not w.mx:
        xp = host(run.saved("x_perm", torch.int16, (R, H))).view(np.uint16)
        assert np.array_equal(xp, inp["x"][src])
    else:
        codes, scales = mx_quantize(oracle.numerics.bf16_to_f64(inp["x"]), axis=1)
        assert np.array_equal(host(run.saved("x_perm", torch.uint8, (R, H))), codes[src])
        xs = unblock_scales(host(run.saved("x_scale", torch.uint8, (R, H // 32))), R, H)
        assert np.array_equal(xs, scales[src])
        xh = host(run.saved("x_hat", torch.int16, (R, H))).view(np.uint16)
        assert np.array_equal(xh, bf16_bits(mx_dequantize(codes, scales, axis=1))[src])

    # a sample of tokens through the oracle's forward and backward
    S = np.sort(rng.choice(T, n_tok, replace=False))
    sub = dict(inp, x=inp["x"][S], dout=inp["dout"][S])
    note(f"  oracle forward + backward over {n_tok} sampled tokens")
    fw = oracle.forward(sub, k, mx=w.mx, logits=Lg[S])
    bw = oracle.backward(sub, fw)
    assert np.array_equal(fw["idx"], idx[S])
    g = run.grads
    St = torch.as_tensor(S, device="cuda")
    check_rel("out (sampled tokens)", bf(run.out.index_select(0, St)), fw["out"], tol)
    check_rel("dx (sampled tokens)", bf(g["dx"].index_select(0, St)), bw["dx"], tol)
    check_rel("dtopk_w (sampled tokens)", host(g["dtopk_w"].index_select(0, St)), bw["dw"], tol)
    f_full = (S[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    rows_gpu = torch.as_tensor(inv[f_full], device="cuda")
    rows_ora = fw["inv"]                     # sample row of (i, j) for f_sub = i*k + j
    check_rel("Y (sampled rows)", bf(run.saved("y", torch.int16, (R, H)).index_select(0, rows_gpu)),
              fw["Y"][rows_ora], tol)
    check_rel("act (sampled rows)",
              bf(run.saved("act", torch.int16, (R, I)).index_select(0, rows_gpu)),
              fw["ahat"][rows_ora], tol)
    if w.shared_I:
        check_rel("y_shared (sampled tokens)",
                  bf(run.saved("y_shared", torch.int16, (T, H)).index_select(0, St)),
                  fw["shared"]["y"], tol)

    # weight gradients: 16 experts' seeded columns, over all their rows
    hot = np.asarray(inp["hot"])
    cold = np.setdiff1d(np.arange(E), hot)
    experts = np.concatenate([rng.choice(hot, n_hot, replace=False),
                              rng.choice(cold, n_cold, replace=False)])
    cols = {int(e): np.sort(rng.choice(I, n_cols, replace=False)) for e in experts}
    note(f"  weight-gradient columns of experts {experts.tolist()} and the shared expert")
    lazy = _LazyWeights(inp, w.mx, keep=len(experts))
    refs = {}

    def one(e):
        refs[e] = expert_weight_grad_columns(inp, k, w.mx, e, cols[e], weights=lazy[e],
                                             logits=Lg)
    _each(one, list(cols))
    for e, c in cols.items():
        ref = refs[e]
        assert ref["rows"] == counts[e]
        ct = torch.as_tensor(c, device="cuda")
        check_rel(f"dW_down[{e}]", host(g["dw_down"][e].index_select(0, ct)), ref["dWd"], tol)
        check_rel(f"dW_gate[{e}]", host(g["dw_gate"][e].index_select(1, ct)).T, ref["dWg"], tol)
        check_rel(f"dW_up[{e}]", host(g["dw_up"][e].index_select(1, ct)).T, ref["dWu"], tol)
    if w.shared_I:
        Is = w.shared_I
        c = np.sort(rng.choice(Is, n_cols, replace=False))
        ref = expert_weight_grad_columns(inp, k, w.mx, 0, c, shared=True)
        ct = torch.as_tensor(c, device="cuda")
        dws = g["dws"]
        dWsg = dws[:H * Is].view(H, Is)
        dWsu = dws[H * Is:2 * H * Is].view(H, Is)
        dWsd = dws[2 * H * Is:].view(Is, H)
        check_rel("dWs_down", host(dWsd.index_select(0, ct)), ref["dWd"], tol)
        check_rel("dWs_gate", host(dWsg.index_select(1, ct)).T, ref["dWg"], tol)
        check_rel("dWs_up", host(dWsu.index_select(1, ct)).T, ref["dWu"], tol)


def test_dsv3_bf16_full_size():
    _check_dsv3("dsv3-bf16")


def test_dsv3_mx_full_size():
    _check_dsv3("dsv3-mx")
