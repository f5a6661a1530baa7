"""MXFP8 weight gradients (moe_sched.mx_wgrad = 1) against the oracle.

With the option the two weight-gradient GEMMs take MX operands quantised
down the rows (their contraction axis): E8M0 blocks of 32 rows of one
column starting at each expert's first row, the last block zero-padded
(the oracle's backward(..., mx_wgrad=True)).

What is checked:
- the data gradients, dx, dw and the router gradient are untouched
  (bit-identical to the default MX backward);
- parity: the whole layer against the oracle's whole forward and backward
  with the MX weight-gradient recipe, at the MXFP8 tolerance (4e-2 of each
  tensor's maximum); the oracle routes from the GPU's fp32 logits through
  its own top-k and layout (the selection is defined given the logits),
  nothing else of the GPU's enters it;
- a consistency check of the step on its own: the GPU's weight gradients
  equal the row-quantised product of the GPU's own bf16 operands (dy and dh
  from the workspace, act and the dispatched rows' round trip from the
  forward context) up to the matrix instruction's summation error, 1e-3 of
  the maximum -- a single operand code that differed (one E4M3 ulp, 1/8 of
  a product term) would move an output by ~7e-3 of the maximum at these
  row counts;
- staged and pipelined schedules bit-identical.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_offsets_amd as m
import oracle
import synth
from gpu_util import (TOL_MX, check_rel, check_routing_layout, dev, host, note,
                      oracle_forward, shape_of)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    from mixture_experts_layer_offsets_amd import _lib
    if not __import__("os").path.exists(_lib.LIB_PATH):
        from mixture_experts_layer_offsets_amd import build
        build.build(verbose=False)
    m.load()


CASES = {
    # expert segments of every length mod 32 and mod 128, six experts
    "mx-supplied": synth.custom(T=700, H=768, E=6, k=8, I=384, zipf_s=1.2,
                                routing="supplied", mx=True, seed=7),
    # a shared expert (its own weight gradients in MX too) and router routing
    "mx-shared-router": synth.custom(T=512, H=512, E=16, k=4, I=256, shared_I=256,
                                     routing="router", router_std=1 / np.sqrt(512),
                                     hot_experts=2, hot_bias=1.0, mx=True, seed=3),
    # more experts than rows need: some experts get no rows (zero gradients)
    "mx-sparse": synth.custom(T=40, H=256, E=24, k=2, I=128, zipf_s=2.0, routing="supplied",
                              mx=True, seed=11),
}


def sched(mode, **kw):
    s = m.MoeSched()
    s.schedule = mode
    s.mx_wgrad = 1
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def logits_of_layer(layer, w):
    if w.routing != "router":
        return None
    return host(layer.saved_tensor("logits", torch.float32, (w.T, w.E)))


def _run(w, inp, sc_f, sc_b):
    layer = m.MoeLayer(shape_of(w, m.MOE_MXFP8))
    d = {k: dev(v) for k, v in inp.items() if v is not None and k != "hot"}
    layer.prepare(d["w_gate"], d["w_up"], d["w_down"], d.get("ws_gate"), d.get("ws_up"),
                  d.get("ws_down"))
    layer.forward(d["x"], w_router=d.get("w_router"), bias=d.get("bias"),
                  topk_idx=d.get("topk_idx"), topk_w=d.get("topk_w"), sched=sc_f)
    g = layer.backward(d["dout"], d["x"], w_router=d.get("w_router"), sched=sc_b)
    torch.cuda.synchronize()
    return layer, {k: host(v).copy() for k, v in g.items()}


@pytest.mark.parametrize("name", list(CASES))
def test_mx_wgrad_matches_oracle(name):
    w = CASES[name]
    note(f"mx wgrad {name}: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I} shared={w.shared_I}")
    inp = synth.make_inputs(w)
    _, g0 = _run(w, inp, None, None)                                   # bf16 weight gradients
    layer, g1 = _run(w, inp, None, sched(m.MOE_SCHED_STAGED))           # MX weight gradients
    for k in ("dx", "dtopk_w") + (("dw_router",) if w.routing == "router" else ()):
        assert np.array_equal(g0[k], g1[k]), f"{k} changed"
    fw = oracle_forward(inp, w, logits_of_layer(layer, w))
    check_routing_layout(layer, w, fw)
    bw = oracle.backward(inp, fw, mx_wgrad=True)
    # the step on the GPU's own operands: accumulation order only
    from oracle.mx import mx_rows_roundtrip
    from oracle.numerics import bf16_to_f64
    R, H, I = w.T * w.k, w.H, w.I

    def rd(t):
        return bf16_to_f64(host(t).view(np.uint16))
    dy = rd(layer.work_tensor("dy", torch.int16, (R, H)))
    dh = rd(layer.work_tensor("dh", torch.int16, (R, 2 * I)))
    xh = rd(layer.saved_tensor("x_hat", torch.int16, (R, H)))
    ah = rd(layer.saved_tensor("act", torch.int16, (R, I)))
    blk = dh.reshape(R, I // 32, 2, 32)
    dg, du = blk[:, :, 0, :].reshape(R, I), blk[:, :, 1, :].reshape(R, I)
    off = host(layer.saved_tensor("offsets", torch.int32, (w.E + 1,)))
    # Tolerance 1e-3 of the tensor maximum.  The scaled fp8 matrix
    # instruction does not sum like fp32: measured on MI355X, its outputs
    # differ from the exact sum of the same quantised operands by up to ~4e-4
    # relative (~2e-4 of the tensor maximum), independent of the contraction
    # length, so a gamma_K bound does not hold.  A single operand code that
    # differed from the oracle's (one E4M3 ulp, 1/8 of a product term) would
    # move an output by ~7e-3 of the maximum at these row counts, far above.
    ref = {"dw_gate": np.zeros((w.E, H, I)), "dw_up": np.zeros((w.E, H, I)),
           "dw_down": np.zeros((w.E, I, H))}
    for e in range(w.E):
        rs = slice(int(off[e]), int(off[e + 1]))
        if rs.stop == rs.start:
            continue
        qx = mx_rows_roundtrip(xh[rs])
        ref["dw_gate"][e] = qx.T @ mx_rows_roundtrip(dg[rs])
        ref["dw_up"][e] = qx.T @ mx_rows_roundtrip(du[rs])
        ref["dw_down"][e] = mx_rows_roundtrip(ah[rs]).T @ mx_rows_roundtrip(dy[rs])
    for key, v in ref.items():
        check_rel(key + " (the step on the GPU's own operands)", g1[key], v, 1e-3)
    # parity of the whole backward against the oracle's
    tol = TOL_MX
    check_rel("dW_gate", g1["dw_gate"], bw["dWg"], tol)
    check_rel("dW_up", g1["dw_up"], bw["dWu"], tol)
    check_rel("dW_down", g1["dw_down"], bw["dWd"], tol)
    check_rel("dx", bf16_to_f64(g1["dx"].view(np.uint16)), bw["dx"], tol)
    check_rel("dtopk_w", g1["dtopk_w"], bw["dw"], tol)
    if w.shared_I:
        Is = w.shared_I
        dws = g1["dws"]
        check_rel("dWs_gate", dws[:H * Is].reshape(H, Is), bw["dWsg"], tol)
        check_rel("dWs_up", dws[H * Is:2 * H * Is].reshape(H, Is), bw["dWsu"], tol)
        check_rel("dWs_down", dws[2 * H * Is:].reshape(Is, H), bw["dWsd"], tol)
    counts = np.bincount(np.asarray(fw["idx"]).reshape(-1), minlength=w.E)
    for e in np.flatnonzero(counts == 0):
        assert not g1["dw_gate"][e].any() and not g1["dw_down"][e].any()


@pytest.mark.parametrize("name", ["mx-supplied", "mx-shared-router"])
def test_mx_wgrad_pipelined_matches_staged(name):
    w = CASES[name]
    inp = synth.make_inputs(w)
    _, gs = _run(w, inp, None, sched(m.MOE_SCHED_STAGED))
    for kw in (dict(), dict(minibatch_rows=512)):
        note(f"  pipelined {kw}")
        _, gp = _run(w, inp, sched(m.MOE_SCHED_PIPELINED, **kw),
                     sched(m.MOE_SCHED_PIPELINED, **kw))
        for k in gs:
            assert np.array_equal(gp[k], gs[k]), f"{k} differs"


def test_mx_wgrad_kimi_shape_pipelined_matches_staged():
    """The Kimi-shaped MXFP8 share: staged and pipelined MX weight
    gradients bit-identical, and within the MX tolerance of the bf16 ones."""
    w = synth.workload("kimi-mx")
    note("mx wgrad kimi-mx full size")
    inp = synth.make_inputs(w)
    _, g0 = _run(w, inp, None, None)
    _, gs = _run(w, inp, None, sched(m.MOE_SCHED_STAGED))
    _, gp = _run(w, inp, sched(m.MOE_SCHED_PIPELINED), sched(m.MOE_SCHED_PIPELINED))
    for k in gs:
        assert np.array_equal(gp[k], gs[k]), f"{k} differs"
    for k in ("dw_gate", "dw_up", "dw_down"):
        check_rel(k + " (MX vs bf16 weight gradients)", gs[k], g0[k], TOL_MX)
