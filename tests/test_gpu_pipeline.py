"""The minibatch-pipelined schedule (moe_sched.schedule = MOE_SCHED_PIPELINED)
against the staged schedule and the oracle.

The pipelined layer runs the staged path's arithmetic on minibatches of
sorted rows: each GEMM output element is the same fixed-order sum over the
contraction (only which tiles run when differs), dispatch and combine do the
same per-row / per-token work, the row-driven reverse-combine reproduces the
token-driven one's reduction order, and the weight gradients run over all
rows as in the staged path.  So every output, every saved tensor and every
gradient must be bit-identical to the staged layer's, for any minibatch size,
window (ring slots) and CU split.  One case of each dtype is also compared
with the oracle directly.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_offsets_amd as m
import oracle
import synth
from gpu_util import TOL_BF16, TOL_MX, bf, check_rel, dev, host, note, shape_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    from mixture_experts_layer_offsets_amd import _lib
    if not __import__("os").path.exists(_lib.LIB_PATH):
        from mixture_experts_layer_offsets_amd import build
        build.build(verbose=False)
    m.load()


SAVED_BF16 = [("x_perm", torch.int16, "RH"), ("gu", torch.int16, "R2I"), ("act", torch.int16, "RI"),
              ("y", torch.int16, "RH")]
SAVED_MX = [("x_perm", torch.uint8, "RH"), ("x_scale", torch.uint8, "RH32"),
            ("x_hat", torch.int16, "RH"), ("gu", torch.int16, "R2I"), ("act", torch.int16, "RI"),
            ("act_q", torch.uint8, "RI"), ("act_scale", torch.uint8, "RI32"),
            ("y", torch.int16, "RH")]


def _dims(w, code):
    R, H, I = w.T * w.k, w.H, w.I
    return {"RH": (R, H), "R2I": (R, 2 * I), "RI": (R, I), "RH32": (R, H // 32),
            "RI32": (R, I // 32)}[code]


def sched(**kw):
    s = m.MoeSched()
    s.schedule = m.MOE_SCHED_PIPELINED
    for k, v in kw.items():
        setattr(s, k, v)
    return s


class Pair:
    """One set of device inputs, run through the staged (layer 0) and the
    pipelined (layer 1) schedule, each with its own saved context."""

    def __init__(self, w, inp=None):
        self.w = w
        self.inp = inp if inp is not None else synth.make_inputs(w)
        self.shape = shape_of(w, m.MOE_MXFP8 if w.mx else m.MOE_BF16)
        self.d = {k: dev(v) for k, v in self.inp.items() if v is not None and k != "hot"}
        self.layers = []
        for _ in range(2):
            L = m.MoeLayer(self.shape)
            L.prepare(self.d["w_gate"], self.d["w_up"], self.d["w_down"], self.d.get("ws_gate"),
                      self.d.get("ws_up"), self.d.get("ws_down"))
            self.layers.append(L)

    def forward(self, i, sc=None):
        out = self.layers[i].forward(self.d["x"], w_router=self.d.get("w_router"),
                                     bias=self.d.get("bias"), topk_idx=self.d.get("topk_idx"),
                                     topk_w=self.d.get("topk_w"), sched=sc)
        torch.cuda.synchronize()
        return out

    def backward(self, i, sc=None):
        g = self.layers[i].backward(self.d["dout"], self.d["x"],
                                    w_router=self.d.get("w_router"), sched=sc)
        torch.cuda.synchronize()
        return g


def _assert_same_forward(pair, out_s, out_p):
    assert np.array_equal(host(out_p), out_s), "out differs"
    for name, dt, code in (SAVED_MX if pair.w.mx else SAVED_BF16):
        a = host(pair.layers[0].saved_tensor(name, dt, _dims(pair.w, code)))
        b = host(pair.layers[1].saved_tensor(name, dt, _dims(pair.w, code)))
        assert np.array_equal(a, b), f"saved {name} differs"
    if pair.w.shared_I:
        T, H = pair.w.T, pair.w.H
        a = host(pair.layers[0].saved_tensor("y_shared", torch.int16, (T, H)))
        b = host(pair.layers[1].saved_tensor("y_shared", torch.int16, (T, H)))
        assert np.array_equal(a, b), "saved y_shared differs"


def _assert_same_grads(g_s, g_p):
    assert set(g_s) == set(g_p)
    for k in g_s:
        assert np.array_equal(host(g_p[k]), g_s[k]), f"gradient {k} differs"


CASES = {
    "tiny-router": synth.workload("tiny"),
    "shared-router": synth.custom(T=512, H=512, E=16, k=4, I=192, shared_I=256,
                                  routing="router", router_std=1 / np.sqrt(512),
                                  hot_experts=2, hot_bias=1.0, seed=3),
    "supplied-dup": synth.custom(T=700, H=768, E=6, k=8, I=320, zipf_s=1.0,
                                 routing="supplied", seed=7),
    "ragged": synth.custom(T=777, H=320, E=5, k=3, I=192, routing="supplied", seed=7),
    "mx-shared-router": synth.custom(T=512, H=512, E=16, k=4, I=256, shared_I=256,
                                     routing="router", router_std=1 / np.sqrt(512),
                                     hot_experts=2, hot_bias=1.0, mx=True, seed=3),
    "mx-supplied": synth.custom(T=700, H=768, E=6, k=8, I=384, zipf_s=1.2,
                                routing="supplied", mx=True, seed=7),
    # top-k above 8: the 16-slot token-list, combine and reverse kernels
    "k16-router": synth.custom(T=300, H=256, E=32, k=16, I=128, routing="router",
                               router_std=1 / 16, seed=11),
    "mx-k12": synth.custom(T=300, H=384, E=14, k=12, I=256, zipf_s=1.0, routing="supplied",
                           mx=True, seed=13),
    # 1024 experts, most minibatches spanning many of them
    "E1024-router": synth.custom(T=512, H=256, E=1024, k=8, I=64, routing="router",
                                 router_std=1 / 16, seed=21),
}

# default; the smallest minibatch with a one-minibatch window; a minibatch
# that is not a multiple of the 256-row tile; a CU split; a window larger
# than the minibatch count
SCHEDS = [dict(), dict(minibatch_rows=256, ring_slots=1),
          dict(minibatch_rows=1000, ring_slots=2, comm_cus=64),
          dict(minibatch_rows=300, ring_slots=8, comm_cus=8)]


@pytest.mark.parametrize("name", list(CASES))
def test_pipelined_matches_staged(name):
    w = CASES[name]
    note(f"pipelined {name}: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I} shared={w.shared_I} "
         f"mx={w.mx}")
    pair = Pair(w)
    out_s = host(pair.forward(0)).copy()
    g_s = {k: host(v).copy() for k, v in pair.backward(0).items()}
    for sk in SCHEDS:
        note(f"  sched {sk}")
        out_p = pair.forward(1, sched(**sk))
        assert pair.layers[1].status() == m.MOE_OK
        _assert_same_forward(pair, out_s, out_p)
        g_p = pair.backward(1, sched(**sk))
        _assert_same_grads(g_s, g_p)


@pytest.mark.parametrize("name", ["supplied-dup", "mx-supplied"])
def test_pipelined_matches_oracle(name):
    """The pipelined layer against the oracle, forward and backward (supplied
    routing, so the layout is the oracle's exactly)."""
    w = CASES[name]
    note(f"pipelined vs oracle {name}")
    pair = Pair(w)
    sc = sched(minibatch_rows=512, ring_slots=2)
    out = pair.forward(1, sc)
    g = pair.backward(1, sc)
    fw = oracle.forward(pair.inp, w.k, mx=w.mx)
    bw = oracle.backward(pair.inp, fw)
    tol = TOL_MX if w.mx else TOL_BF16
    check_rel("out", bf(out), fw["out"], tol)
    check_rel("dx", bf(g["dx"]), bw["dx"], tol)
    check_rel("dW_gate", host(g["dw_gate"]), bw["dWg"], tol)
    check_rel("dW_up", host(g["dw_up"]), bw["dWu"], tol)
    check_rel("dW_down", host(g["dw_down"]), bw["dWd"], tol)
    check_rel("dtopk_w", host(g["dtopk_w"]), bw["dw"], tol)


def test_pipelined_kimi_shape_matches_staged():
    """The Kimi-shaped expert share (16,384 routed rows, hidden 7168, six
    experts of 2048, Zipf s=1.0) with the default minibatch and a CU split:
    bit-identical to the staged layer."""
    w = synth.workload("kimi-bf16")
    note("pipelined kimi-bf16 full size")
    pair = Pair(w)
    out_s = host(pair.forward(0)).copy()
    g_s = {k: host(v).copy() for k, v in pair.backward(0).items()}
    for sk in (dict(), dict(minibatch_rows=2368, comm_cus=16)):
        note(f"  sched {sk}")
        out_p = pair.forward(1, sched(**sk))
        assert np.array_equal(host(out_p), out_s), "out differs"
        _assert_same_grads(g_s, pair.backward(1, sched(**sk)))


def test_pipelined_rejects_bad_sched():
    w = CASES["tiny-router"]
    pair = Pair(w)
    with pytest.raises(RuntimeError):
        pair.forward(1, sched(comm_cus=-1))
    s = sched()
    s.schedule = 7
    with pytest.raises(RuntimeError):
        pair.forward(1, s)
