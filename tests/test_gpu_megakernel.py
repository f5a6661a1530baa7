"""The persistent pipelined forward (moe_sched.schedule = 1) against the
staged forward and the oracle.

The persistent kernel runs the same tile, dispatch and combine arithmetic as
the staged kernels (only the order of tiles and minibatches differs, and each
output element is still one fixed-order sum), so every output and every
saved tensor must be bit-identical to the staged forward's, for any
minibatch size, window (ring slots) and CU split; the backward that reads
either context then gives identical gradients.  One case is also compared
with the oracle directly, and the watchdog is exercised by giving the waits a
budget of one microsecond (forced from the host: every kernel still exits).
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_offsets_amd as m
import oracle
import synth
from gpu_util import (TOL_BF16, bf, check_rel, check_routing_layout, dev, host, note,
                      oracle_forward, shape_of)

# The persistent forward is switched off in libmoe (moe_layer_fwd refuses
# use_megakernel with MOE_ERR_UNSUPPORTED): its first two GPU runs never
# finished.  The host model of its schedule (tests/test_mk_model.py) shows
# the schedule itself cannot deadlock or outlive its watchdog, so the cause
# lies outside it and is not shown.  These tests stay, skipped.
pytestmark = [pytest.mark.gpu,
              pytest.mark.skip(reason="persistent forward switched off: its GPU runs did not "
                                      "finish and the cause is not shown (the host model of "
                                      "its schedule finishes)")]


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


class Pair:
    """One set of device inputs, run through the staged and the persistent
    forward (separate layers, so separate saved contexts)."""

    def __init__(self, w, inp=None):
        self.w = w
        self.inp = inp if inp is not None else synth.make_inputs(w)
        inp = self.inp
        self.shape = shape_of(w, m.MOE_MXFP8 if w.mx else m.MOE_BF16)
        self.d = {k: dev(v) for k, v in inp.items() if v is not None and k != "hot"}
        self.layers = []
        for _ in range(2):
            L = m.MoeLayer(self.shape)
            L.prepare(self.d["w_gate"], self.d["w_up"], self.d["w_down"], self.d.get("ws_gate"),
                      self.d.get("ws_up"), self.d.get("ws_down"))
            self.layers.append(L)

    def forward(self, i, sched=None):
        L = self.layers[i]
        out = L.forward(self.d["x"], w_router=self.d.get("w_router"), bias=self.d.get("bias"),
                        topk_idx=self.d.get("topk_idx"), topk_w=self.d.get("topk_w"),
                        sched=sched)
        torch.cuda.synchronize()
        return out

    def backward(self, i):
        g = self.layers[i].backward(self.d["dout"], self.d["x"],
                                    w_router=self.d.get("w_router"))
        torch.cuda.synchronize()
        return g


def mk_sched(**kw):
    s = m.MoeSched()
    s.schedule = 1
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def _assert_same_forward(pair, out_s, out_m):
    assert np.array_equal(host(out_m), host(out_s)), "out differs"
    names = SAVED_MX if pair.w.mx else SAVED_BF16
    for name, dt, code in names:
        a = host(pair.layers[0].saved_tensor(name, dt, _dims(pair.w, code)))
        b = host(pair.layers[1].saved_tensor(name, dt, _dims(pair.w, code)))
        assert np.array_equal(a, b), f"saved {name} differs"
    if pair.w.shared_I:
        T, H = pair.w.T, pair.w.H
        a = host(pair.layers[0].saved_tensor("y_shared", torch.int16, (T, H)))
        b = host(pair.layers[1].saved_tensor("y_shared", torch.int16, (T, H)))
        assert np.array_equal(a, b), "saved y_shared differs"


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
}

SCHEDS = [dict(), dict(minibatch_rows=256, ring_slots=1, comm_cus=1),
          dict(minibatch_rows=1000, ring_slots=2, comm_cus=64),
          dict(minibatch_rows=300, ring_slots=8, comm_cus=8)]


@pytest.mark.parametrize("name", list(CASES))
def test_megakernel_matches_staged(name):
    w = CASES[name]
    note(f"megakernel {name}: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I} shared={w.shared_I} "
         f"mx={w.mx}")
    pair = Pair(w)
    out_s = host(pair.forward(0)).copy()
    g_s = {k: host(v).copy() for k, v in pair.backward(0).items()}
    for sk in SCHEDS:
        note(f"  sched {sk}")
        out_m = pair.forward(1, mk_sched(**sk))
        assert pair.layers[1].status() == m.MOE_OK
        _assert_same_forward(pair, torch.from_numpy(out_s), out_m)
    g_m = pair.backward(1)
    for k, v in g_s.items():
        assert np.array_equal(host(g_m[k]), v), f"gradient {k} differs"


def test_megakernel_against_oracle():
    w = CASES["shared-router"]
    note("megakernel vs oracle: shared-router")
    pair = Pair(w)
    out = pair.forward(1, mk_sched(minibatch_rows=512, ring_slots=2, comm_cus=4))
    L = host(pair.layers[1].saved_tensor("logits", torch.float32, (w.T, w.E)))
    fw = oracle_forward(pair.inp, w, L)
    check_routing_layout(pair.layers[1], w, fw)
    check_rel("out", bf(out), fw["out"], TOL_BF16)


def test_megakernel_watchdog_reports_timeout():
    """A one-microsecond budget makes waits give up: the kernel still finishes and the
    status word says MOE_ERR_DEVICE_TIMEOUT; the next call is clean."""
    w = CASES["supplied-dup"]
    note("megakernel watchdog: one microsecond per wait")
    pair = Pair(w)
    pair.forward(1, mk_sched(minibatch_rows=256, ring_slots=1, comm_cus=1, watchdog_us=1))
    assert pair.layers[1].status() == m.MOE_ERR_DEVICE_TIMEOUT
    out_s = pair.forward(0)
    out_m = pair.forward(1, mk_sched())
    assert pair.layers[1].status() == m.MOE_OK
    assert np.array_equal(host(out_m), host(out_s))


@pytest.mark.parametrize("name,mb", [("kimi-bf16", 2368), ("kimi-mx", 2368)])
def test_megakernel_full_size(name, mb):
    w = synth.workload(name)
    note(f"megakernel full size {name}: minibatch {mb}")
    pair = Pair(w, synth.make_inputs(w, threads=16))
    out_s = pair.forward(0)
    out_m = pair.forward(1, mk_sched(minibatch_rows=mb))
    assert pair.layers[1].status() == m.MOE_OK
    _assert_same_forward(pair, out_s, out_m)
