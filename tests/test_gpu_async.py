"""No host synchronisation in the layer calls.

The pages keep the CPU out of the per-step loop (no host-side sizing, no
host wait per minibatch).  Here a bounded sleep kernel (torch.cuda._sleep)
occupies the caller's stream, the layer's forward and backward are then
enqueued behind it, and the calls must return while that stream is still
busy -- they enqueue and do not wait.  The results must still equal those of
an undelayed run: the layer's work is ordered after the sleep on the stream,
including the pipelined schedule's forks onto the library's own streams.
"""
import time

import numpy as np
import pytest
import torch

import mixture_experts_layer_offsets_amd as m
import synth
from gpu_util import dev, host, note, shape_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    from mixture_experts_layer_offsets_amd import _lib
    if not __import__("os").path.exists(_lib.LIB_PATH):
        from mixture_experts_layer_offsets_amd import build
        build.build(verbose=False)
    m.load()


def _sched(mode):
    s = m.MoeSched()
    s.schedule = mode
    if mode == m.MOE_SCHED_PIPELINED:
        s.minibatch_rows = 512
    return s


@pytest.mark.parametrize("mode", [m.MOE_SCHED_STAGED, m.MOE_SCHED_PIPELINED])
@pytest.mark.parametrize("mx", [False, True])
def test_layer_calls_do_not_wait(mode, mx):
    w = synth.custom(T=512, H=512, E=16, k=4, I=256, shared_I=256, routing="router",
                     router_std=1 / np.sqrt(512), hot_experts=2, hot_bias=1.0, mx=mx, seed=3)
    note(f"async: schedule {mode} mx={mx}")
    inp = synth.make_inputs(w)
    d = {k: dev(v) for k, v in inp.items() if v is not None and k != "hot"}
    layer = m.MoeLayer(shape_of(w, m.MOE_MXFP8 if mx else m.MOE_BF16))
    layer.prepare(d["w_gate"], d["w_up"], d["w_down"], d["ws_gate"], d["ws_up"], d["ws_down"])
    sc = _sched(mode)

    def run():
        out = layer.forward(d["x"], w_router=d["w_router"], bias=d["bias"], sched=sc)
        g = layer.backward(d["dout"], d["x"], w_router=d["w_router"], sched=sc)
        return out, g

    out0, g0 = run()
    torch.cuda.synchronize()
    ref = (host(out0).copy(), {k: host(v).copy() for k, v in g0.items()})

    stream = torch.cuda.current_stream()
    torch.cuda._sleep(200_000_000)          # a bounded spin on the caller's stream
    t0 = time.perf_counter()
    out1, g1 = run()
    t_call = time.perf_counter() - t0
    busy = not stream.query()               # the sleep (or the layer) still runs
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t0
    note(f"  calls returned after {t_call * 1e3:.2f} ms; stream busy: {busy}; "
         f"all work done after {t_total * 1e3:.1f} ms")
    assert busy, "the layer calls waited for the device"
    assert t_call < t_total
    assert np.array_equal(host(out1), ref[0])
    for k, v in ref[1].items():
        assert np.array_equal(host(g1[k]), v), k


def test_alternating_comm_cus_does_not_wait():
    """Layer calls whose CU split alternates between calls: each split has its
    own set of streams, kept between calls, so no call waits for the device."""
    w = synth.custom(T=512, H=512, E=16, k=4, I=256, routing="supplied", zipf_s=1.0, seed=5)
    note("async: alternating comm_cus 0 / 16 / 0 / 16")
    inp = synth.make_inputs(w)
    d = {k: dev(v) for k, v in inp.items() if v is not None and k != "hot"}
    layer = m.MoeLayer(shape_of(w))
    layer.prepare(d["w_gate"], d["w_up"], d["w_down"])

    def sc(cus):
        s = _sched(m.MOE_SCHED_PIPELINED)
        s.comm_cus = cus
        return s

    def run(cus):
        out = layer.forward(d["x"], topk_idx=d["topk_idx"], topk_w=d["topk_w"], sched=sc(cus))
        g = layer.backward(d["dout"], d["x"], sched=sc(cus))
        return out, g

    out0, g0 = run(0)
    torch.cuda.synchronize()
    ref = (host(out0).copy(), {k: host(v).copy() for k, v in g0.items()})
    run(16)                                  # first use of this split creates its streams
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    torch.cuda._sleep(200_000_000)
    t0 = time.perf_counter()
    results = [run(cus) for cus in (0, 16, 0, 16)]
    t_call = time.perf_counter() - t0
    busy = not stream.query()
    torch.cuda.synchronize()
    note(f"  four calls returned after {t_call * 1e3:.2f} ms; stream busy: {busy}")
    assert busy, "a layer call waited for the device"
    for out, g in results:
        assert np.array_equal(host(out), ref[0])
        for k, v in ref[1].items():
            assert np.array_equal(host(g[k]), v), k
