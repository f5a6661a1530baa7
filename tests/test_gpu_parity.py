"""GPU parity: libmoe (through the C ABI) against the CPU oracle.

Bit-exact: top-k indices, counts, offsets, perm, inv_perm, dispatched rows.
Floating point: max|gpu - oracle| / max|oracle| <= 2e-2 per tensor (bf16),
routing weights within 1e-5 absolute.  Inputs come from ``synth`` (seeded);
expected values only from ``oracle``.  Router-routed layers: the selection is
defined given the fp32 logits, so the oracle's top-k and layout run on the
GPU's logits (checked against the oracle's own at 1e-4) and everything after
them must match for every token.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_offsets_amd as m
import oracle
import synth
from gpu_util import (Run, bf, check_layer, check_rel, dev, host, logits_of, note,
                      oracle_forward)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    from mixture_experts_layer_offsets_amd import _lib
    if not __import__("os").path.exists(_lib.LIB_PATH):
        from mixture_experts_layer_offsets_amd import build
        build.build(verbose=False)
    m.load()


def _ws(shape):
    return torch.empty(m.moe_workspace_bytes(shape), dtype=torch.uint8, device="cuda")


# ----------------------------------------------------------------------------
# routing


@pytest.mark.parametrize("T,E,k,ties", [
    (1000, 8, 2, False), (1000, 8, 2, True), (513, 64, 6, False), (513, 64, 6, True),
    (300, 256, 8, False), (77, 256, 8, True), (40, 1024, 16, False), (5, 3, 3, True),
    (1, 1, 1, False)])
def test_route_topk(T, E, k, ties):
    note(f"route T={T} E={E} k={k} ties={ties}")
    L = synth.router_logits_inputs(T, E, seed=11, ties=ties)
    shape = m.Shape(T, 64, E, k, 64)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    m.moe_route(shape, dev(L), idx, w)
    torch.cuda.synchronize()
    ref_idx, ref_w = oracle.topk_softmax(L, k)
    assert np.array_equal(host(idx), ref_idx)
    assert np.abs(host(w) - ref_w).max() <= 1e-5


# ----------------------------------------------------------------------------
# layout


@pytest.mark.parametrize("T,E,k,probs", [
    (1, 1, 1, None), (1, 8, 2, None), (1000, 8, 2, None), (4096, 64, 6, None),
    (2048, 6, 8, "zipf1.0"), (2048, 6, 8, "zipf1.2"), (8192, 256, 8, None),
    (3000, 16, 4, "one"), (2500, 6, 8, (1, 0, 0, 3, 0, 2)), (700, 1024, 3, None),
    (1023, 5, 1, None), (1025, 5, 1, None), (333, 3, 7, None)])
def test_layout(T, E, k, probs):
    note(f"layout T={T} E={E} k={k} probs={probs}")
    if probs == "one":
        probs = (1,) + (0,) * (E - 1)
    elif isinstance(probs, str):
        probs = synth._zipf_probs(E, float(probs[4:]))
    idx, _ = synth.supplied_routing(T, E, k, seed=T + 3 * E, probs=probs)
    shape = m.Shape(T, 64, E, k, 64)
    R = T * k
    i32 = dict(dtype=torch.int32, device="cuda")
    counts, offsets = torch.empty(E, **i32), torch.empty(E + 1, **i32)
    perm, inv = torch.empty(R, **i32), torch.empty(R, **i32)
    m.moe_layout(shape, dev(idx), counts, offsets, perm, inv, _ws(shape))
    torch.cuda.synchronize()
    rc, ro, rp, ri = oracle.layout(idx, E)
    assert np.array_equal(host(counts), rc)
    assert np.array_equal(host(offsets), ro)
    assert np.array_equal(host(perm), rp)
    assert np.array_equal(host(inv), ri)


# ----------------------------------------------------------------------------
# dispatch and combine on their own


@pytest.mark.parametrize("shared", [False, True])
def test_dispatch_and_combine(shared):
    note(f"dispatch/combine shared={shared}")
    T, H, E, k = 300, 512, 8, 3
    idx, wts = synth.supplied_routing(T, E, k, seed=2)
    rng = np.random.default_rng(1)
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    y = synth.f32_to_bf16_bits(rng.standard_normal((T * k, H)).astype(np.float32))
    ys = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)) if shared else None
    _, _, perm, inv = oracle.layout(idx, E)
    shape = m.Shape(T, H, E, k, 64)
    xp = torch.empty((T * k, H), dtype=torch.int16, device="cuda")
    m.moe_dispatch(shape, dev(x), dev(perm), xp)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    m.moe_combine(shape, dev(y), dev(wts), dev(inv), dev(ys), out)
    torch.cuda.synchronize()
    assert np.array_equal(host(xp).view(np.uint16), oracle.dispatch(x, perm, k))
    ref = oracle.combine(oracle.numerics.bf16_to_f64(y), wts, inv, k,
                         None if ys is None else oracle.numerics.bf16_to_f64(ys))
    check_rel("combine", bf(out), ref, 4e-3)


# ----------------------------------------------------------------------------
# whole layer


def _small(**kw):
    base = dict(routing="supplied", seed=7)
    base.update(kw)
    return synth.custom(**base)


LAYER_CASES = {
    "tiny": synth.workload("tiny"),
    "shared-router": synth.custom(T=512, H=512, E=16, k=4, I=192, shared_I=256,
                                  routing="router", router_std=1 / np.sqrt(512),
                                  hot_experts=2, hot_bias=1.0, seed=3),
    "supplied-dup": _small(T=700, H=768, E=6, k=8, I=320, zipf_s=1.0),
    "one-expert": _small(T=300, H=256, E=4, k=2, I=128, expert_probs=(0, 0, 1, 0)),
    "E1k1": _small(T=200, H=256, E=1, k=1, I=128),
    "T1": synth.custom(T=1, H=256, E=8, k=2, I=128, routing="router", router_std=0.1, seed=2),
    "ragged": _small(T=777, H=320, E=5, k=3, I=192),
    # top-k above 8 takes the 16-slot kernel instances (router, dispatch,
    # combine, reverse kernels); 16 is the library's bound
    "k16-router": synth.custom(T=300, H=256, E=32, k=16, I=128, routing="router",
                               router_std=1 / 16, seed=11),
    "k12-shared": _small(T=257, H=320, E=20, k=12, I=192, shared_I=128, zipf_s=1.0),
    "k9-router": synth.custom(T=129, H=256, E=16, k=9, I=128, routing="router",
                              router_std=1 / 16, seed=12),
    # the library's expert bound (1024; the router's 16-slot top-k, many
    # experts without rows) and an expert count that is not a multiple of 8
    "E1024-router": synth.custom(T=512, H=256, E=1024, k=8, I=64, routing="router",
                                 router_std=1 / 16, seed=21),
    "E517-supplied": _small(T=400, H=256, E=517, k=6, I=128, zipf_s=0.8),
}


@pytest.mark.parametrize("name", list(LAYER_CASES))
def test_layer_small(name):
    w = LAYER_CASES[name]
    note(f"layer {name}: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I} shared={w.shared_I}")
    run = Run(w)
    fw = oracle_forward(run.inp, w, logits_of(run))
    bw = oracle.backward(run.inp, fw)
    check_layer(run, fw, bw)
    if name == "one-expert":   # experts without rows get exactly zero gradients
        for e in (0, 1, 3):
            assert not host(run.grads["dw_gate"][e]).any()
            assert not host(run.grads["dw_down"][e]).any()


@pytest.fixture(scope="module")
def mid():
    w = synth.workload("mid")
    note("layer mid: T=4096 H=2048 E=64 k=6 I=1408")
    run = Run(w)
    fw = oracle_forward(run.inp, w, logits_of(run))
    bw = oracle.backward(run.inp, fw)
    return run, fw, bw


def test_layer_mid(mid):
    check_layer(*mid)


def test_layer_mid_deterministic(mid):
    run, _, _ = mid
    note("layer mid: second run for determinism")
    out1 = host(run.out).copy()
    g1 = {k: host(v).copy() for k, v in run.grads.items()}
    run2 = Run(run.w, inp=run.inp)
    assert np.array_equal(host(run2.out), out1)
    for k, v in g1.items():
        assert np.array_equal(host(run2.grads[k]), v), k
