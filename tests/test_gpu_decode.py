"""The few-token inference forward (moe_decode_fwd) against the oracle.

The decode path computes the layer's output with its own weight-streaming
kernels (fp32 dot products summed in a different order than the MFMA
tiles), so it is compared with the oracle at the bf16 tolerance, and with
moe_layer_fwd on the same inputs at the same tolerance.  With a router, the
oracle routes from the decode path's own fp32 logits (read from the
workspace), and the decode's selection must equal the oracle's for every
token, weights within 1e-5.  Cases: one token,
a few tokens, a token count that is not a multiple of anything, experts with
more than one 64-row pass (supplied routing with duplicates), unused experts,
the shared expert, the Kimi-shaped dimensions (4 tokens, and 24 tokens with
one to four 16-row blocks per pass and a second pass on the heavy expert:
long contractions, where the weight ring wraps around its slots and a
pass's last steps only fill it), top-k above 8 (router and supplied
routing), and MXFP8 shapes (refused).
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_offsets_amd as m
import oracle
import synth
from gpu_util import TOL_BF16, bf, check_rel, dev, host, note, oracle_forward, shape_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    from mixture_experts_layer_offsets_amd import _lib
    if not __import__("os").path.exists(_lib.LIB_PATH):
        from mixture_experts_layer_offsets_amd import build
        build.build(verbose=False)
    m.load()


CASES = {
    "t1-router": synth.custom(T=1, H=512, E=8, k=2, I=256, routing="router", router_std=0.05,
                              seed=1),
    "t5-router": synth.custom(T=5, H=512, E=16, k=4, I=192, routing="router", router_std=0.05,
                              seed=2),
    "t37-supplied": synth.custom(T=37, H=768, E=6, k=8, I=320, zipf_s=1.0, routing="supplied",
                                 seed=3),
    "t64-dup-passes": synth.custom(T=64, H=256, E=3, k=8, I=128, zipf_s=1.5,
                                   routing="supplied", seed=4),
    "t9-shared": synth.custom(T=9, H=512, E=16, k=4, I=192, shared_I=256, routing="router",
                              router_std=1 / np.sqrt(512), hot_experts=2, hot_bias=1.0, seed=5),
    "kimi-dims-t4": synth.custom(T=4, H=7168, E=6, k=8, I=2048, zipf_s=1.0,
                                 routing="supplied", seed=6),
    # long contractions with every row-block count: 71 rows (a 64-row pass of
    # four blocks, then 7 rows), 44, 32, 21 and 12 rows on the experts
    "kimi-dims-t24": synth.custom(T=24, H=7168, E=6, k=8, I=2048, zipf_s=1.0,
                                  routing="supplied", seed=7),
    "t7-k16-router": synth.custom(T=7, H=512, E=32, k=16, I=256, routing="router",
                                  router_std=0.05, seed=14),
    "t3-k11-supplied": synth.custom(T=3, H=256, E=5, k=11, I=128, routing="supplied", seed=15),
    "t5-E1024-router": synth.custom(T=5, H=256, E=1024, k=8, I=64, routing="router",
                                    router_std=0.05, seed=23),
}


@pytest.mark.parametrize("name", list(CASES))
def test_decode_matches_oracle(name):
    w = CASES[name]
    note(f"decode {name}: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I} shared={w.shared_I}")
    inp = synth.make_inputs(w)
    shape = shape_of(w)
    layer = m.MoeLayer(shape)
    d = {k: dev(v) for k, v in inp.items() if v is not None and k != "hot"}
    layer.prepare(d["w_gate"], d["w_up"], d["w_down"], d.get("ws_gate"), d.get("ws_up"),
                  d.get("ws_down"))
    out = layer.decode(d["x"], w_router=d.get("w_router"), bias=d.get("bias"),
                       topk_idx=d.get("topk_idx"), topk_w=d.get("topk_w"))
    torch.cuda.synchronize()
    if w.routing == "router":
        # the decode path's own routing, left in the workspace: the oracle's
        # top-k runs on its fp32 logits, and the selection must match exactly
        T, k, E = w.T, w.k, w.E
        L = host(layer.work_tensor("dec_logits", torch.float32, (T, E)))
        fw = oracle_forward(inp, w, L)
        assert np.array_equal(host(layer.work_tensor("dec_topk_idx", torch.int32, (T, k))),
                              fw["idx"])
        wts = host(layer.work_tensor("dec_topk_w", torch.float32, (T, k)))
        assert np.abs(wts - fw["w"]).max() <= 1e-5
    else:
        fw = oracle.forward(inp, w.k)
    out_h = bf(out).copy()
    ref = layer.forward(d["x"], w_router=d.get("w_router"), bias=d.get("bias"),
                        topk_idx=d.get("topk_idx"), topk_w=d.get("topk_w"))
    torch.cuda.synchronize()
    check_rel("out vs oracle", out_h, fw["out"], TOL_BF16)
    check_rel("out vs layer forward", out_h, bf(ref), TOL_BF16)


def test_decode_deterministic():
    w = CASES["t37-supplied"]
    inp = synth.make_inputs(w)
    layer = m.MoeLayer(shape_of(w))
    d = {k: dev(v) for k, v in inp.items() if v is not None and k != "hot"}
    layer.prepare(d["w_gate"], d["w_up"], d["w_down"])
    a = host(layer.decode(d["x"], topk_idx=d["topk_idx"], topk_w=d["topk_w"])).copy()
    b = host(layer.decode(d["x"], topk_idx=d["topk_idx"], topk_w=d["topk_w"]))
    assert np.array_equal(a, b)


def test_decode_refuses_mxfp8():
    w = synth.custom(T=4, H=512, E=8, k=2, I=256, routing="supplied", mx=True, seed=1)
    inp = synth.make_inputs(w)
    layer = m.MoeLayer(shape_of(w, m.MOE_MXFP8))
    d = {k: dev(v) for k, v in inp.items() if v is not None and k != "hot"}
    with pytest.raises(m.MoeError) as e:
        layer.decode(d["x"], topk_idx=d["topk_idx"], topk_w=d["topk_w"])
    from mixture_experts_layer_offsets_amd import _lib
    assert e.value.code == _lib.MOE_ERR_UNSUPPORTED
