"""Seeded synthetic inputs for one MoE layer (forward + backward).

This module only draws random numbers and stores them in the layer's input
formats (bf16 bit patterns, fp32, int32).  It holds none of the layer's
arithmetic: no routing, no layout, no quantisation, no FFN.  Both the CPU
oracle (``oracle/``) and the GPU library consume the identical bytes that it
returns, so it is the one piece of code the two sides share.

Recipe (all draws from ``numpy.random.Generator(PCG64)`` seeded by a
``SeedSequence``; fp32 normal draws are rounded to bf16 with
round-to-nearest-even):

* x ~ N(0, 1)                                      [T, H]   bf16
* router W_r ~ N(0, router_std^2), router_std as configured     [H, E]   bf16
* W_gate, W_up ~ N(0, 1/H); W_down ~ N(0, 1/I)     [E,H,I], [E,H,I], [E,I,H] bf16
  (each expert has its own child stream, so the bytes do not depend on how
  many threads draw them)
* shared expert weights (when present) likewise, fan-in H / I_s
* supplied routing: each (token, slot) expert drawn i.i.d. from a categorical
  distribution (Zipf: P(e) proportional to (e+1)^-s, expert 0 hottest), and
  the k slot weights of a token the softmax of k i.i.d. N(0, 1) draws
  (positive, summing to one: what a softmax router gives scores of unit
  spread), stored as fp32
* router bias (skewed configurations): +beta on a seeded set of "hot" experts
* dOut ~ N(0, 1)                                   [T, H]   bf16

The named workloads mirror the layer shapes the pages discuss (hidden 7168,
expert intermediate 2048, 2048 tokens per GPU before routing) plus a tiny and
a mid-sized case.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

BF16 = np.uint16  # bf16 values are carried as their 16-bit patterns


@dataclass(frozen=True)
class Workload:
    name: str
    T: int                      # tokens
    H: int                      # hidden size
    E: int                      # routed experts held by this GPU
    k: int                      # top-k
    I: int                      # expert intermediate size
    mx: bool = False            # MXFP8 (E4M3 + E8M0 per 32-element block)
    wfmt: str = "e4m3"          # with mx: the expert weights' MX element format
                                # (e4m3, or e2m1 / e2m3 / e3m2 for lower-precision experts)
    routing: str = "router"     # "router" (W_r given) or "supplied" (idx, w given)
    router_std: float = 0.0     # std of W_r entries (router routing)
    zipf_s: float = 0.0         # Zipf exponent of supplied routing (0 = uniform)
    expert_probs: Optional[tuple] = None  # explicit categorical for supplied routing
    hot_experts: int = 0        # number of biased ("hot") experts, router routing
    hot_bias: float = 0.0       # bias added to the hot experts' logits
    shared_I: int = 0           # intermediate size of the one shared expert (0 = none)
    backward: bool = True       # whether the workload includes the backward pass
    minibatch_rows: int = 0     # routed rows per minibatch of the pipelined path (0 = default)
    seed: int = 0

    @property
    def R(self) -> int:
        return self.T * self.k


def _named() -> dict:
    kimi = dict(T=2048, H=7168, E=6, k=8, I=2048, routing="supplied",
                minibatch_rows=2368)
    # Hot-expert bias for the DeepSeek-V3-shaped layer: 26 of 256 experts
    # (about 10 %) get +1.09 on their logits, which sends about half of all
    # routed rows to them (the achieved share is checked by the tests).
    dsv3 = dict(T=8192, H=7168, E=256, k=8, I=2048, routing="router",
                router_std=1.0 / math.sqrt(7168), hot_experts=26, hot_bias=1.09,
                shared_I=2048)
    w = [
        Workload("tiny", T=256, H=512, E=8, k=2, I=256, routing="router",
                 router_std=0.02, backward=False),
        Workload("mid", T=4096, H=2048, E=64, k=6, I=1408, routing="router",
                 router_std=1.0 / math.sqrt(2048)),
        Workload("kimi-bf16", zipf_s=1.0, **kimi),
        Workload("kimi-mx", zipf_s=1.2, mx=True, **kimi),
        Workload("kimi-fp4", zipf_s=1.2, mx=True, wfmt="e2m1", **kimi),
        Workload("kimi-fp6", zipf_s=1.2, mx=True, wfmt="e2m3", **kimi),
        Workload("dsv3-bf16", **dsv3),
        Workload("dsv3-mx", mx=True, **dsv3),
    ]
    return {x.name: x for x in w}


WORKLOADS = _named()


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields replaced (e.g. T for a sample)."""
    return replace(WORKLOADS[name], **overrides) if overrides else WORKLOADS[name]


def custom(**kw) -> Workload:
    kw.setdefault("name", "custom")
    return Workload(**kw)


# ----------------------------------------------------------------------------
# drawing helpers

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); return bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    return ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))))
            >> np.uint32(16)).astype(np.uint16)


def _normal_bf16(seq: np.random.SeedSequence, shape, std: float) -> np.ndarray:
    rng = np.random.default_rng(seq)
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return f32_to_bf16_bits(a)


def _expert_stack(seq: np.random.SeedSequence, E: int, shape, std: float,
                  threads: int) -> np.ndarray:
    kids = seq.spawn(E)
    out = np.empty((E,) + tuple(shape), dtype=np.uint16)

    def one(e):
        out[e] = _normal_bf16(kids[e], shape, std)

    if threads > 1 and E > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(E)))
    else:
        for e in range(E):
            one(e)
    return out


def _softmax_draws(rng: np.random.Generator, T: int, k: int) -> np.ndarray:
    """[T, k] fp32 slot weights: per token, the softmax of k N(0, 1) draws."""
    z = rng.standard_normal((T, k))
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def _zipf_probs(E: int, s: float) -> np.ndarray:
    p = (np.arange(1, E + 1, dtype=np.float64)) ** (-s)
    return p / p.sum()


def make_inputs(w: Workload, threads: int = 8, only=None) -> dict:
    """Draw every input of workload ``w`` (or only the keys listed in ``only``;
    each tensor has its own stream, so skipping some changes no other).

    Returns a dict of numpy arrays:
      x [T,H] u16, dout [T,H] u16,
      w_gate [E,H,I] u16, w_up [E,H,I] u16, w_down [E,I,H] u16,
      router: w_router [H,E] u16 and bias [E] f32 (or None),
      supplied routing: topk_idx [T,k] i32, topk_w [T,k] f32,
      shared expert (or None): ws_gate [H,Is], ws_up [H,Is], ws_down [Is,H] u16,
      hot [n_hot] i32 (ids of the biased experts, router routing only).
    """
    root = np.random.SeedSequence(w.seed)
    s_x, s_wr, s_wg, s_wu, s_wd, s_sh, s_rt, s_do = root.spawn(8)
    T, H, E, k, I = w.T, w.H, w.E, w.k, w.I

    def want(key):
        return only is None or key in only

    out: dict = dict.fromkeys(["x", "w_router", "bias", "hot", "w_gate", "w_up", "w_down",
                               "ws_gate", "ws_up", "ws_down", "topk_idx", "topk_w", "dout"])
    if want("x"):
        out["x"] = _normal_bf16(s_x, (T, H), 1.0)
    if w.routing == "router" and want("w_router"):
        out["w_router"] = _normal_bf16(s_wr, (H, E), w.router_std)
    if want("w_gate"):
        out["w_gate"] = _expert_stack(s_wg, E, (H, I), 1.0 / math.sqrt(H), threads)
    if want("w_up"):
        out["w_up"] = _expert_stack(s_wu, E, (H, I), 1.0 / math.sqrt(H), threads)
    if want("w_down"):
        out["w_down"] = _expert_stack(s_wd, E, (I, H), 1.0 / math.sqrt(I), threads)
    if w.shared_I and want("ws_gate"):
        a, b, c = s_sh.spawn(3)
        Is = w.shared_I
        out["ws_gate"] = _normal_bf16(a, (H, Is), 1.0 / math.sqrt(H))
        out["ws_up"] = _normal_bf16(b, (H, Is), 1.0 / math.sqrt(H))
        out["ws_down"] = _normal_bf16(c, (Is, H), 1.0 / math.sqrt(Is))
    rng = np.random.default_rng(s_rt)
    if w.routing == "router":
        if w.hot_experts:
            hot = np.sort(rng.choice(E, w.hot_experts, replace=False)).astype(np.int32)
            bias = np.zeros(E, np.float32)
            bias[hot] = np.float32(w.hot_bias)
            out["bias"] = bias
            out["hot"] = hot
    elif w.routing == "supplied":
        if w.expert_probs is not None:
            p = np.asarray(w.expert_probs, np.float64)
            p = p / p.sum()
        else:
            p = _zipf_probs(E, w.zipf_s)
        out["topk_idx"] = rng.choice(E, size=(T, k), p=p).astype(np.int32)
        out["topk_w"] = _softmax_draws(rng, T, k)
    else:
        raise ValueError(f"unknown routing {w.routing!r}")
    if want("dout"):
        out["dout"] = _normal_bf16(s_do, (T, H), 1.0)
    return out


def router_logits_inputs(T: int, E: int, seed: int = 0, ties: bool = False) -> np.ndarray:
    """Synthetic fp32 router logits [T,E] for testing top-k selection alone.

    With ``ties`` the logits are drawn from a small set of values so that many
    tokens have exactly equal logits (exercises the lower-index tie rule),
    including +0.0 / -0.0 pairs.
    """
    rng = np.random.default_rng(np.random.SeedSequence([seed, T, E, int(ties)]))
    if ties:
        vals = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 1.0, 3.0], np.float32)
        return vals[rng.integers(0, len(vals), size=(T, E))]
    return rng.standard_normal((T, E), dtype=np.float32)


def supplied_routing(T: int, E: int, k: int, seed: int = 0, probs=None):
    """Synthetic supplied routing: (topk_idx [T,k] i32, topk_w [T,k] f32)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, T, E, k, 7]))
    p = None if probs is None else np.asarray(probs, np.float64) / np.sum(probs)
    idx = rng.choice(E, size=(T, k), p=p).astype(np.int32)
    return idx, _softmax_draws(rng, T, k)
