"""Helpers of the GPU parity tests: device copies, bf16 decoding, tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

import mixture_experts_layer_offsets_amd as m
import oracle
from oracle.mx import e4m3_decode, e4m3_encode, mx_dequantize
from oracle.numerics import bf16_bits, bf16_to_f64

TOL_BF16 = 2e-2   # max|gpu - oracle| / max|oracle| per tensor, bf16 path
TOL_MX = 4e-2     # same, MXFP8 path


def dev(a):
    """numpy -> torch on cuda:0 (bf16 bit patterns travel as int16)."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t):
    return t.detach().cpu().numpy()


def bf(t):
    """A device int16/bf16 tensor -> fp64 values."""
    return bf16_to_f64(host(t).view(np.uint16))


def rel_err(gpu, ref) -> float:
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    den = np.abs(ref).max()
    if den == 0:
        return float(np.abs(gpu).max())
    return float(np.abs(gpu - ref).max() / den)


def check_rel(name, gpu, ref, tol):
    e = rel_err(gpu, ref)
    note(f"    {name}: max|gpu-oracle|/max|oracle| = {e:.2e} (tolerance {tol})")
    assert e <= tol, f"{name}: max|gpu-oracle|/max|oracle| = {e:.3e} > {tol}"
    return e


def unblock_scales(s, rows, K):
    """E8M0 scales as the library stores them, K-blocked ([K/128][rows][4]:
    the scale of row r, block b at (b/4 * rows + r) * 4 + b%4), to the
    oracle's [rows][K/32]."""
    a = np.asarray(s).reshape(K // 128, rows, 4)
    return np.ascontiguousarray(a.transpose(1, 0, 2).reshape(rows, K // 32))


def note(msg: str):
    """Print and flush a progress line (names the case before GPU work)."""
    print(msg, flush=True)
    sys.stdout.flush()


def dtype_of(w):
    """The library datatype of workload ``w``."""
    if not w.mx:
        return m.MOE_BF16
    return {"e4m3": m.MOE_MXFP8, "e2m1": m.MOE_MXFP8_W4, "e2m3": m.MOE_MXFP8_W6,
            "e3m2": m.MOE_MXFP8_W6E3M2}[w.wfmt]


def shape_of(w, dtype=None):
    return m.Shape(w.T, w.H, w.E, w.k, w.I, w.shared_I, dtype_of(w) if dtype is None else dtype)


class Run:
    """Inputs of a workload on the device plus one forward (+ backward) pass
    (``sched``: the moe_sched of both calls; None = staged)."""

    def __init__(self, w, inp=None, backward=True, sched=None):
        self.w = w
        self.inp = inp if inp is not None else __import__("synth").make_inputs(w)
        inp = self.inp
        self.shape = shape_of(w)
        self.layer = m.MoeLayer(self.shape)
        self.layer.prepare(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]),
                           dev(inp["ws_gate"]), dev(inp["ws_up"]), dev(inp["ws_down"]))
        self.x = dev(inp["x"])
        self.wr = dev(inp["w_router"])
        self.bias = dev(inp["bias"])
        self.idx = dev(inp["topk_idx"])
        self.tw = dev(inp["topk_w"])
        self.out = self.layer.forward(self.x, w_router=self.wr, bias=self.bias,
                                      topk_idx=self.idx, topk_w=self.tw, sched=sched)
        self.grads = None
        if backward:
            self.dout = dev(inp["dout"])
            self.grads = self.layer.backward(self.dout, self.x, w_router=self.wr, sched=sched)
        torch.cuda.synchronize()

    def saved(self, name, dtype, shape):
        return self.layer.saved_tensor(name, dtype, shape)


def oracle_forward(inp, w, logits_gpu=None, mx=None):
    """The oracle's forward of workload ``w`` on ``inp``.

    Router routing is defined given the fp32 logits, so the oracle's own top-k
    and layout run on the GPU's fp32 logits (``logits_gpu``), and the GPU's
    idx, weights, counts, offsets, perm and inv_perm must then match bit for
    bit (weights to 1e-5).  The GPU's logits are checked against the oracle's
    own fp64-summed logits at 1e-4 of their maximum; how many tokens those
    would route differently (a near-tie moved by the fp32 summation order) is
    reported, not failed.
    """
    mx = w.mx if mx is None else mx
    if w.routing != "router":
        return oracle.forward(inp, w.k, mx=mx, wfmt=w.wfmt)
    own = oracle.router_logits(inp["x"], inp["w_router"], inp.get("bias"))
    check_rel("logits", logits_gpu, own, 1e-4)
    fw = oracle.forward(inp, w.k, mx=mx, logits=logits_gpu, wfmt=w.wfmt)
    own_idx, _ = oracle.topk_softmax(own, w.k)
    n = int(np.any(own_idx != fw["idx"], axis=1).sum())
    note(f"  routing from the GPU's logits; {n} of {w.T} tokens would route differently "
         f"from the oracle's own fp64 logits (near-ties)")
    return fw


def check_routing_layout(layer, w, fw):
    """idx, counts, offsets, perm, inv_perm bit-exact; routing weights to 1e-5."""
    T, k, E = w.T, w.k, w.E
    R = T * k
    assert np.array_equal(host(layer.saved_tensor("topk_idx", torch.int32, (T, k))), fw["idx"])
    wts = host(layer.saved_tensor("topk_w", torch.float32, (T, k)))
    assert np.abs(wts - fw["w"]).max() <= 1e-5
    assert np.array_equal(host(layer.saved_tensor("counts", torch.int32, (E,))), fw["counts"])
    assert np.array_equal(host(layer.saved_tensor("offsets", torch.int32, (E + 1,))),
                          fw["offsets"])
    assert np.array_equal(host(layer.saved_tensor("perm", torch.int32, (R,))), fw["perm"])
    assert np.array_equal(host(layer.saved_tensor("inv_perm", torch.int32, (R,))), fw["inv"])


def logits_of(run):
    """The GPU's saved fp32 router logits (None for supplied routing)."""
    w = run.w
    if w.routing != "router":
        return None
    return host(run.saved("logits", torch.float32, (w.T, w.E)))


def check_layer(run, fw, bw, tol=TOL_BF16):
    """Every saved tensor, output and gradient of a bf16 layer run against the
    oracle routed from the GPU's logits (gpu_util.oracle_forward): routing and
    layout bit-exact, dispatched rows bit-exact, the rest within ``tol``."""
    w = run.w
    T, k, E, H, I = w.T, w.k, w.E, w.H, w.I
    R = T * k
    check_routing_layout(run.layer, w, fw)
    xp = host(run.saved("x_perm", torch.int16, (R, H))).view(np.uint16)
    assert np.array_equal(xp, oracle.dispatch(run.inp["x"], fw["perm"], k))
    check_rel("y", bf(run.saved("y", torch.int16, (R, H))), fw["Y"], tol)
    check_rel("act", bf(run.saved("act", torch.int16, (R, I))), fw["ahat"], tol)
    check_rel("out", bf(run.out), fw["out"], tol)
    if bw is None:
        return
    g = run.grads
    check_rel("dx", bf(g["dx"]), bw["dx"], tol)
    check_rel("dW_gate", host(g["dw_gate"]), bw["dWg"], tol)
    check_rel("dW_up", host(g["dw_up"]), bw["dWu"], tol)
    check_rel("dW_down", host(g["dw_down"]), bw["dWd"], tol)
    check_rel("dtopk_w", host(g["dtopk_w"]), bw["dw"], tol)
    if fw["logits"] is not None:
        check_rel("dW_router", host(g["dw_router"]), bw["dWr"], tol)
    if w.shared_I:
        Is = w.shared_I
        check_rel("y_shared", bf(run.saved("y_shared", torch.int16, (T, H))),
                  fw["shared"]["y"], tol)
        dws = host(g["dws"])
        check_rel("dWs_gate", dws[:H * Is].reshape(H, Is), bw["dWsg"], tol)
        check_rel("dWs_up", dws[H * Is:2 * H * Is].reshape(H, Is), bw["dWsu"], tol)
        check_rel("dWs_down", dws[2 * H * Is:].reshape(Is, H), bw["dWsd"], tol)


def _quantise_at(v, s):
    """Values of the E4M3 codes of v at the block scale 2^s (s broadcast per
    element): the oracle's element conversion with the scale given."""
    sc = np.clip(np.ldexp(v, -s), -448.0, 448.0)
    return e4m3_decode(e4m3_encode(sc)) * np.ldexp(1.0, s)


def _block_scale(amax):
    _, ex = np.frexp(amax)
    return np.where(amax > 0, np.clip(ex.astype(np.int64) - 1 - 8, -127, 127), -127)


def _check_act_codes(aq, as_, fw, K):
    """The SwiGLU epilogue's MX codes of a against the oracle.

    The GPU forms g and u by fp32 accumulation in its own order; any order
    keeps |g_gpu - g| <= gamma * sum_h |x_h w_h| with gamma = K 2^-24 / (1 -
    K 2^-24) (the standard bound of recursive summation), likewise u.  From
    these bounds (and a few ulps for silu and the product) each element's a
    lies in [a - da, a + da]; the GPU's block scale must be the scale of some
    block maximum in the resulting range, and each GPU code must be the code,
    at that scale, of some value in its element's range (quantisation is
    monotone).  Codes equal to the oracle's need no bound; the fraction of the
    others is reported.
    """
    W, Xh, off = fw["W"], fw["Xhat"], fw["offsets"]
    g, u = fw["g"], fw["u"]
    Sg = np.zeros_like(g)
    Su = np.zeros_like(u)

    def sums(e):
        rs = slice(int(off[e]), int(off[e + 1]))
        We = W.fwd(e)
        Sg[rs] = np.abs(Xh[rs]) @ np.abs(We["g"])
        Su[rs] = np.abs(Xh[rs]) @ np.abs(We["u"])
    oracle.layer._each(sums, [e for e in range(len(off) - 1) if off[e + 1] > off[e]])
    eps = 2.0 ** -24
    gamma = K * eps / (1 - K * eps) + eps          # + the final fp32 rounding of g, u
    dg, du = gamma * Sg, gamma * Su
    sg = 1.0 / (1.0 + np.exp(-g))
    a = g * sg * u
    # |silu'| <= 1.1 everywhere; 16 ulps for silu (hardware exp) and the product
    da = 1.1 * (np.abs(u) + du) * dg + np.abs(g * sg) * du + 16 * eps * np.abs(a) + 1e-38
    got = mx_dequantize(aq, as_, axis=1)
    s_gpu = np.repeat(as_.astype(np.int64) - 127, 32, axis=1)
    R, I = a.shape
    amax_lo = np.maximum(np.abs(a) - da, 0).reshape(R, -1, 32).max(axis=2)
    amax_hi = (np.abs(a) + da).reshape(R, -1, 32).max(axis=2)
    s_lo = np.repeat(_block_scale(amax_lo), 32, axis=1)
    s_hi = np.repeat(_block_scale(amax_hi), 32, axis=1)
    assert np.all((s_gpu >= s_lo) & (s_gpu <= s_hi)), "act: block scale outside its range"
    lo = _quantise_at(a - da, s_gpu)
    hi = _quantise_at(a + da, s_gpu)
    diff = got != fw["ahat"]
    bad = diff & ((got < lo) | (got > hi))
    assert not bad.any(), f"act: {bad.sum()} codes outside the range the fp32 bound allows"
    return float(diff.mean())


def check_layer_mx(run, fw, bw, tol=TOL_MX):
    """Every saved tensor, output and gradient of an MXFP8 layer run against
    the oracle routed from the GPU's logits: routing, layout and the
    dispatched rows' codes, scales and round trips bit-exact; the SwiGLU
    epilogue's codes equal to the oracle's or within the fp32 accumulation
    bound (_check_act_codes); the rest within ``tol``."""
    w = run.w
    T, k, E, H, I = w.T, w.k, w.E, w.H, w.I
    R = T * k
    check_routing_layout(run.layer, w, fw)
    perm = fw["perm"]
    codes, scales = oracle.dispatch(run.inp["x"], perm, k, mx=True)
    assert np.array_equal(host(run.saved("x_perm", torch.uint8, (R, H))), codes)
    xs = unblock_scales(host(run.saved("x_scale", torch.uint8, (R, H // 32))), R, H)
    assert np.array_equal(xs, scales)
    xh = host(run.saved("x_hat", torch.int16, (R, H))).view(np.uint16)
    assert np.array_equal(xh, bf16_bits(mx_dequantize(codes, scales, axis=1)))
    # the activation's codes and its bf16 round trip agree with each other
    aq = host(run.saved("act_q", torch.uint8, (R, I)))
    as_ = unblock_scales(host(run.saved("act_scale", torch.uint8, (R, I // 32))), R, I)
    act = bf(run.saved("act", torch.int16, (R, I)))
    assert np.array_equal(act, mx_dequantize(aq, as_, axis=1))
    frac = _check_act_codes(aq, as_, fw, H)
    note(f"  act: {frac:.2e} of the codes differ from the oracle's, all within the "
         f"fp32 accumulation bound")
    check_rel("act", act, fw["ahat"], tol)
    check_rel("y", bf(run.saved("y", torch.int16, (R, H))), fw["Y"], tol)
    check_rel("out", bf(run.out), fw["out"], tol)
    if bw is None:
        return
    g = run.grads
    check_rel("dx", bf(g["dx"]), bw["dx"], tol)
    check_rel("dW_gate", host(g["dw_gate"]), bw["dWg"], tol)
    check_rel("dW_up", host(g["dw_up"]), bw["dWu"], tol)
    check_rel("dW_down", host(g["dw_down"]), bw["dWd"], tol)
    check_rel("dtopk_w", host(g["dtopk_w"]), bw["dw"], tol)
    if fw["logits"] is not None:
        check_rel("dW_router", host(g["dw_router"]), bw["dWr"], tol)
    if w.shared_I:
        Is = w.shared_I
        check_rel("y_shared", bf(run.saved("y_shared", torch.int16, (T, H))),
                  fw["shared"]["y"], tol)
        dws = host(g["dws"])
        check_rel("dWs_gate", dws[:H * Is].reshape(H, Is), bw["dWsg"], tol)
        check_rel("dWs_up", dws[H * Is:2 * H * Is].reshape(H, Is), bw["dWsu"], tol)
        check_rel("dWs_down", dws[2 * H * Is:].reshape(Is, H), bw["dWsd"], tol)


