"""GPU parity of the MXFP8 path (E4M3 codes, E8M0 scales per 32) against the
CPU oracle.

Bit-exact: dispatch codes, scales and round trips (the conversion is a
deterministic function of the bf16 input), routing, layout.  The SwiGLU
epilogue's codes come from fp32 g, u on the GPU and fp64-then-fp32 in the
oracle, so a value lying within rounding of a code boundary may land on the
neighbouring code: every such code is checked to be the code of a value
within the fp32 accumulation error bound of the oracle's (see
_check_act_codes).  Floating point: max|gpu - oracle| / max|oracle| <= 4e-2
per tensor.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_offsets_amd as m
import oracle
import synth
from gpu_util import TOL_MX, Run, bf, check_rel, dev, host, note, unblock_scales
from oracle.mx import e4m3_decode, e4m3_encode, mx_dequantize
from oracle.numerics import bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    from mixture_experts_layer_offsets_amd import _lib
    if not __import__("os").path.exists(_lib.LIB_PATH):
        from mixture_experts_layer_offsets_amd import build
        build.build(verbose=False)
    m.load()


def _edge_rows(T, H, seed):
    """bf16 rows whose 32-blocks cover the conversion's edge cases: zero
    blocks, signed zeros, a lone nonzero, values that round to zero,
    saturation at 448, round-half ties, very large and very small (bf16
    subnormal) magnitudes, and plain normal data at scales 2^-30 .. 2^30."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    nb = H // 32
    blk = x.reshape(T, nb, 32)
    scale = np.ldexp(1.0, rng.integers(-30, 31, size=(T, nb)))
    blk *= scale[..., None]
    kinds = rng.integers(0, 10, size=(T, nb))
    for (t, b), kind in np.ndenumerate(kinds):
        v = blk[t, b]
        if kind == 0:
            v[:] = 0.0
            v[::3] = -0.0
        elif kind == 1:
            v[:] = 0.0
            v[rng.integers(32)] = rng.choice([-1.0, 1.0]) * 2.0 ** rng.integers(-20, 20)
        elif kind == 2:          # one large value, most others round to (signed) zero
            v[:] = rng.standard_normal(32) * 2.0 ** -19
            v[0] = 1.0
        elif kind == 3:          # 460 and 500 of 2^s saturate to 448
            v[:] = rng.choice([-1.0, 1.0], 32) * rng.choice([448.0, 460.0, 500.0, 3.0], 32)
            v *= 2.0 ** rng.integers(-8, 8)
        elif kind == 4:          # halfway between codes at the top binade: ties to even
            v[:] = rng.choice([-1.0, 1.0], 32) * rng.choice([264.0, 280.0, 296.0, 256.0], 32)
        elif kind == 5:          # large magnitudes (finite in bf16)
            v[:] = rng.standard_normal(32) * 2.0 ** 100
        elif kind == 6:          # bf16 subnormals
            v[:] = rng.standard_normal(32) * 2.0 ** -130
    assert np.all(np.isfinite(x.astype(np.float32)))
    return synth.f32_to_bf16_bits(x.astype(np.float32))


def _assert_codes_equal(name, got, ref):
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{name}: {len(bad)} differ, first {bad[:5].tolist()} " \
        f"gpu {got[tuple(bad[:5].T)].tolist()} oracle {ref[tuple(bad[:5].T)].tolist()}"


@pytest.mark.parametrize("T,H,k", [(300, 512, 3), (64, 7168, 8), (1, 128, 1)])
def test_dispatch_mx_bit_exact(T, H, k):
    note(f"dispatch mx T={T} H={H} k={k}")
    E = 8
    x = _edge_rows(T, H, seed=T + H)
    idx, _ = synth.supplied_routing(T, E, k, seed=5)
    _, _, perm, _ = oracle.layout(idx, E)
    shape = m.Shape(T, H, E, k, 128, 0, m.MOE_MXFP8)
    R = T * k
    xq = torch.empty((R, H), dtype=torch.uint8, device="cuda")
    xs = torch.empty((R, H // 32), dtype=torch.uint8, device="cuda")
    m.moe_dispatch(shape, dev(x), dev(perm), xq, xs)
    torch.cuda.synchronize()
    codes, scales = oracle.dispatch(x, perm, k, mx=True)
    _assert_codes_equal("scales", unblock_scales(host(xs), R, H), scales)
    _assert_codes_equal("codes", host(xq), codes)


# ----------------------------------------------------------------------------
# whole layer


def _mx(**kw):
    base = dict(routing="supplied", seed=7, mx=True)
    base.update(kw)
    return synth.custom(**base)


MX_CASES = {
    "mx-tiny-router": synth.custom(T=256, H=512, E=8, k=2, I=256, routing="router",
                                   router_std=0.02, mx=True, seed=1),
    "mx-shared-router": synth.custom(T=512, H=512, E=16, k=4, I=256, shared_I=256,
                                     routing="router", router_std=1 / np.sqrt(512),
                                     hot_experts=2, hot_bias=1.0, mx=True, seed=3),
    "mx-supplied-dup": _mx(T=700, H=768, E=6, k=8, I=384, zipf_s=1.2),
    "mx-one-expert": _mx(T=300, H=256, E=4, k=2, I=128, expert_probs=(0, 0, 1, 0)),
    "mx-ragged": _mx(T=777, H=384, E=5, k=3, I=256),
    "mx-T1": synth.custom(T=1, H=256, E=8, k=2, I=128, routing="router", router_std=0.1,
                          mx=True, seed=2),
    "mx-k16-router": synth.custom(T=200, H=256, E=24, k=16, I=128, routing="router",
                                  router_std=1 / 16, mx=True, seed=12),
    "mx-k12": _mx(T=300, H=384, E=14, k=12, I=256, zipf_s=1.0),
    "mx-E264-router": synth.custom(T=256, H=256, E=264, k=4, I=128, routing="router",
                                   router_std=1 / 16, mx=True, seed=24),
}


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
    for e in range(len(off) - 1):
        rs = slice(int(off[e]), int(off[e + 1]))
        if rs.stop > rs.start:
            Sg[rs] = np.abs(Xh[rs]) @ np.abs(W["g"][e])
            Su[rs] = np.abs(Xh[rs]) @ np.abs(W["u"][e])
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
    w = run.w
    T, k, E, H, I = w.T, w.k, w.E, w.H, w.I
    R = T * k
    idx = host(run.saved("topk_idx", torch.int32, (T, k)))
    amb = np.zeros(T, bool)
    if fw["logits"] is not None:
        L = host(run.saved("logits", torch.float32, (T, E)))
        check_rel("logits", L, fw["logits"], 1e-4)
        ref_idx = fw["idx"]
        amb = np.any(idx != ref_idx, axis=1)
        d = np.abs(L - fw["logits"]).max()
        for t in np.flatnonzero(amb):
            sel = fw["logits"][t, idx[t]]
            assert sel.min() >= np.sort(fw["logits"][t])[-k] - 2 * d
        assert amb.mean() < 0.01
    ok = ~amb
    assert np.array_equal(idx[ok], fw["idx"][ok])
    wts = host(run.saved("topk_w", torch.float32, (T, k)))
    assert np.abs(wts[ok] - fw["w"][ok]).max() <= 1e-5
    perm = host(run.saved("perm", torch.int32, (R,)))
    # dispatch: codes, scales and round trip of the rows the GPU laid out
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
    if not amb.any():
        assert np.array_equal(host(run.saved("counts", torch.int32, (E,))), fw["counts"])
        assert np.array_equal(host(run.saved("offsets", torch.int32, (E + 1,))), fw["offsets"])
        assert np.array_equal(perm, fw["perm"])
        assert np.array_equal(host(run.saved("inv_perm", torch.int32, (R,))), fw["inv"])
        frac = _check_act_codes(aq, as_, fw, H)
        note(f"  act: {frac:.2e} of the codes differ from the oracle's, all within the "
             f"fp32 accumulation bound")
        check_rel("y", bf(run.saved("y", torch.int16, (R, H))), fw["Y"], tol)
    check_rel("out", bf(run.out)[ok], fw["out"][ok], tol)
    if bw is None:
        return
    g = run.grads
    check_rel("dx", bf(g["dx"])[ok], bw["dx"][ok], tol)
    if not amb.any():
        check_rel("dW_gate", host(g["dw_gate"]), bw["dWg"], tol)
        check_rel("dW_up", host(g["dw_up"]), bw["dWu"], tol)
        check_rel("dW_down", host(g["dw_down"]), bw["dWd"], tol)
        check_rel("dtopk_w", host(g["dtopk_w"]), bw["dw"], tol)
        if fw["logits"] is not None:
            check_rel("dW_router", host(g["dw_router"]), bw["dWr"], tol)
        if w.shared_I:
            Is = w.shared_I
            dws = host(g["dws"])
            check_rel("dWs_gate", dws[:H * Is].reshape(H, Is), bw["dWsg"], tol)
            check_rel("dWs_up", dws[H * Is:2 * H * Is].reshape(H, Is), bw["dWsu"], tol)
            check_rel("dWs_down", dws[2 * H * Is:].reshape(Is, H), bw["dWsd"], tol)


@pytest.mark.parametrize("name", list(MX_CASES))
def test_layer_mx_small(name):
    w = MX_CASES[name]
    note(f"layer {name}: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I} shared={w.shared_I}")
    run = Run(w)
    fw = oracle.forward(run.inp, w.k, mx=True)
    bw = oracle.backward(run.inp, fw)
    check_layer_mx(run, fw, bw)
    if name == "mx-one-expert":
        for e in (0, 1, 3):
            assert not host(run.grads["dw_gate"][e]).any()
            assert not host(run.grads["dw_down"][e]).any()


def test_layer_mx_mid():
    # a mid-sized router layer whose oracle (with the MX weight round trips)
    # finishes in under a minute on the host
    w = synth.custom(T=2048, H=1024, E=32, k=6, I=768, routing="router",
                     router_std=1 / 32, mx=True, seed=4)
    note(f"layer mid-mx: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I}")
    run = Run(w)
    fw = oracle.forward(run.inp, w.k, mx=True)
    bw = oracle.backward(run.inp, fw)
    check_layer_mx(run, fw, bw)
    # the same inputs twice give the same bits
    run2 = Run(w, inp=run.inp)
    assert np.array_equal(host(run2.out), host(run.out))
    for key, v in run.grads.items():
        assert np.array_equal(host(run2.grads[key]), host(v)), key


def test_expert_ffn_entry_point_mx():
    """moe_dispatch + moe_expert_ffn + moe_combine on their own (MXFP8)."""
    w = _mx(T=400, H=384, E=6, k=4, I=256)
    note(f"expert_ffn mx: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I}")
    inp = synth.make_inputs(w)
    fw = oracle.forward(inp, w.k, mx=True)
    shape = m.Shape(w.T, w.H, w.E, w.k, w.I, 0, m.MOE_MXFP8)
    layer = m.MoeLayer(shape)
    layer.prepare(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]))
    R = w.T * w.k
    xq = torch.empty((R, w.H), dtype=torch.uint8, device="cuda")
    xs = torch.empty((R, w.H // 32), dtype=torch.uint8, device="cuda")
    m.moe_dispatch(shape, dev(inp["x"]), dev(fw["perm"]), xq, xs)
    y = torch.empty((R, w.H), dtype=torch.int16, device="cuda")
    m.moe_expert_ffn(shape, xq, xs, dev(fw["offsets"]), layer.packed, y, layer.ws)
    out = torch.empty((w.T, w.H), dtype=torch.int16, device="cuda")
    m.moe_combine(shape, y, dev(np.asarray(fw["w"], np.float32)), dev(fw["inv"]), None, out)
    torch.cuda.synchronize()
    check_rel("y", bf(y), fw["Y"], TOL_MX)
    check_rel("out", bf(out), fw["out"], TOL_MX)
