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
from gpu_util import (TOL_MX, Run, bf, check_layer_mx, check_rel, dev, host, logits_of, note,
                      oracle_forward, unblock_scales)

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
    subnormal) magnitudes, tiny values beside a huge block maximum (scaled by
    2^-s they underflow fp32: the sign rule must still give negative values
    the sign bit), -0.0 inside nonzero blocks, and plain normal data at
    scales 2^-30 .. 2^30."""
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
        elif kind == 7:          # huge maximum, the rest underflow once scaled
            v[:] = rng.standard_normal(32) * 2.0 ** rng.choice([-60, -100, -130], 32)
            v[rng.integers(32)] = rng.choice([-1.0, 1.0]) * 2.0 ** 100
        elif kind == 8:          # -0.0 (and +0.0) among normal values
            v[rng.integers(0, 32, 8)] = -0.0
            v[rng.integers(0, 32, 4)] = 0.0
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


@pytest.mark.parametrize("name", list(MX_CASES))
def test_layer_mx_small(name):
    w = MX_CASES[name]
    note(f"layer {name}: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I} shared={w.shared_I}")
    run = Run(w)
    fw = oracle_forward(run.inp, w, logits_of(run))
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
    fw = oracle_forward(run.inp, w, logits_of(run))
    bw = oracle.backward(run.inp, fw)
    check_layer_mx(run, fw, bw)
    # the same inputs twice give the same bits
    run2 = Run(w, inp=run.inp)
    assert np.array_equal(host(run2.out), host(run.out))
    for key, v in run.grads.items():
        assert np.array_equal(host(run2.grads[key]), host(v)), key


@pytest.mark.parametrize("name,mode", [("mx-supplied-dup", m.MOE_SCHED_STAGED),
                                       ("mx-supplied-dup", m.MOE_SCHED_PIPELINED),
                                       ("mx-k16-router", m.MOE_SCHED_STAGED),
                                       ("mx-shared-router", m.MOE_SCHED_PIPELINED)])
def test_backward_mx_operands_bit_exact(name, mode):
    """The data-gradient GEMMs' MX operands (dy written by the reverse-combine,
    dh by the row quantiser) are the oracle's E4M3/E8M0 quantisation of the
    bf16 dy and dh the backward stored, code for code.  The quantisation of a
    bf16 value is decided exactly in fp32 and in fp64 (a power-of-two scale,
    then one rounding), so the two sides must agree bit for bit."""
    from oracle.numerics import bf16_to_f64
    from oracle.mx import mx_quantize
    w = MX_CASES[name]
    note(f"MX backward operands {name} schedule {mode}: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I}")
    s = m.MoeSched()
    s.schedule = mode
    run = Run(w, sched=s)
    torch.cuda.synchronize()
    R, H, I = w.T * w.k, w.H, w.I
    lay = run.layer
    for name_t, cols in (("dy", H), ("dh", 2 * I)):
        vals = bf16_to_f64(host(lay.work_tensor(name_t, torch.int16, (R, cols))).view(np.uint16))
        codes, scales = mx_quantize(vals, axis=1)
        got_c = host(lay.work_tensor(name_t + "_codes", torch.uint8, (R, cols)))
        got_s = unblock_scales(host(lay.work_tensor(name_t + "_scales", torch.uint8,
                                                    (R, cols // 32))), R, cols)
        _assert_codes_equal(name_t + " codes", got_c, codes)
        _assert_codes_equal(name_t + " scales", got_s, scales)


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
