"""Lower-precision experts: MXFP8 activations with the expert weights' MX
copies in FP4 E2M1, FP6 E2M3 or FP6 E3M2 (MOE_MXFP8_W4 / _W6 / _W6E3M2),
against the oracle with the same weight format.

Bit-exact: the four MX copies of the packed weights (codes and E8M0 scales
of each GEMM's contraction-contiguous layout, read through
moe_packed_pointers) against the oracle's quantiser of the same
arrangement; routing, layout and the dispatched rows.  Floating point: the
whole layer, forward and backward, within the MXFP8 tolerance 4e-2 of each
tensor's maximum (the oracle quantises the weights the same way, so only
accumulation order and the re-quantised intermediates differ), small layers
in the staged schedule and the Kimi-shaped share in full in the pipelined
schedule the benchmark times.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_offsets_amd as m
import oracle
import synth
from gpu_util import (Run, check_layer_mx, dev, host, logits_of, note, oracle_forward,
                      shape_of, unblock_scales)
from oracle.mx import mx_quantize
from oracle.numerics import bf16_to_f64

pytestmark = pytest.mark.gpu

FMTS = ["e2m1", "e2m3", "e3m2"]


@pytest.fixture(scope="module", autouse=True)
def _built():
    from mixture_experts_layer_offsets_amd import _lib
    if not __import__("os").path.exists(_lib.LIB_PATH):
        from mixture_experts_layer_offsets_amd import build
        build.build(verbose=False)
    m.load()


def _interleave_rows(g, u):
    """Gate and up [E][X][I] -> [E][2I][X]: rows 64b .. 64b+31 are gate
    columns 32b .., the next 32 up columns (the packed gate/up layout)."""
    E, X, I = g.shape
    out = np.empty((E, 2 * I, X), g.dtype)
    for b in range(I // 32):
        out[:, 64 * b:64 * b + 32] = np.swapaxes(g[:, :, 32 * b:32 * b + 32], 1, 2)
        out[:, 64 * b + 32:64 * b + 64] = np.swapaxes(u[:, :, 32 * b:32 * b + 32], 1, 2)
    return out


def _pack(codes, fmt):
    """Codes [rows][K] (one per byte) -> the library's byte layout."""
    if fmt == "e4m3":
        return codes
    rows, K = codes.shape
    c = codes.astype(np.uint64).reshape(rows, K // 32, 32)
    W = 4 if fmt == "e2m1" else 6
    acc = [[0] * (K // 32) for _ in range(rows)]
    for p in range(32):
        for r in range(rows):
            for b in range(K // 32):
                acc[r][b] |= int(c[r, b, p]) << (W * p)
    nbytes = 16 if fmt == "e2m1" else 24
    slot = 16 if fmt == "e2m1" else 32
    out = np.zeros((rows, K // 32, slot), np.uint8)
    for r in range(rows):
        for b in range(K // 32):
            out[r, b, :nbytes] = np.frombuffer(acc[r][b].to_bytes(nbytes, "little"), np.uint8)
    return out.reshape(rows, -1)


@pytest.mark.parametrize("fmt", ["e4m3"] + FMTS)
def test_packed_weight_codes_bit_exact(fmt):
    w = synth.custom(T=16, H=256, E=2, k=2, I=128, routing="supplied", mx=True, wfmt=fmt,
                     seed=3)
    note(f"packed weights {fmt}: E={w.E} H={w.H} I={w.I}")
    inp = synth.make_inputs(w)
    layer = m.MoeLayer(shape_of(w))
    layer.prepare(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]))
    torch.cuda.synchronize()
    E, H, I = w.E, w.H, w.I
    g, u, d = (bf16_to_f64(inp[n]) for n in ("w_gate", "w_up", "w_down"))
    copies = {
        "gate_up": _interleave_rows(g, u),                               # [E][2I][H]
        "down": np.swapaxes(d, 1, 2),                                     # [E][H][I]
        "down_t": d,                                                      # [E][I][H]
    }
    # gate_up_t: [E][H][2I], the interleave along 2I
    gt = np.empty((E, H, 2 * I))
    for b in range(I // 32):
        gt[:, :, 64 * b:64 * b + 32] = g[:, :, 32 * b:32 * b + 32]
        gt[:, :, 64 * b + 32:64 * b + 64] = u[:, :, 32 * b:32 * b + 32]
    copies["gate_up_t"] = gt
    half = fmt == "e2m1"
    for name, arr in copies.items():
        rows, K = arr.shape[0] * arr.shape[1], arr.shape[2]
        codes, scales = mx_quantize(arr.reshape(rows, K), axis=1, fmt=fmt)
        want = _pack(codes, fmt)
        got = host(layer.packed_tensor(name, (rows, K // 2 if half else K)))
        assert np.array_equal(got, want), f"{fmt} {name}: codes differ"
        gs = unblock_scales(host(layer.packed_tensor(name + "_scale", (rows * K // 32,))),
                            rows, K)
        assert np.array_equal(gs, scales), f"{fmt} {name}: scales differ"
    assert m.moe_packed_pointers(layer.shape, layer.packed)["fmt"] == \
        {"e4m3": 0, "e2m3": 2, "e3m2": 3, "e2m1": 4}[fmt]


CASES = {
    "router-shared": dict(T=512, H=512, E=16, k=4, I=256, shared_I=256, routing="router",
                          router_std=1 / np.sqrt(512), hot_experts=2, hot_bias=1.0, seed=3),
    "supplied-dup": dict(T=700, H=768, E=6, k=8, I=384, zipf_s=1.2, routing="supplied", seed=7),
}


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("case", list(CASES))
def test_layer_low_precision_experts(fmt, case):
    w = synth.custom(mx=True, wfmt=fmt, **CASES[case])
    note(f"layer {case} weights {fmt}: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I}")
    run = Run(w)
    fw = oracle_forward(run.inp, w, logits_of(run))
    bw = oracle.backward(run.inp, fw)
    check_layer_mx(run, fw, bw)


def test_kimi_shape_fp4_experts_in_full():
    w = synth.workload("kimi-mx", wfmt="e2m1")
    note("full-size kimi-mx with FP4 E2M1 expert weights, pipelined schedule")
    sc = m.MoeSched()
    sc.schedule = m.MOE_SCHED_PIPELINED
    run = Run(w, synth.make_inputs(w, threads=16), sched=sc)
    fw = oracle_forward(run.inp, w, logits_of(run))
    bw = oracle.backward(run.inp, fw)
    check_layer_mx(run, fw, bw)
