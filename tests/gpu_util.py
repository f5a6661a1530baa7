"""Helpers of the GPU parity tests: device copies, bf16 decoding, tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

import mixture_experts_layer_offsets_amd as m
from oracle.numerics import bf16_to_f64

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


def shape_of(w, dtype=m.MOE_BF16):
    return m.Shape(w.T, w.H, w.E, w.k, w.I, w.shared_I, dtype)


class Run:
    """Inputs of a workload on the device plus one forward (+ backward) pass."""

    def __init__(self, w, inp=None, backward=True):
        self.w = w
        self.inp = inp if inp is not None else __import__("synth").make_inputs(w)
        inp = self.inp
        self.shape = shape_of(w, m.MOE_MXFP8 if w.mx else m.MOE_BF16)
        self.layer = m.MoeLayer(self.shape)
        self.layer.prepare(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]),
                           dev(inp["ws_gate"]), dev(inp["ws_up"]), dev(inp["ws_down"]))
        self.x = dev(inp["x"])
        self.wr = dev(inp["w_router"])
        self.bias = dev(inp["bias"])
        self.idx = dev(inp["topk_idx"])
        self.tw = dev(inp["topk_w"])
        self.out = self.layer.forward(self.x, w_router=self.wr, bias=self.bias,
                                      topk_idx=self.idx, topk_w=self.tw)
        self.grads = None
        if backward:
            self.dout = dev(inp["dout"])
            self.grads = self.layer.backward(self.dout, self.x, w_router=self.wr)
        torch.cuda.synchronize()

    def saved(self, name, dtype, shape):
        return self.layer.saved_tensor(name, dtype, shape)
