"""Caller-side buffers of one MoE layer, allocated with torch, driven via libmoe."""
from __future__ import annotations

import torch

from . import _lib
from ._lib import Shape


def _empty_bytes(n: int, device) -> torch.Tensor:
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)


class MoeLayer:
    """Workspace, forward->backward context and packed weights of one layer.

    bf16 tensors are torch.int16 tensors holding bf16 bit patterns (or
    torch.bfloat16 tensors); every call enqueues on the current stream.
    """

    def __init__(self, shape: Shape, device="cuda"):
        self.shape = shape
        self.device = torch.device(device)
        self.ws = _empty_bytes(_lib.moe_workspace_bytes(shape), self.device)
        self.saved = _empty_bytes(_lib.moe_saved_bytes(shape), self.device)
        self.packed = _empty_bytes(_lib.moe_packed_weight_bytes(shape), self.device)

    # -- weights
    def prepare(self, w_gate, w_up, w_down, ws_gate=None, ws_up=None, ws_down=None):
        _lib.moe_prepare_weights(self.shape, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
                                 self.packed)

    # -- forward / backward
    def forward(self, x, w_router=None, bias=None, topk_idx=None, topk_w=None, sched=None,
                out=None):
        s = self.shape
        if out is None:
            out = torch.empty((s.tokens, s.hidden), dtype=torch.int16, device=self.device)
        _lib.moe_layer_fwd(s, sched, x, w_router, bias, topk_idx, topk_w, self.packed, out,
                           self.saved, self.ws)
        return out

    def decode(self, x, w_router=None, bias=None, topk_idx=None, topk_w=None, out=None):
        """Few-token inference forward (no forward context is written)."""
        s = self.shape
        if out is None:
            out = torch.empty((s.tokens, s.hidden), dtype=torch.int16, device=self.device)
        _lib.moe_decode_fwd(s, x, w_router, bias, topk_idx, topk_w, self.packed, out, self.ws)
        return out

    def backward(self, dout, x, w_router=None, sched=None, grads=None):
        s = self.shape
        dev = self.device
        if grads is None:
            grads = self.grad_buffers(router=w_router is not None)
        _lib.moe_layer_bwd(s, sched, dout, x, w_router, self.saved, self.packed, grads["dx"],
                           grads.get("dw_router"), grads["dw_gate"], grads["dw_up"],
                           grads["dw_down"], grads.get("dws"), grads.get("dtopk_w"), self.ws)
        return grads

    def grad_buffers(self, router: bool) -> dict:
        s = self.shape
        dev = self.device
        f32 = dict(dtype=torch.float32, device=dev)
        g = dict(dx=torch.empty((s.tokens, s.hidden), dtype=torch.int16, device=dev),
                 dw_gate=torch.empty((s.experts, s.hidden, s.inter), **f32),
                 dw_up=torch.empty((s.experts, s.hidden, s.inter), **f32),
                 dw_down=torch.empty((s.experts, s.inter, s.hidden), **f32),
                 dtopk_w=torch.empty((s.tokens, s.top_k), **f32))
        if router:
            g["dw_router"] = torch.empty((s.hidden, s.experts), **f32)
        if s.shared_inter:
            g["dws"] = torch.empty(3 * s.hidden * s.shared_inter, **f32)
        return g

    # -- views of the forward context
    def saved_tensor(self, name: str, dtype, shape) -> torch.Tensor:
        ptr = _lib.moe_saved_pointers(self.shape, self.saved)[name]
        if not ptr:
            raise KeyError(name)
        off = ptr - self.saved.data_ptr()
        n = 1
        for d in shape:
            n *= d
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return self.saved[off:off + nbytes].view(dtype).view(*shape)

    def work_tensor(self, name: str, dtype, shape) -> torch.Tensor:
        """A view of an intermediate left in the workspace (the backward's dy,
        dh, dx_rows and, with MXFP8, dy_codes, dy_scales, dh_codes,
        dh_scales; the decode forward's dec_logits, dec_topk_idx,
        dec_topk_w), valid until the next call that uses this workspace."""
        ptr = _lib.moe_workspace_pointers(self.shape, self.ws)[name]
        if not ptr:
            raise KeyError(name)
        off = ptr - self.ws.data_ptr()
        n = 1
        for d in shape:
            n *= d
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return self.ws[off:off + nbytes].view(dtype).view(*shape)

    def packed_tensor(self, name: str, shape) -> torch.Tensor:
        """A uint8 view of one of the packed weights' MX copies or scale
        planes (moe_packed_pointers), e.g. "gate_up" or "down_t_scale"."""
        ptr = _lib.moe_packed_pointers(self.shape, self.packed)[name]
        if not ptr:
            raise KeyError(name)
        off = ptr - self.packed.data_ptr()
        n = 1
        for d in shape:
            n *= d
        return self.packed[off:off + n].view(*shape)

    def status(self) -> int:
        return _lib.moe_read_status(self.ws)
