"""ctypes binding of libmoe.so: the C entry points under the same names.

Argument marshalling only.  Tensors are torch tensors on the current HIP
device (PyTorch supplies device memory and streams; every step of the layer
runs in libmoe's kernels).  A missing library raises at import of the first
call -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4
MOE_ERR_DEVICE_TIMEOUT = 5
MOE_BF16 = 0
MOE_MXFP8 = 1
MOE_MXFP8_W4 = 2        # MXFP8 activations, FP4 E2M1 expert weights
MOE_MXFP8_W6 = 3        # MXFP8 activations, FP6 E2M3 expert weights
MOE_MXFP8_W6E3M2 = 4    # MXFP8 activations, FP6 E3M2 expert weights
# expert-weight element format of each MX datatype (the oracle's names)
WEIGHT_FORMAT = {MOE_MXFP8: "e4m3", MOE_MXFP8_W4: "e2m1", MOE_MXFP8_W6: "e2m3",
                 MOE_MXFP8_W6E3M2: "e3m2"}
MOE_SCHED_STAGED = 0
MOE_SCHED_PERSISTENT = 1
MOE_SCHED_PIPELINED = 2

c_void_p = ctypes.c_void_p
c_size_t = ctypes.c_size_t
c_int = ctypes.c_int


class MoeShape(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


STAGE_HOOK = ctypes.CFUNCTYPE(None, c_void_p, ctypes.c_int32)


class MoeSched(ctypes.Structure):
    _fields_ = [("minibatch_rows", ctypes.c_int32), ("ring_slots", ctypes.c_int32),
                ("comm_cus", ctypes.c_int32), ("schedule", ctypes.c_int32),
                ("stage_events", ctypes.POINTER(c_void_p)), ("n_stage_events", ctypes.c_int32),
                ("watchdog_us", ctypes.c_int32), ("mx_wgrad", ctypes.c_int32),
                ("stage_hook", STAGE_HOOK), ("stage_hook_user", c_void_p),
                ("kernel_stamps", c_void_p)]


class MoeSavedView(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in (
        "topk_idx", "topk_w", "logits", "counts", "offsets", "perm", "inv_perm",
        "x_perm", "x_scale", "x_hat", "gu", "act", "act_q", "act_scale", "y", "y_shared")]


# name -> (restype, argtypes); keep in the order of include/moe.h
SIGNATURES = {
    "moe_workspace_bytes": (c_size_t, [c_void_p]),
    "moe_saved_bytes": (c_size_t, [c_void_p]),
    "moe_packed_weight_bytes": (c_size_t, [c_void_p]),
    "moe_prepare_weights": (c_int, [c_void_p] + [c_void_p] * 6 + [c_void_p, c_void_p]),
    "moe_router_logits": (c_int, [c_void_p] + [c_void_p] * 4 + [c_void_p, c_size_t, c_void_p]),
    "moe_route": (c_int, [c_void_p] * 4 + [c_void_p]),
    "moe_layout": (c_int, [c_void_p] * 6 + [c_void_p, c_size_t, c_void_p]),
    "moe_layout_noalloc": (c_int, [c_void_p] * 6 + [c_void_p]),
    "moe_dispatch": (c_int, [c_void_p] * 5 + [c_void_p]),
    "moe_expert_ffn": (c_int, [c_void_p] * 6 + [c_void_p, c_size_t, c_void_p]),
    "moe_combine": (c_int, [c_void_p] * 6 + [c_void_p]),
    "moe_layer_fwd": (c_int, [c_void_p] * 10 + [c_void_p, c_size_t, c_void_p]),
    "moe_layer_bwd": (c_int, [c_void_p] * 14 + [c_void_p, c_size_t, c_void_p]),
    "moe_decode_fwd": (c_int, [c_void_p] * 8 + [c_void_p, c_size_t, c_void_p]),
    "moe_saved_pointers": (c_int, [c_void_p, c_void_p, c_void_p]),
    "moe_packed_pointers": (c_int, [c_void_p, c_void_p, c_void_p]),
    "moe_workspace_pointers": (c_int, [c_void_p, c_void_p, c_void_p]),
    "moe_read_status": (c_int, [c_void_p, c_void_p, c_void_p]),
    "moe_strerror": (ctypes.c_char_p, [c_int]),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load libmoe.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run `python -m "
                               "mixture_experts_layer_offsets_amd.build` first")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = load().moe_strerror(code).decode()
        super().__init__(f"{where}: libmoe error {code} ({msg})")


@dataclass(frozen=True)
class Shape:
    tokens: int
    hidden: int
    experts: int
    top_k: int
    inter: int
    shared_inter: int = 0
    dtype: int = MOE_BF16

    def c(self) -> MoeShape:
        return MoeShape(self.tokens, self.hidden, self.experts, self.top_k, self.inter,
                        self.shared_inter, self.dtype)


def _p(t):
    """Pointer of a torch tensor (or None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _ck(rc: int, where: str):
    if rc != MOE_OK:
        raise MoeError(rc, where)


def _shape(shape) -> ctypes.Structure:
    s = shape.c() if isinstance(shape, Shape) else shape
    return ctypes.byref(s)


def moe_workspace_bytes(shape) -> int:
    return load().moe_workspace_bytes(_shape(shape))


def moe_saved_bytes(shape) -> int:
    return load().moe_saved_bytes(_shape(shape))


def moe_packed_weight_bytes(shape) -> int:
    return load().moe_packed_weight_bytes(_shape(shape))


def moe_prepare_weights(shape, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, packed,
                        stream=None):
    _ck(load().moe_prepare_weights(_shape(shape), _p(w_gate), _p(w_up), _p(w_down),
                                   _p(ws_gate), _p(ws_up), _p(ws_down), _p(packed),
                                   _stream(stream)), "moe_prepare_weights")


def moe_router_logits(shape, x, w_router, bias, logits, ws, stream=None):
    _ck(load().moe_router_logits(_shape(shape), _p(x), _p(w_router), _p(bias), _p(logits),
                                 _p(ws), ws.numel() * ws.element_size(), _stream(stream)),
        "moe_router_logits")


def moe_route(shape, logits, topk_idx, topk_w, stream=None):
    _ck(load().moe_route(_shape(shape), _p(logits), _p(topk_idx), _p(topk_w), _stream(stream)),
        "moe_route")


def moe_layout(shape, topk_idx, counts, offsets, perm, inv_perm, ws, stream=None):
    _ck(load().moe_layout(_shape(shape), _p(topk_idx), _p(counts), _p(offsets), _p(perm),
                          _p(inv_perm), _p(ws), ws.numel() * ws.element_size(),
                          _stream(stream)), "moe_layout")


def moe_layout_noalloc(shape, topk_idx, counts, offsets, perm, inv_perm, stream=None):
    _ck(load().moe_layout_noalloc(_shape(shape), _p(topk_idx), _p(counts), _p(offsets),
                                  _p(perm), _p(inv_perm), _stream(stream)), "moe_layout_noalloc")


def moe_dispatch(shape, x, perm, x_perm, x_scale=None, stream=None):
    _ck(load().moe_dispatch(_shape(shape), _p(x), _p(perm), _p(x_perm), _p(x_scale),
                            _stream(stream)), "moe_dispatch")


def moe_expert_ffn(shape, x_perm, x_scale, offsets, packed, y, ws, stream=None):
    _ck(load().moe_expert_ffn(_shape(shape), _p(x_perm), _p(x_scale), _p(offsets), _p(packed),
                              _p(y), _p(ws), ws.numel() * ws.element_size(), _stream(stream)),
        "moe_expert_ffn")


def moe_combine(shape, y, topk_w, inv_perm, y_shared, out, stream=None):
    _ck(load().moe_combine(_shape(shape), _p(y), _p(topk_w), _p(inv_perm), _p(y_shared),
                           _p(out), _stream(stream)), "moe_combine")


def _sched(sched):
    if sched is None:
        return None
    return ctypes.byref(sched)


def moe_layer_fwd(shape, sched, x, w_router, bias, topk_idx_in, topk_w_in, packed, out, saved,
                  ws, stream=None):
    _ck(load().moe_layer_fwd(_shape(shape), _sched(sched), _p(x), _p(w_router), _p(bias),
                             _p(topk_idx_in), _p(topk_w_in), _p(packed), _p(out), _p(saved),
                             _p(ws), ws.numel() * ws.element_size(), _stream(stream)),
        "moe_layer_fwd")


def moe_layer_bwd(shape, sched, dout, x, w_router, saved, packed, dx, dw_router, dw_gate, dw_up,
                  dw_down, dws, dtopk_w, ws, stream=None):
    _ck(load().moe_layer_bwd(_shape(shape), _sched(sched), _p(dout), _p(x), _p(w_router),
                             _p(saved), _p(packed), _p(dx), _p(dw_router), _p(dw_gate),
                             _p(dw_up), _p(dw_down), _p(dws), _p(dtopk_w), _p(ws),
                             ws.numel() * ws.element_size(), _stream(stream)), "moe_layer_bwd")


def moe_decode_fwd(shape, x, w_router, bias, topk_idx_in, topk_w_in, packed, out, ws,
                   stream=None):
    _ck(load().moe_decode_fwd(_shape(shape), _p(x), _p(w_router), _p(bias), _p(topk_idx_in),
                              _p(topk_w_in), _p(packed), _p(out), _p(ws),
                              ws.numel() * ws.element_size(), _stream(stream)), "moe_decode_fwd")


def moe_saved_pointers(shape, saved) -> dict:
    view = MoeSavedView()
    _ck(load().moe_saved_pointers(_shape(shape), _p(saved), ctypes.byref(view)),
        "moe_saved_pointers")
    return {n: getattr(view, n) for n, _ in MoeSavedView._fields_}


class MoePackedView(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in (
        "gate_up", "gate_up_scale", "down", "down_scale", "gate_up_t", "gate_up_t_scale",
        "down_t", "down_t_scale")] + [("fmt", ctypes.c_int32)]


def moe_packed_pointers(shape, packed) -> dict:
    view = MoePackedView()
    _ck(load().moe_packed_pointers(_shape(shape), _p(packed), ctypes.byref(view)),
        "moe_packed_pointers")
    return {n: getattr(view, n) for n, _ in MoePackedView._fields_}


class MoeWorkView(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("dy", "dh", "dx_rows", "dec_logits", "dec_topk_idx",
                                        "dec_topk_w", "dy_codes", "dy_scales", "dh_codes",
                                        "dh_scales")]


def moe_workspace_pointers(shape, ws) -> dict:
    view = MoeWorkView()
    _ck(load().moe_workspace_pointers(_shape(shape), _p(ws), ctypes.byref(view)),
        "moe_workspace_pointers")
    return {n: getattr(view, n) for n, _ in MoeWorkView._fields_}


def moe_read_status(ws, stream=None) -> int:
    st = ctypes.c_int32(-1)
    _ck(load().moe_read_status(_p(ws), ctypes.byref(st), _stream(stream)), "moe_read_status")
    return st.value


def moe_strerror(code: int) -> str:
    return load().moe_strerror(code).decode()
