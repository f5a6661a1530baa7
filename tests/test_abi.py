"""The C ABI: libmoe.so loads and exports every entry point include/moe.h
declares, the binding covers exactly those, and host-side checks (sizes,
argument validation) behave as documented.  No test here launches a kernel:
every validation case returns before the library touches the device.
"""
import ctypes
import dataclasses
import os
import re

import pytest

import mixture_experts_layer_offsets_amd as m
from mixture_experts_layer_offsets_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^[A-Za-z_][\w \*]*?\b(moe_\w+)\s*\(", text, flags=re.M))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from mixture_experts_layer_offsets_amd import build
        build.build(verbose=False)
    return _lib.load()


def test_header_declares_the_layer_calls():
    names = declared_functions()
    for n in ("moe_route", "moe_layout", "moe_dispatch", "moe_expert_ffn", "moe_combine",
              "moe_layer_fwd", "moe_layer_bwd", "moe_workspace_bytes", "moe_strerror"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(lib, n), n
    assert names == set(_lib.SIGNATURES), names ^ set(_lib.SIGNATURES)


def declared_arity():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    out = {}
    for name, params in re.findall(r"\b(moe_\w+)\s*\(([^;{]*?)\)\s*;", text, flags=re.S):
        params = params.strip()
        out[name] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_argument_counts_match_header():
    ar = declared_arity()
    assert set(ar) == set(_lib.SIGNATURES)
    for n, (_, args) in _lib.SIGNATURES.items():
        assert len(args) == ar[n], (n, len(args), ar[n])


def test_struct_layouts_match_header():
    text = open(HEADER).read()
    for cname, pyt in (("moe_shape", _lib.MoeShape), ("moe_sched", _lib.MoeSched),
                       ("moe_saved_view", _lib.MoeSavedView),
                       ("moe_work_view", _lib.MoeWorkView),
                       ("moe_packed_view", _lib.MoePackedView)):
        body = re.search(r"typedef struct %s \{(.*?)\} %s;" % (cname, cname), text, re.S).group(1)
        body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
        fields = []
        for decl in body.split(";")[:-1]:
            fp = re.search(r"\(\s*\*\s*(\w+)\s*\)", decl)       # function pointer
            fields.append(fp.group(1) if fp else re.findall(r"\w+", decl)[-1])
        assert fields == [f for f, _ in pyt._fields_], cname


def test_sizes(lib):
    kimi = m.Shape(2048, 7168, 6, 8, 2048)
    ws, sv, pk = (m.moe_workspace_bytes(kimi), m.moe_saved_bytes(kimi),
                  m.moe_packed_weight_bytes(kimi))
    R, H, I, E = 2048 * 8, 7168, 2048, 6
    assert sv >= R * H * 2 * 2 + R * 3 * I * 2       # x_perm, y, g|u, a
    assert ws >= R * H * 2 * 2 + R * 2 * I * 2       # dY, dX, dh
    assert pk >= 4 * 3 * E * H * I // 2 * 2          # four bf16 copies of 3 E H I / 2 ... lower bound
    for v in (ws, sv, pk):
        assert v % 256 == 0
    bad = m.Shape(0, 7168, 6, 8, 2048)
    assert m.moe_workspace_bytes(bad) == 0
    assert m.moe_saved_bytes(m.Shape(16, 100, 4, 2, 64)) == 0      # H not a multiple of 64
    assert m.moe_packed_weight_bytes(m.Shape(16, 64, 2000, 2, 64)) == 0  # E > 1024


def _rc(fn, *args):
    return fn(*args)


def test_argument_validation_returns_codes(lib):
    s = ctypes.byref(m.Shape(64, 128, 8, 2, 64).c())
    # NULL required pointers
    assert lib.moe_route(s, None, None, None, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch(s, None, None, None, None, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(s, None, None, None, None, None, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_fwd(s, None, None, None, None, None, None, None, None, None, None, 0,
                             None) == _lib.MOE_ERR_INVALID_ARG
    # a workspace that is too small (pointer is never dereferenced on this path)
    fake = 1 << 40
    assert lib.moe_layout(s, fake, fake, fake, fake, fake, fake, 16, None) == \
        _lib.MOE_ERR_WORKSPACE
    # both a router and supplied routing
    assert lib.moe_layer_fwd(s, None, fake, fake, None, fake, fake, fake, fake, fake, fake,
                             1 << 40, None) == _lib.MOE_ERR_INVALID_ARG
    # k > E when routing from logits
    s2 = ctypes.byref(m.Shape(64, 128, 4, 6, 64).c())
    assert lib.moe_route(s2, fake, fake, fake, None) == _lib.MOE_ERR_INVALID_ARG
    # shapes outside the kernels' limits
    s3 = ctypes.byref(m.Shape(64, 96, 4, 2, 64).c())
    assert lib.moe_route(s3, fake, fake, fake, None) == _lib.MOE_ERR_UNSUPPORTED
    s4 = ctypes.byref(m.Shape(64, 128, 4, 17, 64).c())
    assert lib.moe_layout(s4, fake, fake, fake, fake, fake, fake, 1 << 40, None) == \
        _lib.MOE_ERR_UNSUPPORTED
    assert lib.moe_route(None, fake, fake, fake, None) == _lib.MOE_ERR_INVALID_ARG


def test_strerror(lib):
    assert m.moe_strerror(0) == "ok"
    assert "workspace" in m.moe_strerror(_lib.MOE_ERR_WORKSPACE)
    assert m.moe_strerror(12345) == "unknown error"


def test_mx_sizes_and_shape_rules(lib):
    """MXFP8 needs H, I and the shared I in multiples of 128; its buffers add
    the E4M3 codes and E8M0 scales to the bf16 ones."""
    bf = m.Shape(2048, 7168, 6, 8, 2048)
    mx = m.Shape(2048, 7168, 6, 8, 2048, 0, m.MOE_MXFP8)
    R, H, I, E = 2048 * 8, 7168, 2048, 6
    assert m.moe_saved_bytes(mx) >= m.moe_saved_bytes(bf) + R * (H + I) * 33 // 32
    assert m.moe_workspace_bytes(mx) >= m.moe_workspace_bytes(bf) + R * (H + 2 * I) * 33 // 32
    assert m.moe_packed_weight_bytes(mx) >= \
        m.moe_packed_weight_bytes(bf) + 2 * 3 * E * H * I * 33 // 32
    assert m.moe_workspace_bytes(m.Shape(64, 256, 8, 2, 128, 0, m.MOE_MXFP8)) > 0
    # the MX operands' 32-bit descriptor limits: padded routed rows Rp =
    # R + 127 E (to 128) below 2^23, Rp * max(H, 2I) below 2^36 and
    # E * H * I below 2^35; the same shapes in bf16 are accepted
    rp_max = m.Shape((1 << 20) - 256, 128, 8, 8, 128, 0, m.MOE_MXFP8)  # Rp = 2^23 - 1024
    assert m.moe_workspace_bytes(rp_max) > 0
    for big in (m.Shape(1 << 20, 128, 8, 8, 128, 0, m.MOE_MXFP8),         # Rp >= 2^23
                m.Shape(1 << 19, 4096, 8, 8, 8192, 0, m.MOE_MXFP8),       # Rp * 2I >= 2^36
                m.Shape(64, 16384, 1024, 2, 4096, 0, m.MOE_MXFP8)):       # E H I >= 2^35
        assert m.moe_workspace_bytes(big) == 0, big
        assert lib.moe_route(ctypes.byref(big.c()), 1 << 40, 1 << 40, 1 << 40, None) == \
            _lib.MOE_ERR_UNSUPPORTED
        assert m.moe_workspace_bytes(dataclasses.replace(big, dtype=m.MOE_BF16)) > 0
    for bad in (m.Shape(64, 192, 8, 2, 128, 0, m.MOE_MXFP8),
                m.Shape(64, 256, 8, 2, 192, 0, m.MOE_MXFP8),
                m.Shape(64, 256, 8, 2, 128, 64, m.MOE_MXFP8)):
        assert m.moe_workspace_bytes(bad) == 0
        assert lib.moe_route(ctypes.byref(bad.c()), 1 << 40, 1 << 40, 1 << 40, None) == \
            _lib.MOE_ERR_UNSUPPORTED


def test_megakernel_request_is_refused(lib):
    """The persistent forward is switched off: asking for it returns
    MOE_ERR_UNSUPPORTED before any device work."""
    s = ctypes.byref(m.Shape(64, 128, 8, 2, 64).c())
    sched = m.MoeSched()
    sched.schedule = 1
    fake = 1 << 40
    assert lib.moe_layer_fwd(s, ctypes.byref(sched), fake, None, None, fake, fake, fake, fake,
                             fake, fake, 1 << 40, None) == _lib.MOE_ERR_UNSUPPORTED


def test_schedule_validation(lib):
    """An unknown schedule and a negative CU count for the pipelined schedule
    are rejected before any device work (forward and backward)."""
    s = ctypes.byref(m.Shape(64, 128, 8, 2, 64).c())
    fake = 1 << 40
    for mode, cus in ((7, 0), (-1, 0), (m.MOE_SCHED_PIPELINED, -4)):
        sched = m.MoeSched()
        sched.schedule = mode
        sched.comm_cus = cus
        assert lib.moe_layer_fwd(s, ctypes.byref(sched), fake, None, None, fake, fake, fake, fake,
                                 fake, fake, 1 << 40, None) == _lib.MOE_ERR_INVALID_ARG
        assert lib.moe_layer_bwd(s, ctypes.byref(sched), fake, fake, None, fake, fake, fake, None,
                                 fake, fake, fake, None, None, fake, 1 << 40,
                                 None) == _lib.MOE_ERR_INVALID_ARG


def test_decode_argument_validation(lib):
    """moe_decode_fwd: MXFP8 shapes are refused; routing must be either the
    router or supplied indices and weights; k > E needs supplied routing."""
    fake = 1 << 40
    mx = ctypes.byref(m.Shape(4, 256, 8, 2, 128, 0, m.MOE_MXFP8).c())
    assert lib.moe_decode_fwd(mx, fake, None, None, fake, fake, fake, fake, fake, 1 << 40,
                              None) == _lib.MOE_ERR_UNSUPPORTED
    s = ctypes.byref(m.Shape(4, 256, 8, 2, 128).c())
    # both a router and supplied routing
    assert lib.moe_decode_fwd(s, fake, fake, None, fake, fake, fake, fake, fake, 1 << 40,
                              None) == _lib.MOE_ERR_INVALID_ARG
    # neither
    assert lib.moe_decode_fwd(s, fake, None, None, None, None, fake, fake, fake, 1 << 40,
                              None) == _lib.MOE_ERR_INVALID_ARG
    # indices without weights
    assert lib.moe_decode_fwd(s, fake, None, None, fake, None, fake, fake, fake, 1 << 40,
                              None) == _lib.MOE_ERR_INVALID_ARG
    # router with k > E
    big_k = ctypes.byref(m.Shape(4, 256, 8, 9, 128).c())
    assert lib.moe_decode_fwd(big_k, fake, fake, None, None, None, fake, fake, fake, 1 << 40,
                              None) == _lib.MOE_ERR_INVALID_ARG
    # workspace too small
    assert lib.moe_decode_fwd(s, fake, None, None, fake, fake, fake, fake, fake, 16,
                              None) == _lib.MOE_ERR_WORKSPACE


def test_workspace_pointers(lib):
    """The backward's row intermediates lie inside the workspace, disjoint,
    at the sizes the header states."""
    shape = m.Shape(100, 256, 6, 4, 128)
    base = 1 << 40
    nbytes = _lib.moe_workspace_bytes(shape)
    view = _lib.MoeWorkView()
    assert lib.moe_workspace_pointers(ctypes.byref(shape.c()), base,
                                      ctypes.byref(view)) == _lib.MOE_OK
    R, H, I = 100 * 4, 256, 128
    spans = sorted([(view.dy, R * H * 2), (view.dh, R * 2 * I * 2), (view.dx_rows, R * H * 2)])
    for (p, n), (q, _) in zip(spans, spans[1:]):
        assert p + n <= q
    for p, n in spans:
        assert base <= p and p + n <= base + nbytes
    bad = m.Shape(0, 256, 6, 4, 128)
    assert lib.moe_workspace_pointers(ctypes.byref(bad.c()), base,
                                      ctypes.byref(view)) == _lib.MOE_ERR_INVALID_ARG
    assert view.dy is None and view.dh is None


def test_layout_noalloc_refuses_oversized_shapes_before_any_device_work(lib):
    """Its scratch is a 4 MiB static array: a shape needing more is refused
    with MOE_ERR_WORKSPACE before any HIP call (so this runs without a GPU)."""
    big = ctypes.byref(m.Shape(1 << 19, 64, 1024, 8, 64).c())     # 16 MiB of chunk counts
    fake = 1 << 40
    assert lib.moe_layout_noalloc(big, fake, fake, fake, fake, fake, None) == \
        _lib.MOE_ERR_WORKSPACE
    assert lib.moe_layout_noalloc(big, None, fake, fake, fake, fake, None) == \
        _lib.MOE_ERR_INVALID_ARG
