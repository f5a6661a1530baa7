"""moe_layout_noalloc: the layout with its scratch in the library's static
device array, against moe_layout with a caller's workspace (bit-exact), on
two calls in a row, the second with a smaller input (the array keeps the
first call's contents, which the second must not depend on), and against the
oracle's layout.  Shapes whose scratch exceeds the array are refused before
anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import mixture_experts_layer_offsets_amd as m
import oracle
import synth
from gpu_util import dev, host, note
from mixture_experts_layer_offsets_amd import _lib

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    import os
    if not os.path.exists(_lib.LIB_PATH):
        from mixture_experts_layer_offsets_amd import build
        build.build(verbose=False)
    m.load()


def _outputs(T, E, k):
    i32 = dict(dtype=torch.int32, device="cuda")
    return (torch.full((E,), -7, **i32), torch.full((E + 1,), -7, **i32),
            torch.full((T * k,), -7, **i32), torch.full((T * k,), -7, **i32))


def test_noalloc_layout_matches_layout_twice_shrinking():
    # the second call is smaller in rows and experts: the array then holds a
    # stale, larger chunk table from the first call
    for T, E, k, probs in [(20000, 256, 8, None), (1500, 6, 8, "zipf")]:
        note(f"layout_noalloc T={T} E={E} k={k}")
        p = synth._zipf_probs(E, 1.2) if probs else None
        idx, _ = synth.supplied_routing(T, E, k, seed=T + E, probs=p)
        shape = m.Shape(T, 64, E, k, 64)
        ws = torch.empty(m.moe_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
        d_idx = dev(idx)
        ref = _outputs(T, E, k)
        m.moe_layout(shape, d_idx, *ref, ws)
        got = _outputs(T, E, k)
        m.moe_layout_noalloc(shape, d_idx, *got)
        torch.cuda.synchronize()
        for name, a, b in zip(("counts", "offsets", "perm", "inv_perm"), ref, got):
            assert np.array_equal(host(a), host(b)), name
        rc, ro, rp, ri = oracle.layout(idx, E)
        assert np.array_equal(host(got[0]), rc) and np.array_equal(host(got[1]), ro)
        assert np.array_equal(host(got[2]), rp) and np.array_equal(host(got[3]), ri)


def test_noalloc_layout_refuses_oversized_shapes():
    lib = m.load()
    # 2^22 rows over 1024 experts need 4096 x 1024 chunk counts (16 MiB)
    big = ctypes.byref(m.Shape(1 << 19, 64, 1024, 8, 64).c())
    fake = 1 << 40            # never dereferenced: the call refuses first
    assert lib.moe_layout_noalloc(big, fake, fake, fake, fake, fake, None) == \
        _lib.MOE_ERR_WORKSPACE
