"""The expert GEMMs' workgroup -> tile orders, checked on the host.

tests/tile_order_check.cpp compiles the library's own order functions
(mixture_experts_layer_offsets_amd/csrc/tile_order.h) with g++ and checks,
over the Kimi-, mid- and DeepSeek-shaped tile counts and small, odd and
partial-round ones: both orders are bijections from workgroups onto tiles
(every tile computed exactly once); the row GEMMs' order hands each XCD's
32 workgroups of a full round a 4 x 8 block of tiles; the weight gradients'
XCD-major order keeps every group on one XCD.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_tile_orders(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "tile_order_check")
    subprocess.run([gxx, "-O2", "-std=c++17", "-Wall", "-Werror", "-o", exe,
                    os.path.join(HERE, "tile_order_check.cpp")], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout[-4000:]
    assert r.stdout.strip() == "ok"
