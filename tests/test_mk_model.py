"""Host model of the persistent forward's schedule (CPU).

tests/mk_model.cpp compiles the library's own schedule code
(mixture_experts_layer_offsets_amd/csrc/mk_schedule.h: the plan, both task
queues, every wait and signal) with g++ and runs it with one thread per
workgroup.  Each case must finish with every task run exactly once and no
task started before what it reads was produced (dispatched rows, gate/up
tiles of the row tile, down tiles of every row of a combined token, the
in-flight window of dispatch), also when only some workgroups are resident
at a time, with random pauses inside tasks, and at the full Kimi-shaped and
DeepSeek-V3-shaped sizes.  A lost completion signal must end the run
through the watchdog with the timeout status, every workgroup finished.

The shapes and schedules are those of the persistent kernel's GPU tests
(tests/test_gpu_megakernel.py) and of the library's defaults (minibatch 2048
rows raised to the schedule's minimum, 4 ring slots, 16 communication
workgroups, one workgroup per CU of a 256-CU device).
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mk_model.cpp")

DEFAULT = dict(MB=2048, S=4, n_comm=16, grid=256, resident=256)
SHAPES = {
    "tiny-router": dict(T=256, H=512, E=8, k=2, I=256),
    "shared-router": dict(T=512, H=512, E=16, k=4, I=192, Is=256),
    "supplied-dup": dict(T=700, H=768, E=6, k=8, I=320, zipf=1.0),
    "ragged": dict(T=777, H=320, E=5, k=3, I=192),
    "mx-supplied": dict(T=700, H=768, E=6, k=8, I=384, zipf=1.2),
}
SCHEDS = [dict(), dict(MB=256, S=1, n_comm=1), dict(MB=1000, S=2, n_comm=64),
          dict(MB=300, S=8, n_comm=8)]


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("mk_model") / "mk_model")
    subprocess.run([gxx, "-O2", "-std=c++17", "-pthread", "-Wall", "-Werror", "-o", exe, SRC],
                   check=True)
    return exe


def run(exe, timeout=120, **kw):
    args = [exe] + [f"{k}={v}" for k, v in kw.items()]
    r = subprocess.run(args, capture_output=True, text=True, timeout=timeout)
    line = (r.stdout.strip().splitlines() or [""])[-1]
    print(" ".join(args[1:]), "->", line)
    assert r.returncode == 0 and line.startswith("ok"), line + r.stderr
    return dict(kv.split("=") for kv in line.split()[1:])


@pytest.mark.parametrize("shape", sorted(SHAPES))
@pytest.mark.parametrize("si", range(len(SCHEDS)))
def test_schedule_completes_in_dependency_order(model, shape, si):
    for seed in (1, 2):
        run(model, **{**DEFAULT, **SHAPES[shape], **SCHEDS[si], "seed": seed})


@pytest.mark.parametrize("resident", [2, 17, 40])
def test_schedule_completes_with_few_resident_workgroups(model, resident):
    """Workgroups start in index order as earlier ones finish: the queue order
    needs only one communication workgroup and one more resident."""
    for shape in ("shared-router", "supplied-dup"):
        sched = dict(DEFAULT, n_comm=min(16, resident - 1), resident=resident)
        run(model, **{**sched, **SHAPES[shape], "MB": 256, "S": 2})


def test_schedule_kimi_shape(model):
    kimi = dict(T=2048, H=7168, E=6, k=8, I=2048, zipf=1.0)
    for mb in (2048, 2368, 8192):
        r = run(model, **{**DEFAULT, **kimi, "MB": mb})
        assert int(r["R"]) == 16384
    run(model, **{**DEFAULT, **kimi, "MB": 256, "S": 1, "n_comm": 1})


def test_schedule_dsv3_shape(model):
    dsv3 = dict(T=8192, H=7168, E=256, k=8, I=2048, Is=2048, zipf=0.3)
    r = run(model, timeout=300, **{**DEFAULT, **dsv3})
    assert int(r["NM"]) == 32


@pytest.mark.parametrize("resident", [256, 20])
def test_lost_signal_ends_through_the_watchdog(model, resident):
    """Minibatch 0's first dispatch signal is dropped, so the waits on it can
    never be satisfied: every workgroup must still return, through the
    watchdog, with the timeout status in the status word."""
    r = run(model, **{**DEFAULT, **SHAPES["supplied-dup"], "MB": 256, "S": 1,
                      "n_comm": 4, "resident": resident, "drop": 1, "budget_s": 0.05})
    assert int(r["status"]) == 5
