"""bench.py's command line on the CPU: it refuses more than one GPU with a
message and a non-zero exit (the layer runs on one GPU; there is no
multi-GPU path), and its help text lists the options."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_help_lists_the_options():
    r = _bench("--help")
    assert r.returncode == 0
    for opt in ("--gpus", "--steps", "--warmup", "--workload"):
        assert opt in r.stdout
