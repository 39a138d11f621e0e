"""bench.py's command line, checked without a GPU.

The benchmark measures one GPU: asked for more it must stop with a message and a
non-zero status before touching a device, and its help must list the flags the
timing contract uses.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = run("--gpus", n, "--steps", "1", "--warmup", "0")
        assert r.returncode == 2
        assert "one GPU" in r.stderr
        assert r.stdout == ""          # no JSON line for a run that did not happen


def test_help_lists_the_timing_flags():
    r = run("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--no-cpu-baseline", "--cpu-seconds", "--traffic"):
        assert flag in r.stdout
