"""Build libcpattn.so in-tree with hipcc for gfx950.

Usage: ``python -m long_sequence_bidirectional_amd.build`` (or ``build()``).
The library is always rebuilt when this runs.
"""
from __future__ import annotations

import os
import subprocess
import sys
import time

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libcpattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["api.hip", "attn_fwd_bf16.hip", "attn_fwd_f32.hip", "merge.hip", "relayout.hip"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-shared", "-fvisibility=hidden",
    # No packed-fp32 instructions anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False, extra_flags=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = [HIPCC, *FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"), "-o", tmp, *srcs]
    t0 = time.time()
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        noise = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if noise:
            sys.stderr.write("\n".join(noise) + "\n")
        print(f"built {LIB_PATH} in {time.time() - t0:.1f}s")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
