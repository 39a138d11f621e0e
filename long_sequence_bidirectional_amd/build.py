"""Build libcpattn.so in-tree with hipcc for gfx950.

Usage: ``python -m long_sequence_bidirectional_amd.build`` (or ``build()``).
The library is always rebuilt when this runs.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
import time

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libcpattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["api.hip", "attn_fwd_bf16.hip", "attn_fwd_f16.hip", "attn_fwd_bf16_kt.hip", "attn_fwd_f16_kt.hip",
           "attn_fwd_f32.hip", "attn_fwd_fp8.hip", "merge.hip", "relayout.hip", "qk_norm.hip"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-shared", "-fvisibility=hidden",
    # No packed-fp32 instructions anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # The attention kernel's work claim is one lane's atomic whose result is first needed after
    # the epilogue; the wave-aggregating rewrite would wait for it on the spot.
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wno-unused-command-line-argument",
]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    return res.stderr


def build(verbose: bool = False, extra_flags=(), out: str = LIB_PATH) -> str:
    """Compile every translation unit in parallel, then link the shared library at ``out``.

    ``extra_flags`` go to every compile and to the link (e.g. host-only sanitizer flags
    for a checking build written somewhere other than the package's library)."""
    from concurrent.futures import ThreadPoolExecutor

    t0 = time.time()
    tmpdir = tempfile.mkdtemp(prefix="cpattn_build_")
    try:
        compile_flags = [f for f in FLAGS if f != "-shared"]
        jobs = []
        for src in SOURCES:
            obj = os.path.join(tmpdir, src.replace(".hip", ".o"))
            jobs.append((obj, [HIPCC, *compile_flags, *extra_flags, "-I", os.path.join(ROOT, "include"), "-c",
                               os.path.join(CSRC, src), "-o", obj]))
        workers = min(len(jobs), max(1, min(os.cpu_count() or 1, 16)))
        with ThreadPoolExecutor(max_workers=workers) as pool:
            logs = list(pool.map(lambda j: _run(j[1]), jobs))
        tmp = out + f".tmp{os.getpid()}"
        logs.append(_run([HIPCC, *FLAGS, *extra_flags, "-o", tmp, *[o for o, _ in jobs]]))
        os.replace(tmp, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    if verbose:
        noise = [l for log in logs for l in log.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if noise:
            sys.stderr.write("\n".join(noise) + "\n")
        print(f"built {out} in {time.time() - t0:.1f}s")
    return out


if __name__ == "__main__":
    build(verbose=True)
