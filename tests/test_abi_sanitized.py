"""The C-ABI validation tests again, against a build whose host code carries
AddressSanitizer and UndefinedBehaviorSanitizer.

Every entry point's argument checks run on the host before any HIP call, so the
ABI tests exercise exactly that code with fake pointers and out-of-range values
(bad dtypes, directions and status codes, overflowing sizes).  Here the library is
rebuilt with the sanitizers on the host side only (each -fsanitize flag behind
-Xarch_host; the gfx950 code objects are unchanged) into a temporary directory,
never over the package's own library, and tests/test_abi.py runs in a child
interpreter with the ASan runtime preloaded ahead of whatever is preloaded already.
Any report fails the test and is printed.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from long_sequence_bidirectional_amd import build as cpbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]

CHILD = """
import sys
sys.path.insert(0, {root!r})
from long_sequence_bidirectional_amd import _lib
_lib.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", {tests!r}]))
"""


def asan_runtime():
    clang = os.path.join(os.path.dirname(os.path.realpath(cpbuild.HIPCC)), "..", "lib", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        return None
    res = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    return path if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_abi_checks_clean_under_host_asan_and_ubsan(tmp_path):
    if shutil.which(cpbuild.HIPCC) is None and not os.path.exists(cpbuild.HIPCC):
        pytest.skip("hipcc not available")
    rt = asan_runtime()
    if rt is None:
        pytest.skip("ASan runtime not found next to hipcc's clang")
    lib = cpbuild.build(extra_flags=HOST_SANITIZE, out=str(tmp_path / "libcpattn_san.so"))
    logs = str(tmp_path / "sanlog")
    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join(p for p in (rt, os.environ.get("LD_PRELOAD", "")) if p)
    env["ASAN_OPTIONS"] = f"detect_leaks=0:halt_on_error=1:log_path={logs}"
    env["UBSAN_OPTIONS"] = f"halt_on_error=1:print_stacktrace=1:log_path={logs}"
    code = CHILD.format(root=ROOT, lib=lib, tests=os.path.join(ROOT, "tests", "test_abi.py"))
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    reports = "".join(open(f).read() for f in sorted(glob.glob(logs + "*")))
    assert res.returncode == 0 and not reports, (res.stdout[-4000:] + res.stderr[-4000:] + reports[-8000:])
