"""CPU check of the attention kernels' unit schedules (csrc/unit_sched.h).

The header's unit map and its grid-id-to-unit and ticket-to-unit mappings are plain host/device
arithmetic; `unit_sched_check.hip` builds them for the host only, walks the static order and
simulates persistent workgroups claiming units in random interleavings, at the bench's shapes and
at random tile counts (up to 4600 tiles, some split into pieces) on 8 to 512 resident workgroups
(or an unknown count).  In both orders every unit must run exactly once.  No GPU is used."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("sched") / "unit_sched_check")
    res = subprocess.run([HIPCC, "-O2", "-std=c++20", "--offload-host-only", "-I", os.path.join(ROOT, "include"),
                          os.path.join(HERE, "unit_sched_check.hip"), "-o", exe], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_every_unit_runs_exactly_once(checker, seed):
    res = subprocess.run([checker, str(seed), "1500"], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0 and res.stdout.strip().startswith("ok"), res.stdout + res.stderr
