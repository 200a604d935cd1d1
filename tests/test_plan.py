"""Host check of the stream-K schedule (csrc/stream_plan.h), CPU only.

tests/host/plan_check.cpp includes the schedule code that the kernels and
the host planner of fa_fwd_ws run and checks, over many shapes, compute-unit
counts and lead values, that every key tile of every query tile is computed
exactly once, that partial results go to distinct workspace slots, and that
the combine step enumerates exactly the pieces of each cut tile.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_stream_schedule_host_check(tmp_path):
    exe = str(tmp_path / "plan_check")
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-Werror",
                    f"-I{os.path.join(ROOT, 'include')}", "-o", exe,
                    os.path.join(ROOT, "tests", "host", "plan_check.cpp")],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok "), r.stdout
    assert int(r.stdout.split()[1]) > 10000
