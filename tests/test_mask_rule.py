"""Host check of the mask block tests (csrc/mask.h), CPU only.

tests/host/mask_check.cpp includes the local-window + global-token rule the
masked kernels run and checks, by brute force over every block of small
squares and over the kernels' aligned and ragged block shapes, that the
block-skip test `any` is exact and that the mask-free test `all` never
holds for a block with a hidden pair.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_mask_block_tests_host_check(tmp_path):
    exe = str(tmp_path / "mask_check")
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-Werror", "-o", exe,
                    os.path.join(ROOT, "tests", "host", "mask_check.cpp")],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok "), r.stdout
    assert int(r.stdout.split()[1]) > 1000000
