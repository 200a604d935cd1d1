"""Builds libfa.so (the HIP kernels and the C ABI of include/fa.h) for gfx950.

    python -m transformer_attention_07_amd.build

hipcc cross-compiles for gfx950 without a GPU.  Packed-fp32 instruction
selection is switched off for device code (-packed-fp32-ops); the host pass
reports that it does not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", "fa_fwd.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in VGPRs: the softmax and the rescale read them
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def build(out: str = LIBRARY, extra=(), verbose: bool = False) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, f"-I{INCLUDE}", "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode})")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
