"""Builds libfa.so (the HIP kernels and the C ABI of include/fa.h) for gfx950.

    python -m transformer_attention_07_amd.build

hipcc cross-compiles for gfx950 without a GPU.  Packed-fp32 instruction
selection is switched off for device code (-packed-fp32-ops); the host pass
reports that it does not know the feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
# (source, extra flags): each source is compiled on its own, then linked
SOURCES = [
    # keep MFMA accumulators in VGPRs: the softmax and the rescale read them
    (os.path.join(PKG, "csrc", "fa_fwd.hip"), ["-mllvm", "-amdgpu-mfma-vgpr-form"]),
    # the backward kernels keep their dK/dV/dQ accumulators in AGPRs
    (os.path.join(PKG, "csrc", "fa_bwd.hip"), []),
    # FP8 (e4m3) forward
    (os.path.join(PKG, "csrc", "fa_fp8.hip"), []),
]
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libfa.so")
# the same sources with the ring-barrier checks compiled in (include/fa_debug.h)
DEBUG_LIBRARY = os.path.join(PKG, "libfa_debug.so")
DEBUG_FLAGS = ("-DFA_DEBUG_BARRIERS=1",)
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode})")


def build(out: str = LIBRARY, extra=(), verbose: bool = False, link_extra=()) -> str:
    """Compiles every source (in parallel) and links `out`.  `extra` goes to
    each compile, `link_extra` to the link (e.g. host-only sanitizer
    flags)."""
    tmp = out + ".tmp"
    jobs = []
    for src, flags in SOURCES:
        obj = out + "." + os.path.splitext(os.path.basename(src))[0] + ".o"
        jobs.append((obj, [HIPCC, *FLAGS, *flags, *extra, f"-I{INCLUDE}", "-c", "-o", obj, src]))
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as pool:
        for f in [pool.submit(_run, cmd, verbose) for _, cmd in jobs]:
            f.result()
    objs = [obj for obj, _ in jobs]
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, "-o", tmp, *objs],
         verbose)
    for obj in objs:
        os.remove(obj)
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False) -> None:
    """The release library and the debug one, side by side."""
    with concurrent.futures.ThreadPoolExecutor(max_workers=2) as pool:
        jobs = [pool.submit(build, LIBRARY, (), verbose),
                pool.submit(build, DEBUG_LIBRARY, DEBUG_FLAGS, verbose)]
        for f in jobs:
            f.result()


if __name__ == "__main__":
    build_all(verbose=True)
    print(LIBRARY, DEBUG_LIBRARY)
