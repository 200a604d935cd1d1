"""The debug build (libfa_debug.so, include/fa_debug.h) on the GPU: every
kernel with ring barriers, run through it, records no barrier mismatch, and
its results equal the release library's bit for bit (the checks add LDS
counters and waits, no arithmetic).  Covered: the pipelined forward on the
stream-K schedule in both layouts (pair-split 128-row tiles, 256-row tiles)
and on the one-workgroup-per-tile grid, the masked and variable-length
forwards, and the D = 64 / 128 backward with its dQ and dK/dV kernels on
both schedules and under the window mask."""
import ctypes
import math

import numpy as np
import pytest
import torch

import transformer_attention_07_amd as fa
from workloads import gen_grad_out, gen_qkv

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _log(msg):
    print(f"[debug-barriers] {msg}", flush=True)


@pytest.fixture(scope="module")
def libs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rel = fa.library()
    dbg = fa.debug_library()
    _faults(dbg)  # start from zero
    return rel, dbg


def _faults(dbg):
    n = ctypes.c_uint(0)
    assert dbg.fa_debug_barrier_faults(ctypes.byref(n), 1) == fa.FA_OK
    return n.value


def _with(lib, fn):
    saved = fa._lib
    fa._lib = lib
    try:
        out = fn()
        torch.cuda.synchronize()
    finally:
        fa._lib = saved
    return [t.cpu() for t in out]


def _same(libs, fn, what):
    rel, dbg = libs
    _log(what)
    a = _with(rel, fn)
    b = _with(dbg, fn)
    assert _faults(dbg) == 0, f"{what}: ring-barrier mismatch recorded"
    for x, y in zip(a, b):
        assert torch.equal(x, y), f"{what}: debug build differs from the release build"


def _dev(*ts):
    return [t.to(DEV) for t in ts]


@pytest.mark.parametrize("shape,split", [
    ((2, 3, 700, 700, 128), True),    # stream schedule, pair-split tiles
    ((8, 1, 1024, 1024, 64), True),   # stream schedule, 256-row tiles
    ((1, 2, 1000, 1000, 128), False),  # one workgroup per tile
])
def test_forward(libs, shape, split):
    B, H, N, _, D = shape
    q, k, v = _dev(*gen_qkv(B, H, N, N, D, seed=7000 + N, dtype="bf16"))
    _same(libs, lambda: fa.fwd(q, k, v, causal=True, split=split),
          f"fwd B{B} H{H} N{N} D{D} split={split}")


def test_masked_forward(libs):
    q, k, v = _dev(*gen_qkv(1, 2, 2048, 2048, 128, seed=7100, dtype="bf16"))
    _same(libs, lambda: fa.fwd_masked(q, k, v, 256, 16, causal=True),
          "masked fwd window 256, 16 global")


def test_varlen_forward(libs):
    lens = [300, 1000, 77, 513, 64]
    T, H, D = sum(lens), 2, 128
    q, _, _ = gen_qkv(1, H, T, 1, D, seed=7200, dtype="bf16")
    _, k, v = gen_qkv(1, H, 1, T, D, seed=7201, dtype="bf16")
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    qd, kd, vd, cud = _dev(q[0], k[0], v[0], cu)
    _same(libs, lambda: fa.fwd_varlen(qd, kd, vd, cud, cud, max(lens), causal=True),
          f"varlen fwd lens={lens}")


@pytest.mark.parametrize("shape,causal", [
    ((2, 2, 768, 768, 128), True),   # dQ and dK/dV on their stream schedules
    ((2, 128, 200, 250, 64), True),  # one workgroup per tile
    ((1, 2, 77, 333, 64), False),
])
def test_backward(libs, shape, causal):
    B, H, Nq, Nk, D = shape
    q, k, v = _dev(*gen_qkv(B, H, Nq, Nk, D, seed=7300 + Nq, dtype="bf16"))
    g = gen_grad_out(B, H, Nq, D, seed=7400 + Nq, dtype="bf16").to(DEV)
    scale = 1.0 / math.sqrt(D)
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    _same(libs, lambda: fa.bwd(q, k, v, o, lse, g, causal=causal, scale=scale,
                               grad_dtype=torch.float32),
          f"bwd B{B} H{H} Nq{Nq} Nk{Nk} D{D} causal={causal}")


@pytest.mark.parametrize("D", [64, 128])
def test_masked_backward(libs, D):
    q, k, v = _dev(*gen_qkv(1, 2, 1000, 1000, D, seed=7500 + D, dtype="bf16"))
    g = gen_grad_out(1, 2, 1000, D, seed=7600 + D, dtype="bf16").to(DEV)
    scale = 1.0 / math.sqrt(D)
    o, lse = fa.fwd_masked(q, k, v, 200, 16, causal=True, scale=scale)
    torch.cuda.synchronize()
    _same(libs, lambda: fa.bwd(q, k, v, o, lse, g, causal=True, scale=scale,
                               grad_dtype=torch.float32, window=200, nglobal=16),
          f"masked bwd D{D} window 200, 16 global")
