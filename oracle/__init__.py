"""CPU oracle for the attention forward pass (ctypes wrapper around fa_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline of the benchmark may import this package.  The GPU library never
links or calls it, and it imports nothing from the GPU package.

Functions (all fp64, numpy in / numpy out):
  attention(q, k, v, scale, causal, rows=None) -> (o, lse)
      the plain two-pass definition (page "FlashAttention技术演进全景图"
      §2.1/§2.3; output conventions of "FlashAttention-2实现与优化" §3.1).
  attention_online(q, k, v, scale, causal, bq, bk) -> (o, lse)
      the pages' tiled online-softmax recurrence ("FlashAttention-2实现与优化"
      §3.1), used only to show that it reaches the two-pass result.
  attention_bwd(q, k, v, do, scale, causal, qrows=None, krows=None,
                magnitudes=False) -> (dq, dk, dv[, bq, bk, bv])
      gradients of the forward pass for an upstream gradient do of O, by the
      chain rule (the pages fix no formula for the backward pass; it is the
      derivative of the definition above), plus optional magnitude sums that
      bound rounding effects.
  attention_varlen(q, k, v, cu_q, cu_k, scale, causal) -> (o, lse)
      variable-length batches ("FlashAttention-2实现与优化" §7, ragged input
      sequences): q [H, Tq, D], k and v [H, Tk, D] hold S sequences packed
      along the token axis, sequence s at rows cu_q[s] .. cu_q[s+1] (keys
      cu_k[s] .. cu_k[s+1]); each sequence attends only to its own keys,
      with the forward definition above applied per sequence.  A sequence
      with queries but no keys gets O = 0 and L = -inf (the empty sum).
  attention_bwd_varlen(q, k, v, do, cu_q, cu_k, scale, causal)
      -> (dq, dk, dv): the gradients of attention_varlen, attention_bwd
      applied to each packed sequence (zero where a sequence has no queries
      or no keys).
  attention_masked(q, k, v, scale, causal, window, nglobal, rows=None)
      -> (o, lse): attention under a local-window + global-token mask
      ("FlashAttention-2实现与优化" §7 sparse attention; the pattern is this
      package's reading, stated in fa_oracle.c).
  attention_bwd_masked(q, k, v, do, scale, causal, window, nglobal,
                       qrows=None, krows=None, magnitudes=False)
      -> (dq, dk, dv[, bq, bk, bv]): the gradients of attention_masked (chain
      rule over the visible pairs), with the row sampling and magnitude sums
      of attention_bwd.
  threads() -> int   OpenMP threads the oracle uses.
  set_threads(n) -> int   sets them (the CPU baseline's one-core run).

Parity status: pinned by tests/test_oracle_pins.py (closed forms, invariants,
brute force, a library witness and hand-derived worked examples).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "fa_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(out: str = LIBRARY, source: str = SOURCE, extra_flags=()) -> str:
    """Compile fa_oracle.c with gcc (-O2, OpenMP, IEEE semantics kept)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", *extra_flags, "-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(path: str):
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.fa_oracle_attention.restype = ctypes.c_int
    lib.fa_oracle_attention.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64, i64,
                                        ctypes.c_double, ctypes.c_int,
                                        ctypes.POINTER(i64), i64]
    lib.fa_oracle_online.restype = ctypes.c_int
    lib.fa_oracle_online.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64, i64,
                                     ctypes.c_double, ctypes.c_int, i64, i64]
    lib.fa_oracle_attention_bwd.restype = ctypes.c_int
    lib.fa_oracle_attention_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                            i64, i64, i64, i64, i64,
                                            ctypes.c_double, ctypes.c_int,
                                            ctypes.POINTER(i64), i64,
                                            ctypes.POINTER(i64), i64]
    lib.fa_oracle_attention_masked.restype = ctypes.c_int
    lib.fa_oracle_attention_masked.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64, i64,
                                               ctypes.c_double, ctypes.c_int, i64, i64,
                                               ctypes.POINTER(i64), i64]
    lib.fa_oracle_attention_bwd_masked.restype = ctypes.c_int
    lib.fa_oracle_attention_bwd_masked.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                                   i64, i64, i64, i64, i64,
                                                   ctypes.c_double, ctypes.c_int, i64, i64,
                                                   ctypes.POINTER(i64), i64,
                                                   ctypes.POINTER(i64), i64]
    lib.fa_oracle_threads.restype = ctypes.c_int
    lib.fa_oracle_threads.argtypes = []
    lib.fa_oracle_set_threads.restype = ctypes.c_int
    lib.fa_oracle_set_threads.argtypes = [ctypes.c_int]
    return lib


def load(path: Optional[str] = None):
    """Load (building first if absent) the oracle library."""
    global _lib
    if path is not None:
        return _bind(path)
    if _lib is None:
        if not os.path.exists(LIBRARY):
            build()
        _lib = _bind(LIBRARY)
    return _lib


def _as4d(x) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if a.ndim == 3:
        a = a[:, None]
    if a.ndim != 4:
        raise ValueError("expected [B,N,D] or [B,H,N,D]")
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def attention(q, k, v, scale: float, causal: bool, rows=None, lib=None
              ) -> Tuple[np.ndarray, np.ndarray]:
    """Two-pass fp64 attention.  q [B,(H,)Nq,D]; k, v [B,(H,)Nk,D].

    Returns o and lse shaped like q / q[..., 0] (or [len(rows), D] and
    [len(rows)] when ``rows`` lists flat row ids (b*H + h)*Nq + i).
    """
    lib = lib or load()
    squeeze = np.asarray(q).ndim == 3
    q4, k4, v4 = _as4d(q), _as4d(k), _as4d(v)
    B, H, Nq, D = q4.shape
    Nk = k4.shape[2]
    if k4.shape != (B, H, Nk, D) or v4.shape != (B, H, Nk, D):
        raise ValueError("q/k/v shapes disagree")
    if rows is None:
        o = np.empty((B, H, Nq, D))
        lse = np.empty((B, H, Nq))
        rp, nr = None, 0
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        o = np.empty((r.size, D))
        lse = np.empty((r.size,))
        rp, nr = r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), r.size
    st = lib.fa_oracle_attention(_ptr(q4), _ptr(k4), _ptr(v4), _ptr(o), _ptr(lse),
                                 B, H, Nq, Nk, D, float(scale), int(bool(causal)),
                                 rp, nr)
    if st != 0:
        raise RuntimeError(f"oracle failed with status {st}")
    if rows is None and squeeze:
        return o[:, 0], lse[:, 0]
    return o, lse


def attention_online(q, k, v, scale: float, causal: bool, bq: int, bk: int, lib=None
                     ) -> Tuple[np.ndarray, np.ndarray]:
    """The pages' tiled online recurrence in fp64 (self-check only)."""
    lib = lib or load()
    squeeze = np.asarray(q).ndim == 3
    q4, k4, v4 = _as4d(q), _as4d(k), _as4d(v)
    B, H, Nq, D = q4.shape
    Nk = k4.shape[2]
    o = np.empty((B, H, Nq, D))
    lse = np.empty((B, H, Nq))
    st = lib.fa_oracle_online(_ptr(q4), _ptr(k4), _ptr(v4), _ptr(o), _ptr(lse),
                              B, H, Nq, Nk, D, float(scale), int(bool(causal)),
                              int(bq), int(bk))
    if st != 0:
        raise RuntimeError(f"oracle failed with status {st}")
    if squeeze:
        return o[:, 0], lse[:, 0]
    return o, lse


def _rowlist(rows):
    if rows is None:
        return None, None, 0
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r, r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), r.size


def attention_bwd(q, k, v, do, scale: float, causal: bool, qrows=None, krows=None,
                  magnitudes: bool = False, lib=None):
    """fp64 gradients (dq, dk, dv) of the forward pass for upstream gradient do.

    q, do [B,(H,)Nq,D]; k, v [B,(H,)Nk,D].  With ``qrows`` (flat query rows
    (b*H + h)*Nq + i) dq is [len(qrows), D]; with ``krows`` (flat key rows
    (b*H + h)*Nk + j) dk and dv are [len(krows), D].  With ``magnitudes`` the
    absolute-value sums (bq, bk, bv) of the same shapes follow.
    """
    lib = lib or load()
    squeeze = np.asarray(q).ndim == 3
    q4, k4, v4, g4 = _as4d(q), _as4d(k), _as4d(v), _as4d(do)
    B, H, Nq, D = q4.shape
    Nk = k4.shape[2]
    if k4.shape != (B, H, Nk, D) or v4.shape != (B, H, Nk, D) or g4.shape != q4.shape:
        raise ValueError("q/k/v/do shapes disagree")
    qa, qp, nq = _rowlist(qrows)
    ka, kp, nk = _rowlist(krows)
    qshape = (B, H, Nq, D) if qa is None else (nq, D)
    kshape = (B, H, Nk, D) if ka is None else (nk, D)
    dq, dk, dv = np.empty(qshape), np.empty(kshape), np.empty(kshape)
    if magnitudes:
        bq, bk, bv = np.empty(qshape), np.empty(kshape), np.empty(kshape)
        mp = (_ptr(bq), _ptr(bk), _ptr(bv))
    else:
        mp = (None, None, None)
    st = lib.fa_oracle_attention_bwd(_ptr(q4), _ptr(k4), _ptr(v4), _ptr(g4),
                                     _ptr(dq), _ptr(dk), _ptr(dv), *mp,
                                     B, H, Nq, Nk, D, float(scale), int(bool(causal)),
                                     qp, nq, kp, nk)
    if st != 0:
        raise RuntimeError(f"oracle failed with status {st}")
    out = [dq, dk, dv] + ([bq, bk, bv] if magnitudes else [])
    if squeeze:
        out = [a[:, 0] if a.ndim == 4 else a for a in out]
    return tuple(out)


def attention_varlen(q, k, v, cu_q, cu_k, scale: float, causal: bool, lib=None
                     ) -> Tuple[np.ndarray, np.ndarray]:
    """Variable-length attention in fp64: the two-pass definition applied to
    each packed sequence on its own (q [H,Tq,D], k, v [H,Tk,D]; cu_q, cu_k
    offsets of length S+1).  Returns o [H,Tq,D], lse [H,Tq]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cu_q = [int(x) for x in cu_q]
    cu_k = [int(x) for x in cu_k]
    H, Tq, D = q.shape
    if (k.shape[0] != H or v.shape != k.shape or k.shape[2] != D or len(cu_q) != len(cu_k)
            or cu_q[0] != 0 or cu_k[0] != 0 or cu_q[-1] != Tq or cu_k[-1] != k.shape[1]
            or any(b < a for a, b in zip(cu_q, cu_q[1:]))
            or any(b < a for a, b in zip(cu_k, cu_k[1:]))):
        raise ValueError("inconsistent varlen shapes or offsets")
    o = np.zeros((H, Tq, D))
    lse = np.full((H, Tq), -np.inf)
    for s in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[s], cu_q[s + 1], cu_k[s], cu_k[s + 1]
        if q1 == q0 or k1 == k0:
            continue  # no rows, or no keys: O = 0, L = -inf
        so, sl = attention(q[None, :, q0:q1], k[None, :, k0:k1], v[None, :, k0:k1],
                           scale, causal, lib=lib)
        o[:, q0:q1] = so[0]
        lse[:, q0:q1] = sl[0]
    return o, lse


def attention_bwd_varlen(q, k, v, do, cu_q, cu_k, scale: float, causal: bool, lib=None):
    """fp64 gradients of attention_varlen for upstream gradient do [H,Tq,D]:
    attention_bwd on each packed sequence on its own."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    cu_q = [int(x) for x in cu_q]
    cu_k = [int(x) for x in cu_k]
    H, Tq, D = q.shape
    if do.shape != q.shape or cu_q[-1] != Tq or cu_k[-1] != k.shape[1] or len(cu_q) != len(cu_k):
        raise ValueError("inconsistent varlen shapes or offsets")
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for s in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[s], cu_q[s + 1], cu_k[s], cu_k[s + 1]
        if q1 == q0 or k1 == k0:
            continue
        a, b, c = attention_bwd(q[None, :, q0:q1], k[None, :, k0:k1], v[None, :, k0:k1],
                                do[None, :, q0:q1], scale, causal, lib=lib)
        dq[:, q0:q1], dk[:, k0:k1], dv[:, k0:k1] = a[0], b[0], c[0]
    return dq, dk, dv


def attention_masked(q, k, v, scale: float, causal: bool, window: int, nglobal: int,
                     rows=None, lib=None) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 attention over the keys a local window + global-token mask leaves
    visible (see fa_oracle_attention_masked); shapes as attention()."""
    lib = lib or load()
    squeeze = np.asarray(q).ndim == 3
    q4, k4, v4 = _as4d(q), _as4d(k), _as4d(v)
    B, H, Nq, D = q4.shape
    Nk = k4.shape[2]
    if k4.shape != (B, H, Nk, D) or v4.shape != (B, H, Nk, D):
        raise ValueError("q/k/v shapes disagree")
    if rows is None:
        o, lse = np.empty((B, H, Nq, D)), np.empty((B, H, Nq))
        rp, nr = None, 0
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        o, lse = np.empty((r.size, D)), np.empty((r.size,))
        rp, nr = r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), r.size
    st = lib.fa_oracle_attention_masked(_ptr(q4), _ptr(k4), _ptr(v4), _ptr(o), _ptr(lse),
                                        B, H, Nq, Nk, D, float(scale), int(bool(causal)),
                                        int(window), int(nglobal), rp, nr)
    if st != 0:
        raise RuntimeError(f"oracle failed with status {st}")
    if rows is None and squeeze:
        return o[:, 0], lse[:, 0]
    return o, lse


def attention_bwd_masked(q, k, v, do, scale: float, causal: bool, window: int, nglobal: int,
                         qrows=None, krows=None, magnitudes: bool = False, lib=None):
    """fp64 gradients of attention_masked for upstream gradient do; row
    lists and magnitude sums as attention_bwd (every sum over the visible
    pairs)."""
    lib = lib or load()
    squeeze = np.asarray(q).ndim == 3
    q4, k4, v4, g4 = _as4d(q), _as4d(k), _as4d(v), _as4d(do)
    B, H, Nq, D = q4.shape
    Nk = k4.shape[2]
    if k4.shape != (B, H, Nk, D) or v4.shape != (B, H, Nk, D) or g4.shape != q4.shape:
        raise ValueError("q/k/v/do shapes disagree")
    qa, qp, nq = _rowlist(qrows)
    ka, kp, nk = _rowlist(krows)
    qshape = (B, H, Nq, D) if qa is None else (nq, D)
    kshape = (B, H, Nk, D) if ka is None else (nk, D)
    dq, dk, dv = np.empty(qshape), np.empty(kshape), np.empty(kshape)
    if magnitudes:
        bq, bk, bv = np.empty(qshape), np.empty(kshape), np.empty(kshape)
        mp = (_ptr(bq), _ptr(bk), _ptr(bv))
    else:
        mp = (None, None, None)
    st = lib.fa_oracle_attention_bwd_masked(_ptr(q4), _ptr(k4), _ptr(v4), _ptr(g4), _ptr(dq),
                                            _ptr(dk), _ptr(dv), *mp, B, H, Nq, Nk, D,
                                            float(scale), int(bool(causal)), int(window),
                                            int(nglobal), qp, nq, kp, nk)
    if st != 0:
        raise RuntimeError(f"oracle failed with status {st}")
    out = [dq, dk, dv] + ([bq, bk, bv] if magnitudes else [])
    if squeeze:
        out = [a[:, 0] if a.ndim == 4 else a for a in out]
    return tuple(out)


def threads(lib=None) -> int:
    return int((lib or load()).fa_oracle_threads())


def set_threads(n: int, lib=None) -> int:
    """OpenMP threads of later oracle calls; returns the previous setting."""
    return int((lib or load()).fa_oracle_set_threads(int(n)))
