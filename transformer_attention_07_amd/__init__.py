"""Python binding of libfa.so, the MI355X FlashAttention-2 library.

The binding marshals arguments only: every step of the forward and backward
passes runs in the HIP kernels of libfa.so (csrc/fa_fwd.hip, csrc/fa_bwd.hip).  PyTorch is used to allocate
the outputs and to name the current HIP stream.  There is no fallback: if
libfa.so is missing or fails to load, every call raises.

C-ABI mirrors (same names and meaning as include/fa.h):
    fa_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Nq, Nk, D, scale,
           causal, dtype, stream) -> status
    fa_fwd_workspace_size(B, H, Nq, Nk, D, causal, dtype) -> (status, bytes)
    fa_fwd_ws(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Nq, Nk, D, scale,
              causal, dtype, ws_ptr, ws_bytes, stream) -> status
    fa_fwd_varlen(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, cu_q_ptr, cu_k_ptr, S, H,
                  Tq, Tk, max_seqlen_q, D, scale, causal, dtype, stream) -> status
    fa_fwd_varlen_workspace_size(S, H, Tq, Tk, max_seqlen_q, max_seqlen_k, D, causal,
                  dtype) -> (status, bytes)
    fa_fwd_varlen_ws(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, cu_q_ptr, cu_k_ptr, S, H, Tq,
                  Tk, max_seqlen_q, max_seqlen_k, D, scale, causal, dtype, ws_ptr,
                  ws_bytes, stream) -> status
    fa_fwd_masked(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Nq, Nk, D, scale,
                  causal, window, nglobal, dtype, stream) -> status
    fa_fwd_fp8(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Nq, Nk, D, scale,
               descale_q, descale_k, descale_v, causal, out_f32, stream) -> status
    fa_bwd_workspace_size(B, H, Nq, Nk, D, causal, dtype) -> (status, bytes)
    fa_bwd_masked_workspace_size(B, H, Nq, Nk, D, causal, window, nglobal, dtype)
        -> (status, bytes)
    fa_bwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr, dv_ptr,
           B, H, Nq, Nk, D, scale, causal, dtype, ws_ptr, ws_bytes, stream)
        -> status
    fa_bwd_masked(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr,
                  dv_ptr, B, H, Nq, Nk, D, scale, causal, window, nglobal, dtype,
                  ws_ptr, ws_bytes, stream) -> status
    fa_bwd_varlen(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr,
                  dv_ptr, cu_q_ptr, cu_k_ptr, S, H, Tq, Tk, max_q, max_k, D, scale,
                  causal, dtype, ws_ptr, ws_bytes, stream) -> status
    fa_status_str(status) -> str
    fa_last_hip_error() -> str
    fa_version() -> int
Tensor convenience:
    fwd(q, k, v, causal=False, scale=None, out_dtype=None, split=True)
        -> (o, lse); split=True runs fa_fwd_ws with a workspace from torch's
        allocator, split=False runs fa_fwd
    fwd_varlen(q, k, v, cu_q, cu_k, max_seqlen_q, causal=False, scale=None,
               out_dtype=None) -> (o, lse) through fa_fwd_varlen
    fwd_masked(q, k, v, window, nglobal=0, causal=False, scale=None,
               out_dtype=None) -> (o, lse) through fa_fwd_masked
    fwd_fp8(q8, k8, v8, descale_q, descale_k, descale_v, causal=False, scale=None,
            out_dtype=None, ws=True) -> (o, lse); ws=True runs fa_fwd_fp8_ws (the
        pipelined kernel, workspace from torch's allocator), ws=False fa_fwd_fp8
    bwd(q, k, v, o, lse, do, causal=False, scale=None, grad_dtype=None,
        window=None, nglobal=0) -> (dq, dk, dv) through fa_bwd (fa_bwd_masked
        when a window is given)
    bwd_varlen(q, k, v, o, lse, do, cu_q, cu_k, max_q, max_k, causal=False,
               scale=None, grad_dtype=None) -> (dq, dk, dv) through fa_bwd_varlen
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

__all__ = [
    "FA_F32", "FA_BF16", "FA_BF16_OF32", "FA_F16", "FA_F16_OF32",
    "FA_OK", "FA_ERR_NULLPTR", "FA_ERR_SHAPE", "FA_ERR_HEAD_DIM", "FA_ERR_DTYPE",
    "FA_ERR_SCALE", "FA_ERR_ALIGN", "FA_ERR_HIP", "FA_ERR_OVERLAP", "FA_ERR_WORKSPACE",
    "LIBRARY", "DEBUG_LIBRARY", "EXPORTS", "library", "debug_library", "fa_fwd", "fa_fwd_workspace_size", "fa_fwd_ws",
    "fa_fwd_noalloc", "fa_fwd_varlen", "fa_fwd_varlen_workspace_size", "fa_fwd_varlen_ws", "fa_fwd_masked", "fa_fwd_masked_workspace_size", "fa_fwd_masked_ws", "fa_fwd_fp8", "fa_fwd_fp8_workspace_size", "fa_fwd_fp8_ws",
    "fa_bwd_workspace_size", "fa_bwd_masked_workspace_size", "fa_bwd", "fa_bwd_varlen", "fa_bwd_masked", "fa_status_str",
    "fa_last_hip_error", "fa_version", "fwd", "fwd_varlen", "fwd_masked", "fwd_fp8", "bwd", "bwd_varlen", "FaError",
]

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")
DEBUG_LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_debug.so")

# Scratch of fa_fwd_noalloc per device (include/fa.h)
FA_NOALLOC_SCRATCH_BYTES = 72 * 1024 * 1024

FA_F32, FA_BF16, FA_BF16_OF32, FA_F16, FA_F16_OF32 = 0, 1, 2, 3, 4
(FA_OK, FA_ERR_NULLPTR, FA_ERR_SHAPE, FA_ERR_HEAD_DIM, FA_ERR_DTYPE, FA_ERR_SCALE,
 FA_ERR_ALIGN, FA_ERR_HIP, FA_ERR_OVERLAP, FA_ERR_WORKSPACE) = range(10)

# Every symbol include/fa.h declares.
EXPORTS = ("fa_fwd", "fa_fwd_workspace_size", "fa_fwd_ws", "fa_fwd_noalloc", "fa_fwd_varlen",
           "fa_fwd_varlen_workspace_size", "fa_fwd_varlen_ws", "fa_fwd_masked", "fa_fwd_masked_workspace_size", "fa_fwd_masked_ws", "fa_fwd_fp8",
           "fa_fwd_fp8_workspace_size", "fa_fwd_fp8_ws", "fa_bwd_workspace_size",
           "fa_bwd_masked_workspace_size", "fa_bwd",
           "fa_bwd_varlen", "fa_bwd_masked",
           "fa_status_str", "fa_last_hip_error", "fa_version")

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def library() -> ctypes.CDLL:
    """Load libfa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _bind(LIBRARY)
    return _lib


def debug_library() -> ctypes.CDLL:
    """Load libfa_debug.so, the build with ring-barrier checks
    (include/fa_debug.h), with the same prototypes plus
    fa_debug_barrier_faults.  The wrappers below use it in place of libfa.so
    while ``_lib`` is set to it."""
    lib = _bind(DEBUG_LIBRARY)
    lib.fa_debug_barrier_faults.restype = ctypes.c_int
    lib.fa_debug_barrier_faults.argtypes = [ctypes.POINTER(ctypes.c_uint), ctypes.c_int]
    return lib


def _bind(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m "
            "transformer_attention_07_amd.build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                           ctypes.c_int, ctypes.c_int, vp]
    lib.fa_fwd_workspace_size.restype = ctypes.c_int
    lib.fa_fwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int,
                                          ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
    lib.fa_fwd_ws.restype = ctypes.c_int
    lib.fa_fwd_ws.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                              ctypes.c_int, ctypes.c_int, vp, ctypes.c_size_t, vp]
    lib.fa_fwd_noalloc.restype = ctypes.c_int
    lib.fa_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                                   ctypes.c_int, ctypes.c_int, vp]
    lib.fa_fwd_varlen.restype = ctypes.c_int
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                  ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
    lib.fa_fwd_varlen_workspace_size.restype = ctypes.c_int
    lib.fa_fwd_varlen_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, i64, ctypes.c_int,
                                                 ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
    lib.fa_fwd_varlen_ws.restype = ctypes.c_int
    lib.fa_fwd_varlen_ws.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                     i64, ctypes.c_float, ctypes.c_int, ctypes.c_int, vp,
                                     ctypes.c_size_t, vp]
    lib.fa_fwd_masked.restype = ctypes.c_int
    lib.fa_fwd_masked.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                                  ctypes.c_int, i64, i64, ctypes.c_int, vp]
    lib.fa_fwd_masked_workspace_size.restype = ctypes.c_int
    lib.fa_fwd_masked_workspace_size.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, i64,
                                                 i64, ctypes.c_int,
                                                 ctypes.POINTER(ctypes.c_size_t)]
    lib.fa_fwd_masked_ws.restype = ctypes.c_int
    lib.fa_fwd_masked_ws.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                     ctypes.c_float, ctypes.c_int, i64, i64, ctypes.c_int, vp,
                                     ctypes.c_size_t, vp]
    lib.fa_fwd_fp8.restype = ctypes.c_int
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                               ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_int,
                               ctypes.c_int, vp]
    lib.fa_fwd_fp8_workspace_size.restype = ctypes.c_int
    lib.fa_fwd_fp8_workspace_size.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int,
                                              ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
    lib.fa_fwd_fp8_ws.restype = ctypes.c_int
    lib.fa_fwd_fp8_ws.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                                  ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_int,
                                  ctypes.c_int, vp, ctypes.c_size_t, vp]
    lib.fa_bwd_workspace_size.restype = ctypes.c_int
    lib.fa_bwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int,
                                          ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
    lib.fa_bwd_masked_workspace_size.restype = ctypes.c_int
    lib.fa_bwd_masked_workspace_size.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, i64,
                                                 i64, ctypes.c_int,
                                                 ctypes.POINTER(ctypes.c_size_t)]
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                           ctypes.c_float, ctypes.c_int, ctypes.c_int, vp, ctypes.c_size_t,
                           vp]
    lib.fa_bwd_masked.restype = ctypes.c_int
    lib.fa_bwd_masked.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                  ctypes.c_float, ctypes.c_int, i64, i64, ctypes.c_int, vp,
                                  ctypes.c_size_t, vp]
    lib.fa_bwd_varlen.restype = ctypes.c_int
    lib.fa_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64,
                                  i64, i64, i64, i64, ctypes.c_float, ctypes.c_int,
                                  ctypes.c_int, vp, ctypes.c_size_t, vp]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_status_str.argtypes = [ctypes.c_int]
    lib.fa_last_hip_error.restype = ctypes.c_char_p
    lib.fa_last_hip_error.argtypes = []
    lib.fa_version.restype = ctypes.c_int
    lib.fa_version.argtypes = []
    return lib


def fa_fwd(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, dtype, stream) -> int:
    """Raw C call; pointers are integers (device addresses) or None."""
    return int(library().fa_fwd(q, k, v, o, lse, B, H, Nq, Nk, D, float(scale),
                                int(causal), int(dtype), stream))


def fa_fwd_workspace_size(B, H, Nq, Nk, D, causal, dtype) -> Tuple[int, int]:
    """Raw C call; returns (status, workspace bytes)."""
    n = ctypes.c_size_t(0)
    st = int(library().fa_fwd_workspace_size(B, H, Nq, Nk, D, int(causal), int(dtype),
                                             ctypes.byref(n)))
    return st, int(n.value)


def fa_fwd_ws(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, dtype, ws, ws_bytes,
              stream) -> int:
    """Raw C call; pointers are integers (device addresses) or None."""
    return int(library().fa_fwd_ws(q, k, v, o, lse, B, H, Nq, Nk, D, float(scale),
                                   int(causal), int(dtype), ws, int(ws_bytes), stream))


def fa_fwd_noalloc(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, dtype, stream) -> int:
    """Raw C call; pointers are integers (device addresses) or None."""
    return int(library().fa_fwd_noalloc(q, k, v, o, lse, B, H, Nq, Nk, D, float(scale),
                                        int(causal), int(dtype), stream))


def fa_fwd_varlen_workspace_size(S, H, Tq, Tk, max_seqlen_q, max_seqlen_k, D, causal,
                                 dtype) -> Tuple[int, int]:
    """Raw C call; returns (status, workspace bytes)."""
    n = ctypes.c_size_t(0)
    st = int(library().fa_fwd_varlen_workspace_size(S, H, Tq, Tk, max_seqlen_q, max_seqlen_k,
                                                    D, int(causal), int(dtype),
                                                    ctypes.byref(n)))
    return st, int(n.value)


def fa_fwd_varlen_ws(q, k, v, o, lse, cu_q, cu_k, S, H, Tq, Tk, max_seqlen_q, max_seqlen_k, D,
                     scale, causal, dtype, ws, ws_bytes, stream) -> int:
    """Raw C call; pointers are integers (device addresses) or None."""
    return int(library().fa_fwd_varlen_ws(q, k, v, o, lse, cu_q, cu_k, S, H, Tq, Tk,
                                          max_seqlen_q, max_seqlen_k, D, float(scale),
                                          int(causal), int(dtype), ws, int(ws_bytes), stream))


def fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, S, H, Tq, Tk, max_seqlen_q, D, scale, causal,
                  dtype, stream) -> int:
    """Raw C call; pointers are integers (device addresses) or None."""
    return int(library().fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, S, H, Tq, Tk,
                                       max_seqlen_q, D, float(scale), int(causal),
                                       int(dtype), stream))


def fa_fwd_masked(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, window, nglobal, dtype,
                  stream) -> int:
    """Raw C call; pointers are integers (device addresses) or None."""
    return int(library().fa_fwd_masked(q, k, v, o, lse, B, H, Nq, Nk, D, float(scale),
                                       int(causal), int(window), int(nglobal), int(dtype),
                                       stream))


def fa_fwd_masked_workspace_size(B, H, Nq, Nk, D, causal, window, nglobal,
                                 dtype) -> Tuple[int, int]:
    """Raw C call; returns (status, workspace bytes)."""
    n = ctypes.c_size_t(0)
    st = int(library().fa_fwd_masked_workspace_size(B, H, Nq, Nk, D, int(causal), int(window),
                                                    int(nglobal), int(dtype),
                                                    ctypes.byref(n)))
    return st, int(n.value)


def fa_fwd_masked_ws(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, window, nglobal, dtype,
                     ws, ws_bytes, stream) -> int:
    """Raw C call; pointers are integers (device addresses) or None."""
    return int(library().fa_fwd_masked_ws(q, k, v, o, lse, B, H, Nq, Nk, D, float(scale),
                                          int(causal), int(window), int(nglobal), int(dtype),
                                          ws, int(ws_bytes), stream))


def fa_fwd_fp8(q, k, v, o, lse, B, H, Nq, Nk, D, scale, dq, dk, dv, causal, out_f32,
               stream) -> int:
    """Raw C call; pointers are integers (device addresses) or None."""
    return int(library().fa_fwd_fp8(q, k, v, o, lse, B, H, Nq, Nk, D, float(scale), float(dq),
                                    float(dk), float(dv), int(causal), int(out_f32), stream))


def fa_fwd_fp8_workspace_size(B, H, Nq, Nk, D, causal, out_f32) -> Tuple[int, int]:
    """Raw C call; returns (status, workspace bytes)."""
    n = ctypes.c_size_t(0)
    st = int(library().fa_fwd_fp8_workspace_size(B, H, Nq, Nk, D, int(causal), int(out_f32),
                                                 ctypes.byref(n)))
    return st, int(n.value)


def fa_fwd_fp8_ws(q, k, v, o, lse, B, H, Nq, Nk, D, scale, dq, dk, dv, causal, out_f32, ws,
                  ws_bytes, stream) -> int:
    """Raw C call; pointers are integers (device addresses) or None."""
    return int(library().fa_fwd_fp8_ws(q, k, v, o, lse, B, H, Nq, Nk, D, float(scale),
                                       float(dq), float(dk), float(dv), int(causal),
                                       int(out_f32), ws, ws_bytes, stream))


def fa_bwd_workspace_size(B, H, Nq, Nk, D, causal, dtype) -> Tuple[int, int]:
    """Raw C call; returns (status, workspace bytes)."""
    n = ctypes.c_size_t(0)
    st = int(library().fa_bwd_workspace_size(B, H, Nq, Nk, D, int(causal), int(dtype),
                                             ctypes.byref(n)))
    return st, int(n.value)


def fa_bwd_masked_workspace_size(B, H, Nq, Nk, D, causal, window, nglobal,
                                 dtype) -> Tuple[int, int]:
    """Raw C call; returns (status, workspace bytes)."""
    n = ctypes.c_size_t(0)
    st = int(library().fa_bwd_masked_workspace_size(B, H, Nq, Nk, D, int(causal), int(window),
                                                    int(nglobal), int(dtype),
                                                    ctypes.byref(n)))
    return st, int(n.value)


def fa_bwd(q, k, v, o, lse, do, dq, dk, dv, B, H, Nq, Nk, D, scale, causal, dtype, ws,
           ws_bytes, stream) -> int:
    """Raw C call; pointers are integers (device addresses) or None."""
    return int(library().fa_bwd(q, k, v, o, lse, do, dq, dk, dv, B, H, Nq, Nk, D,
                                float(scale), int(causal), int(dtype), ws, int(ws_bytes),
                                stream))


def fa_bwd_masked(q, k, v, o, lse, do, dq, dk, dv, B, H, Nq, Nk, D, scale, causal, window,
                  nglobal, dtype, ws, ws_bytes, stream) -> int:
    """Raw C call; pointers are integers (device addresses) or None."""
    return int(library().fa_bwd_masked(q, k, v, o, lse, do, dq, dk, dv, B, H, Nq, Nk, D,
                                       float(scale), int(causal), int(window), int(nglobal),
                                       int(dtype), ws, int(ws_bytes), stream))


def fa_bwd_varlen(q, k, v, o, lse, do, dq, dk, dv, cu_q, cu_k, S, H, Tq, Tk, max_q, max_k,
                  D, scale, causal, dtype, ws, ws_bytes, stream) -> int:
    """Raw C call; pointers are integers (device addresses) or None."""
    return int(library().fa_bwd_varlen(q, k, v, o, lse, do, dq, dk, dv, cu_q, cu_k, S, H, Tq,
                                       Tk, max_q, max_k, D, float(scale), int(causal),
                                       int(dtype), ws, int(ws_bytes), stream))


def fa_status_str(status: int) -> str:
    return library().fa_status_str(int(status)).decode()


def fa_last_hip_error() -> str:
    return library().fa_last_hip_error().decode()


def fa_version() -> int:
    return int(library().fa_version())


def _dtype_code(torch, in_dtype, out_dtype) -> int:
    table = {
        (torch.float32, torch.float32): FA_F32,
        (torch.bfloat16, torch.bfloat16): FA_BF16,
        (torch.bfloat16, torch.float32): FA_BF16_OF32,
        (torch.float16, torch.float16): FA_F16,
        (torch.float16, torch.float32): FA_F16_OF32,
    }
    key = (in_dtype, out_dtype)
    if key not in table:
        raise ValueError(f"unsupported (input, output) dtypes {key}")
    return table[key]


def fwd(q, k, v, causal: bool = False, scale: Optional[float] = None,
        out_dtype=None, out=None, stream=None,
        split: bool = True) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """Attention forward on device tensors.

    q: [B,Nq,D] or [B,H,Nq,D]; k, v: [B,Nk,D] or [B,H,Nk,D]; same dtype
    (fp32, bf16 or fp16), same device, contiguous.  Returns (o, lse) with o
    shaped like q in ``out_dtype`` (default: q's dtype) and lse fp32 shaped
    like q[..., 0].  ``scale`` defaults to 1/sqrt(D).  ``out`` may pass
    preallocated (o, lse).  Runs on ``stream`` (default: torch's current
    stream of q's device).  ``split`` selects fa_fwd_ws (the key ranges of
    long query tiles cut over the compute units, scratch from torch's
    allocator) or fa_fwd (one workgroup per query tile).
    """
    import torch

    if q.dim() not in (3, 4) or k.dim() != q.dim() or v.dim() != q.dim():
        raise ValueError("q, k, v must all be [B,N,D] or all [B,H,N,D]")
    three = q.dim() == 3
    q4 = q.unsqueeze(1) if three else q
    k4 = k.unsqueeze(1) if three else k
    v4 = v.unsqueeze(1) if three else v
    B, H, Nq, D = q4.shape
    Nk = k4.shape[2]
    if tuple(k4.shape) != (B, H, Nk, D) or tuple(v4.shape) != (B, H, Nk, D):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} "
                         f"v{tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on the same GPU device")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    code = _dtype_code(torch, q.dtype, out_dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        o = torch.empty(q.shape, dtype=out_dtype, device=q.device)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        if o.shape != q.shape or o.dtype != out_dtype or not o.is_contiguous():
            raise ValueError("out[0] must be contiguous, shaped like q, of out_dtype")
        if lse.shape != q.shape[:-1] or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError("out[1] must be contiguous fp32 shaped like q[..., 0]")
    own_stream = stream is None
    if own_stream:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    if split:
        st, nbytes = fa_fwd_workspace_size(B, H, Nq, Nk, D, causal, code)
        if st == FA_OK:
            # torch's allocator hands this block out again once the kernels
            # queued on the current stream have run; on another stream the
            # block is tied to that stream too.
            ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
            if not own_stream:
                ws.record_stream(torch.cuda.ExternalStream(stream, device=q.device))
            st = fa_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                           lse.data_ptr(), B, H, Nq, Nk, D, scale, causal, code,
                           ws.data_ptr(), nbytes, stream)
    else:
        st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                    lse.data_ptr(), B, H, Nq, Nk, D, scale, causal, code, stream)
    if st != FA_OK:
        msg = fa_status_str(st)
        if st == FA_ERR_HIP:
            msg += ": " + fa_last_hip_error()
        raise FaError(st, msg)
    return o, lse


def bwd(q, k, v, o, lse, do, causal: bool = False, scale: Optional[float] = None,
        grad_dtype=None, out=None, stream=None, window: Optional[int] = None,
        nglobal: int = 0) -> Tuple["torch.Tensor", "torch.Tensor", "torch.Tensor"]:
    """Attention backward on device tensors (fa_bwd).

    q, o, do: [B,Nq,D] or [B,H,Nq,D]; k, v: [B,Nk,D] or [B,H,Nk,D]; all of
    one 16-bit dtype (bf16 or fp16), same device, contiguous; lse fp32 shaped
    like q[..., 0] (the forward's outputs o and lse; with ``window`` the
    outputs of fwd_masked with the same window and ``nglobal``, and the
    gradients are those of the masked pass).  Returns (dq, dk, dv)
    shaped like q, k, v in ``grad_dtype`` (default: the input dtype; fp32
    keeps the gradients unrounded).  ``scale`` defaults to 1/sqrt(D) and
    must equal the forward's.  The row-term workspace comes from torch's
    allocator.
    """
    import torch

    t = (q, k, v, o, do)
    if q.dim() not in (3, 4) or any(x.dim() != q.dim() for x in t):
        raise ValueError("q, k, v, o, do must all be [B,N,D] or all [B,H,N,D]")
    three = q.dim() == 3
    q4, k4 = (x.unsqueeze(1) if three else x for x in (q, k))
    B, H, Nq, D = q4.shape
    Nk = k4.shape[2]
    if (tuple(k.shape) != tuple(v.shape) or tuple(o.shape) != tuple(q.shape)
            or tuple(do.shape) != tuple(q.shape) or tuple(k4.shape) != (B, H, Nk, D)):
        raise ValueError("shape mismatch among q, k, v, o, do")
    if tuple(lse.shape) != tuple(q.shape[:-1]) or lse.dtype != torch.float32:
        raise ValueError("lse must be fp32 shaped like q[..., 0]")
    if not all(x.dtype == q.dtype for x in t):
        raise ValueError("q, k, v, o, do must share a dtype")
    if not all(x.is_cuda and x.device == q.device for x in t + (lse,)):
        raise ValueError("all tensors must be on the same GPU device")
    if not all(x.is_contiguous() for x in t + (lse,)):
        raise ValueError("all tensors must be contiguous")
    grad_dtype = q.dtype if grad_dtype is None else grad_dtype
    code = _dtype_code(torch, q.dtype, grad_dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        dq = torch.empty(q.shape, dtype=grad_dtype, device=q.device)
        dk = torch.empty(k.shape, dtype=grad_dtype, device=q.device)
        dv = torch.empty(v.shape, dtype=grad_dtype, device=q.device)
    else:
        dq, dk, dv = out
    own_stream = stream is None
    if own_stream:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    if window is None:
        st, nbytes = fa_bwd_workspace_size(B, H, Nq, Nk, D, causal, code)
    else:
        st, nbytes = fa_bwd_masked_workspace_size(B, H, Nq, Nk, D, causal, window, nglobal,
                                                  code)
    if st == FA_OK:
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
        if not own_stream:
            ws.record_stream(torch.cuda.ExternalStream(stream, device=q.device))
        ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Nq, Nk, D,
                scale, causal)
        if window is None:
            st = fa_bwd(*ptrs, code, ws.data_ptr(), nbytes, stream)
        else:
            st = fa_bwd_masked(*ptrs, window, nglobal, code, ws.data_ptr(), nbytes, stream)
    if st != FA_OK:
        msg = fa_status_str(st)
        if st == FA_ERR_HIP:
            msg += ": " + fa_last_hip_error()
        raise FaError(st, msg)
    return dq, dk, dv


def fwd_varlen(q, k, v, cu_q, cu_k, max_seqlen_q: int, causal: bool = False,
               scale: Optional[float] = None, out_dtype=None, stream=None,
               max_seqlen_k: Optional[int] = None
               ) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """Variable-length attention forward (fa_fwd_varlen) on device tensors.

    q: [H, Tq, D]; k, v: [H, Tk, D] (bf16 or fp16, contiguous, one device);
    cu_q, cu_k: int32 device tensors of S + 1 offsets (0, ..., Tq / Tk).
    With ``max_seqlen_k`` given, the work is split over the keys
    (fa_fwd_varlen_ws, workspace allocated here): a stream schedule over
    the (head, sequence) pairs up to 512 of them, key-split tiles above.
    Returns (o [H, Tq, D] in ``out_dtype``, lse [H, Tq] fp32).
    """
    import torch

    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [H, T, D]")
    H, Tq, D = q.shape
    Tk = k.shape[1]
    if tuple(k.shape) != (H, Tk, D) or tuple(v.shape) != (H, Tk, D):
        raise ValueError("shape mismatch among q, k, v")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    if cu_q.dtype != torch.int32 or cu_k.dtype != torch.int32 or cu_q.shape != cu_k.shape:
        raise ValueError("cu_q, cu_k must be int32 tensors of equal length")
    t = (q, k, v, cu_q, cu_k)
    if not all(x.is_cuda and x.device == q.device and x.is_contiguous() for x in t):
        raise ValueError("all tensors must be contiguous on the same GPU device")
    S = cu_q.numel() - 1
    out_dtype = q.dtype if out_dtype is None else out_dtype
    code = _dtype_code(torch, q.dtype, out_dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    lse = torch.empty((H, Tq), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    if max_seqlen_k is None:
        st = fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                           lse.data_ptr(), cu_q.data_ptr(), cu_k.data_ptr(), S, H, Tq, Tk,
                           int(max_seqlen_q), D, scale, causal, code, stream)
    else:
        st, nb = fa_fwd_varlen_workspace_size(S, H, Tq, Tk, int(max_seqlen_q),
                                              int(max_seqlen_k), D, causal, code)
        if st == FA_OK:
            ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=q.device)
            st = fa_fwd_varlen_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), cu_q.data_ptr(), cu_k.data_ptr(), S, H, Tq,
                                  Tk, int(max_seqlen_q), int(max_seqlen_k), D, scale, causal,
                                  code, ws.data_ptr() if nb else None, nb, stream)
    if st != FA_OK:
        msg = fa_status_str(st)
        if st == FA_ERR_HIP:
            msg += ": " + fa_last_hip_error()
        raise FaError(st, msg)
    return o, lse


def bwd_varlen(q, k, v, o, lse, do, cu_q, cu_k, max_q: int, max_k: int,
               causal: bool = False, scale: Optional[float] = None, grad_dtype=None,
               stream=None):
    """Variable-length attention backward (fa_bwd_varlen) on device tensors:
    q, o, do [H, Tq, D]; k, v [H, Tk, D]; lse [H, Tq]; cu_q, cu_k int32
    offsets.  Returns (dq, dk, dv) in ``grad_dtype`` (default: the input
    dtype)."""
    import torch

    t = (q, k, v, o, do)
    if any(x.dim() != 3 for x in t):
        raise ValueError("q, k, v, o, do must be [H, T, D]")
    H, Tq, D = q.shape
    Tk = k.shape[1]
    if (tuple(k.shape) != (H, Tk, D) or tuple(v.shape) != (H, Tk, D)
            or tuple(o.shape) != tuple(q.shape) or tuple(do.shape) != tuple(q.shape)):
        raise ValueError("shape mismatch among q, k, v, o, do")
    if tuple(lse.shape) != (H, Tq) or lse.dtype != torch.float32:
        raise ValueError("lse must be fp32 [H, Tq]")
    if not all(x.dtype == q.dtype for x in t):
        raise ValueError("q, k, v, o, do must share a dtype")
    if cu_q.dtype != torch.int32 or cu_k.dtype != torch.int32 or cu_q.shape != cu_k.shape:
        raise ValueError("cu_q, cu_k must be int32 tensors of equal length")
    allt = t + (lse, cu_q, cu_k)
    if not all(x.is_cuda and x.device == q.device and x.is_contiguous() for x in allt):
        raise ValueError("all tensors must be contiguous on the same GPU device")
    S = cu_q.numel() - 1
    grad_dtype = q.dtype if grad_dtype is None else grad_dtype
    code = _dtype_code(torch, q.dtype, grad_dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty(q.shape, dtype=grad_dtype, device=q.device)
    dk = torch.empty(k.shape, dtype=grad_dtype, device=q.device)
    dv = torch.empty(v.shape, dtype=grad_dtype, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    nbytes = H * Tq * 4
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    st = fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                       cu_q.data_ptr(), cu_k.data_ptr(), S, H, Tq, Tk, int(max_q), int(max_k),
                       D, scale, causal, code, ws.data_ptr(), nbytes, stream)
    if st != FA_OK:
        msg = fa_status_str(st)
        if st == FA_ERR_HIP:
            msg += ": " + fa_last_hip_error()
        raise FaError(st, msg)
    return dq, dk, dv


def fwd_masked(q, k, v, window: int, nglobal: int = 0, causal: bool = False,
               scale: Optional[float] = None, out_dtype=None, stream=None
               ) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """Local-window + global-token attention forward (fa_fwd_masked) on
    device tensors shaped as for fwd() (16-bit inputs)."""
    import torch

    if q.dim() not in (3, 4) or k.dim() != q.dim() or v.dim() != q.dim():
        raise ValueError("q, k, v must all be [B,N,D] or all [B,H,N,D]")
    q4, k4 = (x.unsqueeze(1) if q.dim() == 3 else x for x in (q, k))
    B, H, Nq, D = q4.shape
    Nk = k4.shape[2]
    if tuple(k.shape) != tuple(v.shape) or tuple(k4.shape) != (B, H, Nk, D):
        raise ValueError("shape mismatch among q, k, v")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    if not all(x.is_cuda and x.device == q.device and x.is_contiguous() for x in (q, k, v)):
        raise ValueError("q, k, v must be contiguous on the same GPU device")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    code = _dtype_code(torch, q.dtype, out_dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st, nbytes = fa_fwd_masked_workspace_size(B, H, Nq, Nk, D, causal, window, nglobal, code)
    if st == FA_OK:
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device) if nbytes else None
        if ws is not None and stream != torch.cuda.current_stream(q.device).cuda_stream:
            ws.record_stream(torch.cuda.ExternalStream(stream, device=q.device))
        st = fa_fwd_masked_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), B, H, Nq, Nk, D, scale, causal, window, nglobal,
                              code, None if ws is None else ws.data_ptr(), nbytes, stream)
    if st != FA_OK:
        msg = fa_status_str(st)
        if st == FA_ERR_HIP:
            msg += ": " + fa_last_hip_error()
        raise FaError(st, msg)
    return o, lse


def fwd_fp8(q, k, v, descale_q: float, descale_k: float, descale_v: float,
            causal: bool = False, scale: Optional[float] = None, out_dtype=None, stream=None,
            ws: bool = True) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """FP8 attention forward: q, k, v torch.float8_e4m3fn device tensors
    [B,N,D] or [B,H,N,D] (real inputs = values x descale factors).  ws=True
    runs fa_fwd_fp8_ws (the pipelined kernel; workspace allocated here),
    ws=False fa_fwd_fp8.  Returns (o in bf16 or fp32, lse fp32)."""
    import torch

    if q.dim() not in (3, 4) or k.dim() != q.dim() or v.dim() != q.dim():
        raise ValueError("q, k, v must all be [B,N,D] or all [B,H,N,D]")
    q4, k4 = (x.unsqueeze(1) if q.dim() == 3 else x for x in (q, k))
    B, H, Nq, D = q4.shape
    Nk = k4.shape[2]
    if tuple(k.shape) != tuple(v.shape) or tuple(k4.shape) != (B, H, Nk, D):
        raise ValueError("shape mismatch among q, k, v")
    if not all(x.dtype == torch.float8_e4m3fn for x in (q, k, v)):
        raise ValueError("q, k, v must be torch.float8_e4m3fn")
    if not all(x.is_cuda and x.device == q.device and x.is_contiguous() for x in (q, k, v)):
        raise ValueError("q, k, v must be contiguous on the same GPU device")
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be bfloat16 or float32")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    f32 = out_dtype == torch.float32
    if ws:
        st, nb = fa_fwd_fp8_workspace_size(B, H, Nq, Nk, D, causal, f32)
        if st == FA_OK:
            buf = torch.empty(max(nb, 16), dtype=torch.uint8, device=q.device)
            st = fa_fwd_fp8_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                               lse.data_ptr(), B, H, Nq, Nk, D, scale, descale_q, descale_k,
                               descale_v, causal, f32, buf.data_ptr(), nb, stream)
    else:
        st = fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        B, H, Nq, Nk, D, scale, descale_q, descale_k, descale_v, causal, f32,
                        stream)
    if st != FA_OK:
        msg = fa_status_str(st)
        if st == FA_ERR_HIP:
            msg += ": " + fa_last_hip_error()
        raise FaError(st, msg)
    return o, lse
