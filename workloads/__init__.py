"""Seeded synthetic inputs for the attention forward pass.

This module is shared by the CPU oracle side (tests), the GPU side (tests,
smoke, bench) and nothing else.  It holds NO attention arithmetic: it only
draws Gaussian tensors from a seeded CPU generator, rounds them to the
storage dtype, and names the workload shapes.

Workload shapes follow the sweep on the page "FlashAttention-2实现与优化：
高效注意力机制详解" (§2.1: batch 8, one head, head dim 16/32/64/128, sequence
256 ... 16384) and an 8K-context decoder layer of a 70B-class model
(page "FlashAttention技术演进全景图", §5.3).  The pages measure no public
dataset; i.i.d. Gaussian tensors of those shapes stand in for real
activations.

The backward pass also needs an upstream gradient dO of O: ``gen_grad_out``
draws it the same way (i.i.d. N(0,1), its own seed, rounded to the storage
dtype).

Generation recipe (fixed, so every consumer sees identical values):
  * one ``torch.Generator`` on the CPU, ``manual_seed(seed)``;
  * draw q, then k, then v, each ``randn([B, H, N, D])`` in fp32;
  * multiply q by ``q_mult`` and all three by ``std`` (both powers of two in
    every named workload, so scaling commutes with the rounding below);
  * round to the storage dtype (bf16/fp16 by round-to-nearest-even).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import torch

__all__ = [
    "Workload",
    "gen_qkv",
    "gen_grad_out",
    "varlen_lengths",
    "gen_qkv_fp8",
    "sample_rows",
    "WORKLOADS",
    "workload",
    "sweep_workloads",
]

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One named attention-forward problem (shapes, dtype, seeds)."""

    name: str
    dtype: str  # storage dtype of q, k, v: "f32" | "bf16" | "f16"
    B: int
    H: int
    N: int  # Nq == Nk for every named workload
    D: int
    causal: bool
    seed: int
    q_mult: float = 1.0
    std: float = 1.0
    sample: Optional[int] = None  # rows checked against the oracle (None = all)
    sample_seed: Optional[int] = None

    @property
    def shape(self) -> Tuple[int, int, int, int]:
        return (self.B, self.H, self.N, self.D)

    @property
    def rows(self) -> int:
        return self.B * self.H * self.N

    def flops(self) -> float:
        """Algorithmic flop count: the two contractions, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.D
        return f / 2 if self.causal else f


def gen_qkv(B: int, H: int, Nq: int, Nk: int, D: int, seed: int,
            dtype: str = "bf16", q_mult: float = 1.0, std: float = 1.0
            ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Return CPU tensors q [B,H,Nq,D], k and v [B,H,Nk,D] in ``dtype``."""
    if dtype not in _DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((B, H, Nq, D), generator=g, dtype=torch.float32)
    k = torch.randn((B, H, Nk, D), generator=g, dtype=torch.float32)
    v = torch.randn((B, H, Nk, D), generator=g, dtype=torch.float32)
    if q_mult != 1.0:
        q.mul_(q_mult)
    if std != 1.0:
        q.mul_(std)
        k.mul_(std)
        v.mul_(std)
    t = _DTYPES[dtype]
    return q.to(t).contiguous(), k.to(t).contiguous(), v.to(t).contiguous()


def gen_grad_out(B: int, H: int, Nq: int, D: int, seed: int, dtype: str = "bf16"
                 ) -> torch.Tensor:
    """Upstream gradient dO [B,H,Nq,D] for the backward pass: i.i.d. N(0,1) in
    fp32 from its own CPU generator (seeded with ``seed``), rounded to
    ``dtype``."""
    if dtype not in _DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    do = torch.randn((B, H, Nq, D), generator=g, dtype=torch.float32)
    return do.to(_DTYPES[dtype]).contiguous()


def varlen_lengths(total: int, S: int, seed: int, min_len: int = 1) -> List[int]:
    """``S`` sequence lengths >= ``min_len`` summing to ``total``: S - 1 cut
    points drawn uniformly (seeded CPU generator) over the spare tokens."""
    spare = total - S * min_len
    if spare < 0:
        raise ValueError("total too small for S sequences of min_len")
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    cuts = torch.randint(0, spare + 1, (S - 1,), generator=g).sort().values.tolist()
    edges = [0] + cuts + [spare]
    return [min_len + b - a for a, b in zip(edges, edges[1:])]


def gen_qkv_fp8(B: int, H: int, Nq: int, Nk: int, D: int, seed: int, q_mult: float = 1.0):
    """FP8 inputs: the fp32 draws of gen_qkv (same recipe and seed), each
    tensor divided by its own factor amax/448 and rounded to OCP e4m3
    (torch.float8_e4m3fn, round to nearest even; 448 is e4m3's largest
    finite value).  Returns (q8, k8, v8, (sq, sk, sv)); the real inputs are
    q8 * sq etc."""
    q, k, v = gen_qkv(B, H, Nq, Nk, D, seed, dtype="f32", q_mult=q_mult)
    out, scales = [], []
    for t in (q, k, v):
        s = float(t.abs().max()) / 448.0
        s = s if s > 0 else 1.0
        out.append((t / s).to(torch.float8_e4m3fn).contiguous())
        scales.append(s)
    return out[0], out[1], out[2], tuple(scales)


def gen_workload(w: Workload):
    return gen_qkv(w.B, w.H, w.N, w.N, w.D, w.seed, w.dtype, w.q_mult, w.std)


def sample_rows(total: int, n: int, seed: int) -> torch.Tensor:
    """``n`` distinct flat row ids in [0, total), sorted (int64, CPU)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    n = min(n, total)
    return torch.randperm(total, generator=g)[:n].sort().values


def _sweep() -> List[Workload]:
    out = []
    idx = 0
    for n in (8192, 16384):
        for d in (16, 32, 64, 128):
            out.append(Workload(f"sweep_n{n}_d{d}", "bf16", 8, 1, n, d, True,
                                seed=40 + idx, sample=256,
                                sample_seed=4000 + idx))
            idx += 1
    return out


WORKLOADS = {
    # single head, fp32, one tile-ish problem
    "f32_n256_d16": Workload("f32_n256_d16", "f32", 1, 1, 256, 16, False, seed=1),
    # fp32, N not a multiple of any tile: ragged tails, both mask modes
    "f32_n1000_d64": Workload("f32_n1000_d64", "f32", 8, 1, 1000, 64, False, seed=2),
    "f32_n1000_d64_causal": Workload("f32_n1000_d64_causal", "f32", 8, 1, 1000, 64,
                                     True, seed=2),
    # the headline problem: bf16, B=8, N=4096, D=128, causal
    "bf16_b8_n4096_d128_causal": Workload("bf16_b8_n4096_d128_causal", "bf16", 8, 1,
                                          4096, 128, True, seed=3),
    # same, with q scaled by 8 (large logits)
    "bf16_b8_n4096_d128_causal_q8": Workload("bf16_b8_n4096_d128_causal_q8", "bf16",
                                             8, 1, 4096, 128, True, seed=3,
                                             q_mult=8.0),
    # multi-head layer, 64 heads at 8K context, N(0, 0.5^2)
    "bf16_h64_n8192_d128_causal": Workload("bf16_h64_n8192_d128_causal", "bf16", 1,
                                           64, 8192, 128, True, seed=5, std=0.5,
                                           sample=4096, sample_seed=5000),
}
for _w in _sweep():
    WORKLOADS[_w.name] = _w

HEADLINE = "bf16_b8_n4096_d128_causal"


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def sweep_workloads() -> List[Workload]:
    return [w for w in WORKLOADS.values() if w.name.startswith("sweep_")]
