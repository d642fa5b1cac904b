"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the attention arithmetic, and both sides use it: the GPU
tests and bench, and the CPU oracle checks.

Recipe (all on the CPU, independent of any GPU):
  * ``g = torch.Generator().manual_seed(seed)``.
  * Q, K, V (then dO when a backward is wanted) are drawn in that order as
    float32 ``randn`` of shape [B, H, N, d].
  * Large-logit stress (``big_frac > 0``): for each (b, h) in row-major order
    one ``randperm(N)`` is drawn and the K rows at its first
    ``round(big_frac * N)`` entries are multiplied by ``big_scale`` (before
    rounding).
  * Every tensor is then rounded to the storage dtype with round-to-nearest-
    even (``.to(dtype)``).

The five workloads are sized after the pages' own examples: the B=2, N=1024,
d=128 causal call of the snabindia page (chapter 1); the 4096 x 64 blocking
of the yunthe page (section 2.1); the sequence-length-8192 comparison table
of the snabindia page (chapter 1); and the N=16384, 8-head case of the
hotdry blog's bandwidth-bottleneck section.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "f16" or "bf16"
    causal: bool
    backward: bool      # the workload includes the backward pass
    big_frac: float = 0.0
    big_scale: float = 1.0

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]

    def pairs_per_head(self) -> int:
        """Unmasked (query, key) pairs of one head."""
        n = self.N
        return n * (n + 1) // 2 if self.causal else n * n


WORKLOADS = [
    Workload("fwd_B1_H2_N256_d64_f16", 1, 2, 256, 64, "f16", False, False),
    Workload("fwd_B2_H16_N1024_d128_f16_causal", 2, 16, 1024, 128, "f16", True, False),
    Workload("fwd_B4_H16_N4096_d64_bf16_bigK", 4, 16, 4096, 64, "bf16", False, False, 0.01, 20.0),
    Workload("fwdbwd_B1_H32_N8192_d128_bf16_causal", 1, 32, 8192, 128, "bf16", True, True),
    Workload("fwdbwd_B1_H8_N16384_d64_f16", 1, 8, 16384, 64, "f16", False, True),
]


def workload_seed(index: int) -> int:
    return 1000 + index


def default_scale(d: int) -> float:
    """1/sqrt(d), rounded to float32 (the value both sides receive)."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32).item())


def make_inputs(B: int, H: int, N: int, d: int, dtype: str, seed: int,
                with_dout: bool = False, big_frac: float = 0.0, big_scale: float = 1.0):
    """Return a dict of CPU tensors q, k, v (and dout) in the storage dtype."""
    g = torch.Generator().manual_seed(seed)
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    dout = torch.randn(shape, generator=g, dtype=torch.float32) if with_dout else None
    nbig = int(round(big_frac * N))
    if nbig > 0:
        for b in range(B):
            for h in range(H):
                idx = torch.randperm(N, generator=g)[:nbig]
                k[b, h, idx] *= big_scale
    dt = DTYPES[dtype]
    out = {"q": q.to(dt), "k": k.to(dt), "v": v.to(dt)}
    if dout is not None:
        out["dout"] = dout.to(dt)
    return out


def workload_inputs(index: int):
    """Inputs of workload ``index`` (0-based) with its fixed seed."""
    w = WORKLOADS[index]
    return make_inputs(w.B, w.H, w.N, w.d, w.dtype, workload_seed(index),
                       with_dout=w.backward, big_frac=w.big_frac, big_scale=w.big_scale)
