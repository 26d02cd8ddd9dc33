"""Seeded synthetic inputs for the fp16 GEMM workloads.

This module only draws random numbers and casts them to fp16; it holds none of the
product's arithmetic, and both the HIP path's tests/benchmark and the CPU oracle
consume the identical fp16 bits it returns.

Recipe (the tutorial draws ``torch.randn(..., dtype=float16)`` operands on the device;
here the draw is made seeded and on the host so both sides see the same bits):
one CPU ``torch.Generator`` per workload, ``manual_seed(seed)``; draw A, then B, then
the bias (only when the workload has an epilogue), each in fp32, then cast to fp16
(round to nearest even).  Distributions:

* ``"normal"``      N(0, 1)               (``torch.randn``)
* ``"uniform"``     U(-1, 1)              (``torch.rand * 2 - 1``)
* ``"normal_rsqrtk"`` N(0, 1) / sqrt(K)   both A and B divided by sqrt(K) in fp32
  before the cast, which keeps |C| near K**-0.5 at large K.
* ``"zeros"``       all zeros (no draw); only for the benchmark's power measurement.

The bias is always N(0, 1), length N.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dist: str
    epilogues: tuple = ("none",)
    seed: int = 0
    note: str = ""

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def algorithmic_bytes(self, epilogue: str) -> int:
        b = 2 * (self.M * self.K + self.K * self.N + self.M * self.N)
        if epilogue != "none":
            b += 2 * self.N
        return b


# The five workloads the tutorial's GEMM is measured on here (shapes from the
# tutorial's 2048^3 benchmark plus a small, a ragged and a large case).
WORKLOADS = [
    Workload("gemm_256", 256, 256, 256, "normal", ("none",), 0,
             "small case: launch-latency bound"),
    Workload("gemm_2048", 2048, 2048, 2048, "normal", ("none",), 0,
             "the tutorial's section 2 / section 3 problem size"),
    Workload("gemm_2048_bias_gelu", 2048, 2048, 2048, "normal", ("bias_gelu",), 0,
             "2048^3 with the fused bias + erf-GELU epilogue"),
    Workload("gemm_ragged_1000x3000x777", 1000, 3000, 777, "uniform", ("bias_gelu",), 0,
             "no dimension a multiple of any tile; A rows only 2-byte aligned"),
    Workload("gemm_8192", 8192, 8192, 8192, "normal_rsqrtk", ("none", "bias_gelu"), 0,
             "large case, run with and without the epilogue"),
]

BY_NAME = {w.name: w for w in WORKLOADS}


def _draw(shape, dist: str, K: int, gen: torch.Generator) -> torch.Tensor:
    if dist == "normal":
        x = torch.randn(shape, generator=gen, dtype=torch.float32)
    elif dist == "uniform":
        x = torch.rand(shape, generator=gen, dtype=torch.float32) * 2.0 - 1.0
    elif dist == "normal_rsqrtk":
        x = torch.randn(shape, generator=gen, dtype=torch.float32) / math.sqrt(K)
    elif dist == "zeros":
        # all-zero operands: the same work with no switching in the multipliers, to show
        # how much of the clock the operand values cost under the power limit
        x = torch.zeros(shape, dtype=torch.float32)
    else:
        raise ValueError("unknown distribution %r" % dist)
    return x.to(torch.float16)


def make_inputs(M: int, N: int, K: int, dist: str = "normal", with_bias: bool = False,
                seed: int = 0):
    """Return (A, B, bias-or-None) as contiguous CPU float16 tensors."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    A = _draw((M, K), dist, K, gen).contiguous()
    B = _draw((K, N), dist, K, gen).contiguous()
    bias = None
    if with_bias:
        bias = torch.randn((N,), generator=gen, dtype=torch.float32).to(torch.float16)
    return A, B, bias


def workload_inputs(w: Workload, with_bias: bool | None = None):
    if with_bias is None:
        with_bias = any(e != "none" for e in w.epilogues)
    return make_inputs(w.M, w.N, w.K, w.dist, with_bias, w.seed)
