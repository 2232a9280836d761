"""Seeded synthetic workloads for the persistent tile-scheduled GEMM.

This module only describes shapes and draws seeded random inputs; it holds none
of the GEMM's arithmetic.  Both the HIP-path tests/benchmark and the CPU oracle
consume the arrays it returns, so the two sides always see identical inputs.

Recipe: NumPy ``default_rng(seed)`` (PCG64) draws A in full row-major order,
then B, in binary64; the draws are rounded to the compute dtype with torch's
``Tensor.to``; the *rounded* arrays are what both sides receive.
Distributions: uniform on [-1, 1] for the fp16 shapes, normal(0, 1)/sqrt(K) for
the bf16 shapes.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dtype: str            # "fp16" or "bf16" (inputs and output)
    dist: str             # "uniform" or "normal_sqrtk"
    block_M: int
    block_N: int
    block_K: int
    group_size: int
    num_stages: int
    num_workgroups: int   # 0 = one per compute unit
    seed: int

    @property
    def torch_dtype(self):
        return torch.float16 if self.dtype == "fp16" else torch.bfloat16

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> int:
        return 2 * (self.M * self.K + self.K * self.N + self.M * self.N)


# The five benchmark shapes plus the ragged variant of the fourth.
WORKLOADS = {
    "cfg1_512_fp16": Workload("cfg1_512_fp16", 512, 512, 512, "fp16", "uniform",
                              128, 128, 64, 2, 2, 8, 1),
    "cfg2_1024_fp16": Workload("cfg2_1024_fp16", 1024, 1024, 1024, "fp16", "uniform",
                               128, 128, 32, 4, 3, 0, 2),
    "cfg3_8192_bf16": Workload("cfg3_8192_bf16", 8192, 8192, 8192, "bf16", "normal_sqrtk",
                               256, 256, 64, 8, 3, 0, 3),
    "cfg4_16384x4096x4096_fp16": Workload("cfg4_16384x4096x4096_fp16", 16384, 4096, 4096, "fp16",
                                          "uniform", 256, 256, 64, 8, 3, 0, 4),
    "cfg4p_16000x4000x4096_fp16": Workload("cfg4p_16000x4000x4096_fp16", 16000, 4000, 4096, "fp16",
                                           "uniform", 256, 256, 64, 8, 3, 0, 40),
    "cfg5_2048x2048x32768_bf16": Workload("cfg5_2048x2048x32768_bf16", 2048, 2048, 32768, "bf16",
                                          "normal_sqrtk", 256, 256, 32, 4, 4, 0, 5),
}


def draw(rng: np.random.Generator, shape, dist: str, K: int) -> np.ndarray:
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, size=shape)
    if dist == "normal_sqrtk":
        return rng.standard_normal(size=shape) / math.sqrt(K)
    raise ValueError(f"unknown distribution {dist!r}")


def make_inputs(M: int, N: int, K: int, dtype: str, dist: str, seed: int):
    """Seeded A[M,K], B[K,N] as contiguous CPU tensors of the compute dtype."""
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    rng = np.random.default_rng(seed)
    a = torch.from_numpy(draw(rng, (M, K), dist, K)).to(tdt).contiguous()
    b = torch.from_numpy(draw(rng, (K, N), dist, K)).to(tdt).contiguous()
    return a, b


def workload_inputs(w: Workload):
    return make_inputs(w.M, w.N, w.K, w.dtype, w.dist, w.seed)
