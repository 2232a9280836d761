"""Seeded synthetic workloads for the persistent tile-scheduled GEMM.

This module only describes shapes and draws seeded random inputs; it holds none
of the GEMM's arithmetic.  Both the HIP-path tests/benchmark and the CPU oracle
consume the arrays it returns, so the two sides always see identical inputs.

Recipe: NumPy ``default_rng(seed)`` (PCG64) draws A in full row-major order,
then B, in binary64; the draws are rounded to the compute dtype with torch's
``Tensor.to``; the *rounded* arrays are what both sides receive.
Distributions: uniform on [-1, 1] for the fp16 shapes, normal(0, 1)/sqrt(K) for
the bf16 shapes.

Block-scaled FP8 (MX) inputs: the same generator draws A[M,K] then B[N,K] in
binary64 (normal(0, 1), optionally times 2^u per 32-element block with u
uniform on the integers [-spread, spread]) and encodes them the way the OCP
Microscaling Formats specification v1.0 converts a vector to MX: per block of
32 along K the shared exponent is floor(log2(max |v|)) - 8 (8 = largest E4M3
exponent), clamped to [-127, 127] (-127 for an all-zero block), and every
element v / 2^shared is rounded to E4M3 (nearest, ties to even, torch's cast)
after saturation to +-448.  Both sides receive the uint8 element and scale
codes; the encoding is input preparation only.
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


# ---------------------------------------------------------------- MX (block-scaled FP8)
@dataclasses.dataclass(frozen=True)
class MxWorkload:
    name: str
    M: int
    N: int
    K: int
    group_size: int
    num_workgroups: int   # 0 = one per compute unit
    seed: int
    spread: int = 0       # per-block extra exponent range of the drawn values

    block_M = 256
    block_N = 256
    block_K = 128
    num_stages = 2
    dtype = "mxfp8"

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> int:
        # E4M3 elements and E8M0 scales of A and B read once, bf16 C written once
        return self.M * self.K + self.N * self.K + (self.M + self.N) * (self.K // 32) + 2 * self.M * self.N


MX_WORKLOADS = {
    "mx_8192_mxfp8": MxWorkload("mx_8192_mxfp8", 8192, 8192, 8192, 8, 0, 6),
}


def mx_encode(x: np.ndarray, rng: np.random.Generator | None = None, spread: int = 0):
    """Binary64 x[rows, K] (K % 32 == 0) -> (E4M3 codes uint8[rows, K],
    E8M0 scale codes uint8[rows, K/32]); see the module docstring."""
    rows, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    blocks = x.reshape(rows, K // 32, 32)
    if spread:
        blocks = blocks * np.exp2(rng.integers(-spread, spread + 1, size=(rows, K // 32, 1)))
    amax = np.abs(blocks).max(axis=-1)
    with np.errstate(divide="ignore"):
        shared = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, -127)
    shared = np.clip(shared, -127, 127)
    scaled = np.clip(blocks / np.exp2(shared)[..., None], -448.0, 448.0)
    codes = torch.from_numpy(np.ascontiguousarray(scaled)).to(torch.float8_e4m3fn).view(torch.uint8)
    return (codes.reshape(rows, K).numpy().copy(),
            (shared + 127).astype(np.uint8))


def make_mx_inputs(M: int, N: int, K: int, seed: int, spread: int = 0):
    """Seeded MX operands (A codes [M,K], SFA [M,K/32], B codes [N,K], SFB [N,K/32]), numpy uint8."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=(M, K))
    b = rng.standard_normal(size=(N, K))
    A, SFA = mx_encode(a, rng, spread)
    B, SFB = mx_encode(b, rng, spread)
    return A, SFA, B, SFB


def mx_workload_inputs(w: MxWorkload):
    return make_mx_inputs(w.M, w.N, w.K, w.seed, w.spread)
