"""Seeded synthetic inputs for the dense fp16 NT GEMM C = A @ B.T.

This module only draws random numbers; it holds none of the GEMM's
arithmetic.  Both the CPU oracle and the HIP path take their inputs from
here, so the two sides always see the same bits.

Recipe (the same for every workload): ``np.random.default_rng(seed)`` (PCG64);
A [M, K] is drawn first, then B [N, K], each in one call, in fp64, scaled,
then cast to fp16 with numpy's round-to-nearest-even ``astype``.

The pages time one synthetic square problem, M = N = K = 8192 (Tilus "Hopper
matmul" pages, "4. Pipeline Abstraction and Two Consumer Warp Groups" /
Performance, and "6. Register Reallocation, Multicast, and a Persistent
Kernel" / Performance), and state no input distribution; the only
distribution they mention is unit-variance outputs over a K = 8192 reduction
(page 6, note in "Shared-Memory Epilogue").  No public dataset is involved.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dist: str        # "uniform" | "int2" | "normal"
    scale: float     # multiplies every drawn value before the fp16 cast
    seed: int
    note: str = ""

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> int:
        """Read A and B once, write C once (fp16 everywhere)."""
        return 2 * (self.M * self.K + self.N * self.K + self.M * self.N)


def _inv_sqrt(k: int) -> float:
    return 1.0 / math.sqrt(k)


#: The five workloads: shapes, distributions and seeds.
WORKLOADS = {
    w.name: w
    for w in (
        Workload("square256", 256, 256, 256, "uniform", 1.0, 101,
                 "entries uniform in [-1, 1]"),
        Workload("square4096_int", 4096, 4096, 4096, "int2", 1.0, 102,
                 "entries uniform integers in {-2..2}: every partial sum is exact"),
        Workload("square8192", 8192, 8192, 8192, "uniform", _inv_sqrt(8192), 103,
                 "entries uniform in [-1, 1]/sqrt(K): the headline compute-bound shape"),
        Workload("ragged4999x7001x4160", 4999, 7001, 4160, "normal", _inv_sqrt(4160), 104,
                 "entries normal(0, 1)/sqrt(K): M/N tails and a raster remainder group"),
        Workload("skinny128x16384x16384", 128, 16384, 16384, "uniform", _inv_sqrt(16384), 105,
                 "entries uniform in [-1, 1]/sqrt(K): B dominates the traffic"),
    )
}

#: A shape beyond the five: an output whose tiles leave most compute units
#: idle (16 tiles of 256 x 256) over a long reduction, the case the split over
#: K is for.  Not a workload of the pages.
EXTRA_WORKLOADS = {
    w.name: w
    for w in (
        Workload("underfilled1024x1024x65536", 1024, 1024, 65536, "uniform", _inv_sqrt(65536),
                 106, "entries uniform in [-1, 1]/sqrt(K): few output tiles, a long K"),
    )
}

#: One row of A against a B of 4096 x 14336 (a matrix-vector product, 117 MB
#: of B streamed once): the few-rows-of-A case, where the GEMM is bound by
#: HBM and the plan streams B through registers.  Not a workload of the pages.
FEW_ROWS_WORKLOADS = {
    w.name: w
    for w in (
        Workload("gemv1x4096x14336", 1, 4096, 14336, "uniform", _inv_sqrt(14336), 107,
                 "entries uniform in [-1, 1]/sqrt(K): one row of A, B streamed from HBM"),
    )
}

ALL_WORKLOADS = {**WORKLOADS, **EXTRA_WORKLOADS, **FEW_ROWS_WORKLOADS}

#: The workload the benchmark times.
HEADLINE = "square8192"


def draw(rng: np.random.Generator, shape, dist: str, scale: float) -> np.ndarray:
    """One matrix of the given distribution, scaled in fp64, rounded to fp16."""
    if dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size=shape)
    elif dist == "normal":
        x = rng.standard_normal(size=shape)
    elif dist == "int2":
        x = rng.integers(-2, 3, size=shape).astype(np.float64)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    if scale != 1.0:
        x = x * scale
    return x.astype(np.float16)


def int2_matrix(shape, seed: int) -> np.ndarray:
    """Integers in {-2..2} as fp16, drawn through int8: for matrices of more
    than 2^31 bytes, where draw()'s fp64 intermediate would take 4x the
    memory.  Its own stream (not draw(..., "int2"))."""
    rng = np.random.default_rng(seed)
    return rng.integers(-2, 3, size=shape, dtype=np.int8).astype(np.float16)


def make_inputs(M: int, N: int, K: int, dist: str = "uniform", scale: float = 1.0,
                seed: int = 0):
    """A [M, K] and B [N, K] as fp16 numpy arrays; A is drawn before B."""
    rng = np.random.default_rng(seed)
    a = draw(rng, (M, K), dist, scale)
    b = draw(rng, (N, K), dist, scale)
    return a, b


def workload_inputs(name: str):
    w = ALL_WORKLOADS[name]
    return make_inputs(w.M, w.N, w.K, w.dist, w.scale, w.seed)
