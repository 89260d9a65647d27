"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no GEMM arithmetic.  It only draws random operands (as raw
16-bit patterns) and picks sample coordinates, so that the HIP path and the
CPU oracle are fed the same host bits.

Workloads follow the sizes, layouts and value distributions of the dense
half-precision GEMM configurations this library is measured on: square sweeps
at 512, 2048, 4096 and 8192 and a long-K 8192 x 8192 x 16384 case (the size
the "MTT S4000 张量核心 GEMM 优化…" post optimises for, section 1).  The pages
state no value distributions, so uniform and normal draws stand in.

Recipe:
  * generator: numpy ``Generator(PCG64(seed))``, A seed ``1000 + i``,
    B seed ``2000 + i`` for workload index ``i``;
  * fp16: float64 draws, converted with ``astype(float16)`` (round to nearest
    even);
  * bf16: float32 draws, rounded to bfloat16 by round-to-nearest-even on the
    float32 bit pattern;
  * TN: ``A[M, K]`` and ``Bt[N, K]`` row-major; NN: ``A[M, K]``, ``B[K, N]``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    index: int
    layout: str  # "tn" or "nn"
    dtype: str  # "f16" or "bf16"
    M: int
    N: int
    K: int
    dist: str  # "uniform" or "normal"
    lo: float = -1.0
    hi: float = 1.0

    @property
    def name(self) -> str:
        return f"hgemm_{self.layout}_{self.dtype}_{self.M}x{self.N}x{self.K}"

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> int:
        """Each operand read once, C written once (2-byte elements)."""
        return 2 * (self.M * self.K + self.K * self.N + self.M * self.N)

    def describe(self) -> str:
        d = (f"uniform[{self.lo:g},{self.hi:g}]" if self.dist == "uniform" else "normal(0,1)")
        lay = ("A[M,K] row-major, Bt[N,K] row-major" if self.layout == "tn"
               else "A[M,K] row-major, B[K,N] row-major")
        return (f"HGEMM {self.layout.upper()} M={self.M} N={self.N} K={self.K} {self.dtype} "
                f"({lay}), entries {d} rounded to {self.dtype}, fp32 accumulate, "
                f"{self.dtype} output")


WORKLOADS = (
    Workload(1, "tn", "f16", 512, 512, 512, "uniform", -1.0, 1.0),
    Workload(2, "tn", "f16", 2048, 2048, 2048, "uniform", -1.0, 1.0),
    Workload(3, "nn", "bf16", 4096, 4096, 4096, "normal"),
    Workload(4, "tn", "f16", 8192, 8192, 8192, "uniform", -1.0, 1.0),
    Workload(5, "tn", "f16", 8192, 8192, 16384, "uniform", -0.5, 0.5),
)


def workload(index: int) -> Workload:
    return WORKLOADS[index - 1]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); finite input."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def draw(shape, dtype: str, dist: str, seed: int, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    """Seeded random matrix as 16-bit patterns (uint16) of ``dtype``."""
    g = np.random.Generator(np.random.PCG64(seed))
    if dtype in ("f16", "fp16"):
        x = g.uniform(lo, hi, size=shape) if dist == "uniform" else g.standard_normal(size=shape)
        return x.astype(np.float16).view(np.uint16)
    if dtype in ("bf16",):
        if dist == "uniform":
            x = g.uniform(lo, hi, size=shape).astype(np.float32)
        else:
            x = g.standard_normal(size=shape, dtype=np.float32)
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype}")


def operands(w: Workload, M: int | None = None, N: int | None = None, K: int | None = None,
             seed_offset: int = 0):
    """(A, B) bit patterns for workload ``w`` (optionally at another shape).

    TN returns ``(A[M,K], Bt[N,K])``; NN returns ``(A[M,K], B[K,N])``.
    """
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    A = draw((M, K), w.dtype, w.dist, 1000 + w.index + seed_offset, w.lo, w.hi)
    bshape = (N, K) if w.layout == "tn" else (K, N)
    B = draw(bshape, w.dtype, w.dist, 2000 + w.index + seed_offset, w.lo, w.hi)
    return A, B


def stratified_samples(M: int, N: int, seed: int, bands: int = 64):
    """One uniformly drawn (row, col) in each cell of a bands x bands grid.

    Rows and columns are each cut into ``bands`` nearly equal bands, so every
    output tile of at least (M/bands) x (N/bands) elements is hit.  Returns
    (rows, cols) as int64 arrays of length bands_m * bands_n.
    """
    g = np.random.Generator(np.random.PCG64(seed))
    bm, bn = min(bands, M), min(bands, N)
    re = np.linspace(0, M, bm + 1).astype(np.int64)
    ce = np.linspace(0, N, bn + 1).astype(np.int64)
    rows, cols = [], []
    for i in range(bm):
        for j in range(bn):
            rows.append(g.integers(re[i], re[i + 1]))
            cols.append(g.integers(ce[j], ce[j + 1]))
    return np.asarray(rows, dtype=np.int64), np.asarray(cols, dtype=np.int64)


SAMPLE_SEED_BASE = 0x5EED
