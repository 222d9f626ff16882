"""Seeded synthetic f32 inputs for the Q8_0 contraction workloads.

This module only draws random numbers: it holds none of the contraction's
arithmetic and no quantizer.  The oracle (CPU) and the GPU library each
quantize what it returns with their own code.

Workloads (LLM projection shapes: hidden size 4096, FFN width 14336):

===  ========================  =====================================
cfg  M x N x K                 values
===  ========================  =====================================
0    1 x 4096 x 4096            W ~ N(0, 0.02), A ~ N(0, 1)
1    1 x 14336 x 4096           same (FFN up-projection shape)
2    1 x 4096 x 14336           same, plus outliers in A (down-projection)
3    64 x 4096 x 4096           same
4    512 x 14336 x 4096         same (prompt-size projection)
===  ========================  =====================================

Recipe: NumPy ``default_rng(seed)`` (PCG64), ``standard_normal(dtype=float32)``,
W scaled by the standard deviation 0.02 in f32; W seed ``1000 + cfg``, A seed
``2000 + cfg``.  Outliers: in each A row, ``floor(0.01 * K)`` positions drawn
without replacement from ``default_rng(3000 + cfg)`` are multiplied by 20.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    M: int
    N: int
    K: int
    outliers: bool

    @property
    def KB(self) -> int:
        return self.K // 32


WORKLOADS = (
    Workload(0, "q8_matvec_m1_n4096_k4096", 1, 4096, 4096, False),
    Workload(1, "q8_matvec_m1_n14336_k4096", 1, 14336, 4096, False),
    Workload(2, "q8_matvec_m1_n4096_k14336_outliers", 1, 4096, 14336, True),
    Workload(3, "q8_qgemm_m64_n4096_k4096", 64, 4096, 4096, False),
    Workload(4, "q8_qgemm_m512_n14336_k4096", 512, 14336, 4096, False),
)

W_STD = np.float32(0.02)
OUTLIER_FRACTION = 0.01
OUTLIER_FACTOR = np.float32(20.0)


def weights_f32(N: int, K: int, seed: int, std=W_STD) -> np.ndarray:
    """``[N, K]`` f32 draws of N(0, std) from ``default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(std)
    return w


def activations_f32(M: int, K: int, seed: int, outlier_seed: int | None = None) -> np.ndarray:
    """``[M, K]`` f32 draws of N(0, 1); optionally 1 % of each row's entries x20."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((M, K), dtype=np.float32)
    if outlier_seed is not None:
        orng = np.random.default_rng(outlier_seed)
        count = int(np.floor(OUTLIER_FRACTION * K))
        for i in range(M):
            pos = orng.choice(K, size=count, replace=False)
            a[i, pos] *= OUTLIER_FACTOR
    return a


def workload_f32(w: Workload, M: int | None = None, N: int | None = None):
    """The f32 operands of workload ``w``: ``(A [M,K], W [N,K])``.

    ``M``/``N`` override the row counts (same seeds, fewer rows) for checks
    that sample a full-size workload.
    """
    M = w.M if M is None else M
    N = w.N if N is None else N
    W = weights_f32(N, w.K, 1000 + w.index)
    A = activations_f32(M, w.K, 2000 + w.index, (3000 + w.index) if w.outliers else None)
    return A, W


def random_f32(shape, seed: int, std: float = 1.0) -> np.ndarray:
    """Generic seeded N(0, std) f32 array for edge-case tests."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def random_i8(shape, seed: int, low: int = -128, high: int = 127) -> np.ndarray:
    """Seeded uniform int8 in ``[low, high]`` (raw Q8_0 bytes, -128 included)."""
    rng = np.random.default_rng(seed)
    return rng.integers(low, high + 1, size=shape, dtype=np.int16).astype(np.int8)


def random_scales(shape, seed: int, lo: float = 1e-3, hi: float = 1e-1) -> np.ndarray:
    """Seeded positive f32 scales, log-uniform in ``[lo, hi]``."""
    rng = np.random.default_rng(seed)
    e = rng.uniform(np.log(lo), np.log(hi), size=shape)
    return np.exp(e).astype(np.float32)


def random_q50(rows: int, K: int, seed: int) -> np.ndarray:
    """Seeded uniform bytes shaped as Q5_0 weight rows, ``uint8 [rows, K/32 * 20]``.

    Every byte pattern is a valid Q5_0 block (qh word + 16 nibble bytes), so
    uniform bytes give uniform 5-bit codes.
    """
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, size=(rows, K // 32 * 20), dtype=np.uint8)


def cancelling_blocks(M: int, N: int, K: int, seed: int):
    """Operands whose half-block sums are large and cancel within each block.

    Every activation block repeats its first 16 bytes in its second half;
    every weight block's second half is the negated first half with one byte
    moved by one.  The two half-block dot products are then +-(65..260)
    thousand while the block sum P (exact in int32) is a single a*(+-1)
    term, so |P| <= 127.  The contraction's tolerance scales with
    sum_b |AS*WS*P|, so arithmetic that scaled and rounded half-block sums
    before forming P misses it on most outputs.  Only byte patterns and
    seeded scales are made here; nothing of the contraction is computed.
    """
    rng = np.random.default_rng(seed)
    KB = K // 32
    # magnitudes 64..127 with one sign per (block, position) shared by A and
    # W, so every half-block product is positive and the halves are large
    sign = np.where(rng.random((1, KB, 16)) < 0.5, -1, 1).astype(np.int16)
    a = sign * rng.integers(64, 128, size=(M, KB, 16), dtype=np.int16)
    w = sign * rng.integers(64, 128, size=(N, KB, 16), dtype=np.int16)
    A = np.concatenate([a, a], axis=2).reshape(M, K).astype(np.int8)
    w_hi = -w
    w_hi[:, :, 0] = np.where(w_hi[:, :, 0] < 127, w_hi[:, :, 0] + 1, w_hi[:, :, 0] - 1)
    W = np.concatenate([w, w_hi], axis=2).reshape(N, K).astype(np.int8)
    AS = random_scales((M, KB), seed + 1, 1e-3, 1.0)
    WS = random_scales((N, KB), seed + 2, 1e-3, 1.0)
    return A, AS, W, WS
