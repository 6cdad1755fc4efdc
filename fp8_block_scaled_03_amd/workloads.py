"""Seeded synthetic inputs for the five block-scaled GEMM workloads.

This module only draws random numbers and packs them; it holds none of the
method's arithmetic (no quantization, no GEMM).  It is the one piece shared by
the tests, the bench and the CPU oracle checks: both sides receive identical
bf16 input bytes from here.

Recipe (stated once, used everywhere):
  * every workload i has seed 1000 + i; tensor t of it draws from
    numpy PCG64 seeded with SeedSequence([1000 + i, t]);
  * values are drawn in fp32, then rounded to bf16 (nearest, ties to even) on
    the host - the quantizer's input type;
  * "N(0, s)" means standard deviation s;
  * prefill activations carry outliers: an independent Bernoulli(0.01) mask
    multiplies the affected fp32 draws by 50 before the bf16 rounding;
  * the norm workloads (residual add + RMSNorm + token-group quantization
    ahead of the GEMM, hidden size d = K = 8192) draw the layer output x as
    N(0, 1) with the same outliers, the residual stream as N(0, 1) and the
    norm weight gamma as 1 + N(0, 0.1);
  * grouped workloads draw group sizes in 32-row units from a multinomial over
    the non-empty groups (two groups, chosen by the seeded generator, are forced
    empty), so the stacked A has exactly the stated row count.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

T_A, T_B, T_OUTLIER, T_GROUPS, T_EXTRA, T_RESIDUAL, T_GAMMA = 0, 1, 2, 3, 4, 5, 6


def rng_for(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(tensor_id)]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Host-side input packing: fp32 -> bf16 bit pattern, nearest-even (finite x)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def normal_bf16(seed: int, tensor_id: int, rows: int, cols: int, std: float = 1.0,
                outlier_frac: float = 0.0, outlier_mult: float = 50.0) -> np.ndarray:
    """bf16 bits [rows, cols] of N(0, std) draws (optionally with outliers)."""
    g = rng_for(seed, tensor_id)
    x = g.standard_normal((rows, cols), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if outlier_frac > 0.0:
        m = rng_for(seed, T_OUTLIER).random((rows, cols), dtype=np.float32) < np.float32(outlier_frac)
        x[m] *= np.float32(outlier_mult)
    return f32_to_bf16_bits(x)


def group_rows(seed: int, groups: int, total_rows: int, n_empty: int = 2, unit: int = 32) -> np.ndarray:
    """Row counts per group: multiples of `unit` summing to total_rows, n_empty zeros."""
    if total_rows % unit:
        raise ValueError("total_rows must be a multiple of the unit")
    g = rng_for(seed, T_GROUPS)
    empty = g.choice(groups, size=n_empty, replace=False)
    p = np.ones(groups)
    p[empty] = 0.0
    p /= p.sum()
    counts = g.multinomial(total_rows // unit, p)
    return counts.astype(np.int64) * unit


def offsets_from_rows(rows: np.ndarray) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)


@dataclass
class Workload:
    """One GEMM problem: shapes plus how A and B are drawn."""
    name: str
    index: int
    M: int
    N: int
    K: int
    a_std: float = 1.0
    b_std: float = 1.0
    a_outlier_frac: float = 0.0
    groups: int = 0                      # > 0: grouped GEMM with this many B_g
    extra: dict = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return 1000 + self.index

    def a_bits(self) -> np.ndarray:
        return normal_bf16(self.seed, T_A, self.M, self.K, self.a_std, self.a_outlier_frac)

    def b_bits(self) -> np.ndarray:
        """[K, N] for a plain GEMM, [G, K, N] for a grouped one."""
        if self.groups:
            x = normal_bf16(self.seed, T_B, self.groups * self.K, self.N, self.b_std)
            return x.reshape(self.groups, self.K, self.N)
        return normal_bf16(self.seed, T_B, self.K, self.N, self.b_std)

    def offsets(self) -> np.ndarray:
        if not self.groups:
            raise ValueError("not a grouped workload")
        return offsets_from_rows(group_rows(self.seed, self.groups, self.M))

    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K


def square_256() -> Workload:
    return Workload("square-256", 0, 256, 256, 256)


def square_4096() -> Workload:
    return Workload("square-4096", 1, 4096, 4096, 4096)


def prefill(N: int) -> Workload:
    if N not in (10240, 8192, 28672):
        raise ValueError(N)
    return Workload(f"prefill-M8192-K8192-N{N}", 2, 8192, N, 8192, a_std=1.0, b_std=0.02, a_outlier_frac=0.01)


def decode(M: int, N: int) -> Workload:
    """Decode shapes.  A's draw is row-major, so the first M rows of the M=64
    draw equal the M-row draw; the invariance checks quantize the 64-row A once
    and hand its first M rows (and scale rows) to the M-row GEMM."""
    if M not in (1, 8, 32, 64) or N not in (8192, 28672):
        raise ValueError((M, N))
    return Workload(f"decode-M{M}-K8192-N{N}", 3, M, N, 8192, a_std=1.0, b_std=0.02)


def grouped() -> Workload:
    return Workload("grouped-G16-M8192-K7168-N4096", 4, 8192, 4096, 7168, a_std=1.0, b_std=0.02, groups=16)



@dataclass
class NormWorkload:
    """Rows of a residual add + RMSNorm feeding the GEMM's activations."""
    name: str
    index: int
    rows: int
    d: int
    eps: float = 1e-6

    @property
    def seed(self) -> int:
        return 1000 + self.index

    def x_bits(self) -> np.ndarray:
        return normal_bf16(self.seed, T_A, self.rows, self.d, 1.0, 0.01)

    def residual_bits(self) -> np.ndarray:
        return normal_bf16(self.seed, T_RESIDUAL, self.rows, self.d, 1.0)

    def gamma_bits(self) -> np.ndarray:
        g = rng_for(self.seed, T_GAMMA).standard_normal(self.d, dtype=np.float32)
        return f32_to_bf16_bits(np.float32(1.0) + g * np.float32(0.1))


def norm_prefill() -> NormWorkload:
    return NormWorkload("rmsnorm-M8192-d8192", 5, 8192, 8192)


def norm_decode(M: int) -> NormWorkload:
    """The first M rows of the 64-row draw equal the M-row draw (row-major)."""
    if M not in (1, 8, 32, 64):
        raise ValueError(M)
    return NormWorkload(f"rmsnorm-M{M}-d8192", 6, M, 8192)
