"""The SGEMM workloads: shapes, scalars, seeds and fills.

Each case is a row-major FP32 problem C = alpha*op(A)*op(B) + beta*C with its
stored layouts. The shapes are those of the pages' own measurements and
examples: 1024^3 (itan.pw RTX 4090 page, section 2.1), 1000 x 1300 x 700
(klklkl10086.github.io SGEMM page, section 代码框架), 4096^3 (same page,
problem definition), plus a square sweep, layer-shaped products with every
op pair, and a skinny product whose cost is the stream of B from memory.

Drawing order for uniform fills: srand48(seed), then the stored A in
row-major order, then the stored B, then C_in when beta != 0 (otherwise C_in
is zero and is not read). The integer fill (j - i) % 3 needs no seed.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

from . import Drand48, int_pattern_matrix, random_int_matrix, uniform_matrix


@dataclass(frozen=True)
class Case:
    name: str
    transA: str
    transB: str
    M: int
    N: int
    K: int
    alpha: float
    beta: float
    seed: int
    fill: str = "uniform"          # uniform | int_trunc | int_floor | int_rand
    lda: int | None = None          # None: packed
    ldb: int | None = None
    ldc: int | None = None

    @property
    def a_shape(self) -> tuple[int, int]:
        return (self.M, self.K) if self.transA in "Nn" else (self.K, self.M)

    @property
    def b_shape(self) -> tuple[int, int]:
        return (self.K, self.N) if self.transB in "Nn" else (self.N, self.K)

    @property
    def lda_(self) -> int:
        return self.lda if self.lda is not None else max(1, self.a_shape[1])

    @property
    def ldb_(self) -> int:
        return self.ldb if self.ldb is not None else max(1, self.b_shape[1])

    @property
    def ldc_(self) -> int:
        return self.ldc if self.ldc is not None else max(1, self.N)

    @property
    def flops(self) -> int:
        """2MNK, the FLOP count of the klklkl10086 problem definition."""
        return 2 * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> int:
        """Each operand touched once: 4(MK + KN + MN), plus 4MN when C is read."""
        b = 4 * (self.M * self.K + self.K * self.N + self.M * self.N)
        if self.beta != 0.0:
            b += 4 * self.M * self.N
        return b

    def with_(self, **kw) -> "Case":
        return replace(self, **kw)


@dataclass
class Inputs:
    """Dense logical matrices (float32, packed, C-contiguous)."""
    A: np.ndarray      # stored A (a_shape)
    B: np.ndarray      # stored B (b_shape)
    C: np.ndarray      # C_in, M x N


def make_inputs(case: Case) -> Inputs:
    ar, ac = case.a_shape
    br, bc = case.b_shape
    if case.fill == "uniform":
        g = Drand48(case.seed)
        A = uniform_matrix(g, ar, ac)
        B = uniform_matrix(g, br, bc)
        C = uniform_matrix(g, case.M, case.N) if case.beta != 0.0 else np.zeros((case.M, case.N), np.float32)
    elif case.fill in ("int_trunc", "int_floor"):
        fl = case.fill == "int_floor"
        A = int_pattern_matrix(ar, ac, floored=fl)
        B = int_pattern_matrix(br, bc, floored=fl)
        if case.beta != 0.0:
            C = int_pattern_matrix(case.M, case.N, floored=fl)
        else:
            C = np.zeros((case.M, case.N), np.float32)
    elif case.fill == "int_rand":
        g = Drand48(case.seed)
        A = random_int_matrix(g, ar, ac)
        B = random_int_matrix(g, br, bc)
        C = random_int_matrix(g, case.M, case.N) if case.beta != 0.0 else np.zeros((case.M, case.N), np.float32)
    else:
        raise ValueError(case.fill)
    return Inputs(A, B, C)


# --- the five workload families -------------------------------------------------

C1 = Case("nn_1000x1300x700", "N", "N", 1000, 1300, 700, 1.0, 0.0, seed=1)
C2 = Case("nn_1024", "N", "N", 1024, 1024, 1024, 1.0, 0.0, seed=2)
C2_INT = C2.with_(name="nn_1024_int", fill="int_trunc")
C3_SIZES = tuple(range(256, 4096 + 1, 256))


def c3(n: int) -> Case:
    return Case(f"nn_sweep_{n}", "N", "N", n, n, n, 1.5, 0.5, seed=3)


C4 = Case("nn_4096", "N", "N", 4096, 4096, 4096, 1.0, 0.0, seed=4)
C5A = tuple(Case(f"{ta}{tb}_2048x4096x1024".lower(), ta, tb, 2048, 4096, 1024, 1.0, 1.0, seed=5)
            for ta in "NT" for tb in "NT")
C5B = Case("nn_skinny_16x4096x4096", "N", "N", 16, 4096, 4096, 1.0, 1.0, seed=5)

# One GPU's share of C4 and C5b split eight ways (rows of C4, columns of C5b):
# the shard shapes a multi-GPU run would hand each device.
SHARD8 = (Case("nn_shard8_512x4096x4096", "N", "N", 512, 4096, 4096, 1.0, 0.0, seed=4),
          Case("nn_skinny_shard8_16x512x4096", "N", "N", 16, 512, 4096, 1.0, 1.0, seed=5))

HEADLINE = C4


def all_cases() -> list[Case]:
    return [C1, C2, C2_INT, *[c3(n) for n in C3_SIZES], C4, *C5A, C5B]
