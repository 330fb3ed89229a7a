"""Seeded synthetic inputs for the FP32 SGEMM workloads.

This module only draws numbers and lays them out; it holds none of the
GEMM arithmetic. Both sides of every parity check (the CPU oracle and the
HIP library) take their inputs from here.

Uniform inputs follow the harness of "【CUDA】Sgemm单精度矩阵乘法"
(klklkl10086.github.io, section 代码框架): values from the POSIX
``drand48`` stream mapped to [-1, 1), matrix A drawn first, then B, each in
row-major order. Two readings are fixed here because the page leaves them
open:

* the stream is seeded with ``srand48(seed)`` (the page never seeds it);
* each draw is quantised to the 2**-23 grid before the shift, i.e.
  ``floor(drand48() * 2**24) * 2**-23 - 1``, so every value is exact in
  FP32 and strictly below 1 (``2*drand48()-1`` rounded to float can reach
  1.0f).

The integer variant is the same page's alternative fill ``(j - i) % 3``
evaluated with C's truncating remainder (values -2..2); the floored
reading ``(j - i) mod 3`` (values 0..2) is offered too.

drand48 is the 48-bit linear congruential generator defined by POSIX:
``X[n+1] = (0x5DEECE66D * X[n] + 0xB) mod 2**48``, ``srand48(s)`` sets
``X[0] = (s mod 2**32) * 2**16 + 0x330E`` and ``drand48()`` advances once
and returns ``X / 2**48``. Long runs are produced here with the closed-form
jump ``X[n+L] = a^L X[n] + c (a^L - 1)/(a - 1)`` so that a 4096 x 4096
matrix is drawn with a handful of vector operations.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "Drand48",
    "uniform_matrix",
    "int_pattern_matrix",
    "padded",
]

_A = 0x5DEECE66D
_C = 0xB
_MASK = (1 << 48) - 1


def _jump(length: int) -> tuple[int, int]:
    """Return (a^L mod 2^48, c(1+a+...+a^(L-1)) mod 2^48) for L = length."""
    mul, add = 1, 0
    base_mul, base_add = _A, _C
    n = length
    while n:
        if n & 1:
            # compose (mul, add) after (base_mul, base_add)
            mul, add = (mul * base_mul) & _MASK, (add * base_mul + base_add) & _MASK
        base_mul, base_add = (base_mul * base_mul) & _MASK, (base_add * base_mul + base_add) & _MASK
        n >>= 1
    return mul, add


class Drand48:
    """POSIX drand48 stream with a vectorised bulk draw."""

    def __init__(self, seed: int):
        self.state = (((int(seed) & 0xFFFFFFFF) << 16) | 0x330E) & _MASK

    def next_states(self, count: int) -> np.ndarray:
        """Advance ``count`` times; return the states X[1..count] (uint64)."""
        if count <= 0:
            return np.zeros(0, dtype=np.uint64)
        out = np.empty(count, dtype=np.uint64)
        out[0] = ((_A * self.state) + _C) & _MASK
        filled = 1
        mask = np.uint64(_MASK)
        while filled < count:
            take = min(filled, count - filled)
            mul, add = _jump(filled)
            # uint64 products wrap modulo 2**64, which keeps the low 48 bits exact.
            np.multiply(out[:take], np.uint64(mul), out=out[filled:filled + take])
            out[filled:filled + take] += np.uint64(add)
            out[filled:filled + take] &= mask
            filled += take
        self.state = int(out[-1])
        return out

    def drand48(self, count: int) -> np.ndarray:
        """``count`` successive drand48() values as float64."""
        return self.next_states(count).astype(np.float64) * (2.0 ** -48)

    def uniform_f32(self, rows: int, cols: int) -> np.ndarray:
        """rows x cols float32, row-major, values floor(u*2^24)*2^-23 - 1."""
        top24 = (self.next_states(rows * cols) >> np.uint64(24)).astype(np.int64)
        vals = (top24 - (1 << 23)).astype(np.float32) * np.float32(2.0 ** -23)
        return vals.reshape(rows, cols)


def uniform_matrix(gen: Drand48, rows: int, cols: int) -> np.ndarray:
    """Next rows x cols block of the stream (see module docstring)."""
    return gen.uniform_f32(rows, cols)


def int_pattern_matrix(rows: int, cols: int, floored: bool = False) -> np.ndarray:
    """Integer-valued fill (j - i) % 3 over the stored matrix's own indices.

    ``floored=False`` is C's truncating remainder (sign follows j - i);
    ``floored=True`` is the mathematical mod with values 0..2.
    """
    i = np.arange(rows, dtype=np.int64)[:, None]
    j = np.arange(cols, dtype=np.int64)[None, :]
    d = j - i
    r = np.mod(d, 3) if floored else np.fmod(d, 3)
    return r.astype(np.float32)


def random_int_matrix(gen: Drand48, rows: int, cols: int, lo: int = -4, hi: int = 4) -> np.ndarray:
    """Integer values uniform in [lo, hi], drawn from the same stream."""
    u = gen.drand48(rows * cols)
    vals = np.floor(u * (hi - lo + 1)).astype(np.int64) + lo
    return vals.astype(np.float32).reshape(rows, cols)


def padded(mat: np.ndarray, ld: int, fill: float = 0.0, extra_rows: int = 0) -> np.ndarray:
    """Copy ``mat`` into a rows x ld buffer (plus guard rows) filled with ``fill``.

    Returns the padded buffer; the logical matrix is ``buf[:rows, :cols]``.
    """
    rows, cols = mat.shape
    if ld < cols:
        raise ValueError("ld must be >= cols")
    buf = np.full((rows + extra_rows, ld), fill, dtype=np.float32)
    buf[:rows, :cols] = mat
    return buf
