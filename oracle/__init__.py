"""CPU oracle for FP32 SGEMM (FP64 accumulation), loaded with ctypes.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this package. It shares no code with
the HIP library (fp32_gemm_nn_amd) and never imports it.

The arithmetic lives in oracle/sgemm_oracle.c; this file only marshals numpy
arrays into its two entry points.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    _lib = _configure(ctypes.CDLL(_LIB_PATH))
    return _lib


def _configure(lib):
    f = ctypes.c_float
    i = ctypes.c_int
    p = ctypes.c_void_p
    c = ctypes.c_char
    lib.oracle_sgemm.argtypes = [c, c, i, i, i, f, p, i, p, i, f, p, i]
    lib.oracle_sgemm.restype = i
    lib.oracle_sgemm_entries.argtypes = [c, c, i, i, i, f, p, i, p, i, f, p, i, p, p, p]
    lib.oracle_sgemm_entries.restype = i
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i
    return lib


def _ptr(a):
    if a is None:
        return None
    assert a.dtype == np.float32 and a.flags.c_contiguous
    return a.ctypes.data


def _ch(t) -> bytes:
    return t.encode() if isinstance(t, str) else bytes(t)


def sgemm(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc) -> int:
    """C <- alpha*op(A)*op(B) + beta*C in place on float32 numpy buffers.

    A, B, C are C-contiguous float32 arrays holding the stored matrices with
    leading dimensions lda, ldb, ldc (elements). Returns the status code.
    """
    lib = _load()
    return lib.oracle_sgemm(_ch(transA), _ch(transB), int(M), int(N), int(K), float(alpha),
                            _ptr(A), int(lda), _ptr(B), int(ldb), float(beta), _ptr(C), int(ldc))


def sgemm_entries(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, c_in, rows, cols):
    """Oracle outputs at positions (rows[p], cols[p]) only; returns float32 array."""
    lib = _load()
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    cols = np.ascontiguousarray(cols, dtype=np.int32)
    out = np.zeros(rows.shape[0], dtype=np.float32)
    cin = None if c_in is None else np.ascontiguousarray(c_in, dtype=np.float32)
    rc = lib.oracle_sgemm_entries(_ch(transA), _ch(transB), int(M), int(N), int(K), float(alpha),
                                  _ptr(A), int(lda), _ptr(B), int(ldb), float(beta), _ptr(cin),
                                  int(rows.shape[0]), rows.ctypes.data, cols.ctypes.data,
                                  out.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_sgemm_entries returned {rc}")
    return out


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def matmul(transA, transB, alpha, A, B, beta=0.0, C=None):
    """Convenience: dense packed operands; returns a new float32 C (M x N).

    A is the stored matrix (M x K for 'N', K x M for 'T'); likewise B.
    """
    A = np.ascontiguousarray(A, dtype=np.float32)
    B = np.ascontiguousarray(B, dtype=np.float32)
    M = A.shape[0] if transA in "Nn" else A.shape[1]
    K = A.shape[1] if transA in "Nn" else A.shape[0]
    N = B.shape[1] if transB in "Nn" else B.shape[0]
    out = np.zeros((M, N), dtype=np.float32) if C is None else np.array(C, dtype=np.float32, copy=True)
    rc = sgemm(transA, transB, M, N, K, alpha, A, max(A.shape[1], 1), B, max(B.shape[1], 1),
               beta, out, max(N, 1))
    if rc != 0:
        raise ValueError(f"oracle_sgemm returned {rc}")
    return out
