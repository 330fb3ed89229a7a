"""FP32 SGEMM for AMD Instinct MI355X (gfx950) -- Python binding.

The work is done by the HIP library ``libmisgemm.so`` built from
the HIP sources under ``csrc/`` (see ``include/misgemm.h`` for the C ABI). This module only
marshals arguments into it with ctypes; it never computes a result itself and
has no fallback: if the library is missing, every call raises.

Functions with the C names take raw device pointers (ints) and a HIP stream
handle and return the C status code. ``sgemm`` is the torch-tensor form: it
derives sizes and leading dimensions from the tensors, enqueues on the current
torch stream, and raises ``MisgemmError`` on a non-zero status.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "MisgemmError", "library_path", "load_library",
    "mi_sgemm", "mi_sgemm_noalloc", "mi_sgemm_with_config", "mi_sgemm_select_config",
    "mi_sgemm_config_count", "mi_sgemm_config_name", "mi_sgemm_status_string",
    "mi_sgemm_release_workspace", "mi_clock_probe", "sgemm", "config_names",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libmisgemm.so")
_lib = None


class MisgemmError(RuntimeError):
    def __init__(self, status: int, where: str = "mi_sgemm"):
        self.status = status
        super().__init__(f"{where} failed with status {status}: {mi_sgemm_status_string(status)}")


def load_library():
    """Load libmisgemm.so (built by fp32_gemm_nn_amd/build.py); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(
            f"HIP library not built: {library_path} is missing. "
            "Run `python -m fp32_gemm_nn_amd.build` (or __graft_entry__.build()).")
    # torch ships its own HIP runtime (libamdhip64.so.7 under torch/lib). Load
    # it first, so that this library's libamdhip64.so.7 resolves to the same
    # copy: loaded the other way round, the process ends up with two HIP and
    # two HSA runtimes, and the one this library uses finds no device.
    import torch  # noqa: F401
    lib = ctypes.CDLL(library_path)
    c, i, f, p = ctypes.c_char, ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    gemm_args = [c, c, i, i, i, f, p, i, p, i, f, p, i, p]
    lib.mi_sgemm.argtypes = gemm_args
    lib.mi_sgemm.restype = i
    lib.mi_sgemm_noalloc.argtypes = gemm_args
    lib.mi_sgemm_noalloc.restype = i
    lib.mi_sgemm_with_config.argtypes = [i, *gemm_args]
    lib.mi_sgemm_with_config.restype = i
    lib.mi_sgemm_select_config.argtypes = [c, c, i, i, i]
    lib.mi_sgemm_select_config.restype = i
    lib.mi_sgemm_config_count.argtypes = []
    lib.mi_sgemm_config_count.restype = i
    lib.mi_sgemm_config_name.argtypes = [i]
    lib.mi_sgemm_config_name.restype = ctypes.c_char_p
    lib.mi_sgemm_status_string.argtypes = [i]
    lib.mi_sgemm_status_string.restype = ctypes.c_char_p
    lib.mi_sgemm_release_workspace.argtypes = [p]
    lib.mi_sgemm_release_workspace.restype = i
    lib.mi_clock_probe.argtypes = [i, p, ctypes.POINTER(i), p]
    lib.mi_clock_probe.restype = i
    _lib = lib
    return lib


def _ch(t) -> bytes:
    if isinstance(t, bytes):
        return t
    s = str(t)
    if len(s) != 1:
        return b"?"
    return s.encode()


def mi_sgemm(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    """C ABI mi_sgemm with integer device pointers; returns the status code."""
    return load_library().mi_sgemm(_ch(transA), _ch(transB), int(M), int(N), int(K), float(alpha),
                                   A or None, int(lda), B or None, int(ldb), float(beta), C or None,
                                   int(ldc), stream or None)


def mi_sgemm_noalloc(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    """C ABI mi_sgemm_noalloc (no device allocation; the device's static scratch)."""
    return load_library().mi_sgemm_noalloc(_ch(transA), _ch(transB), int(M), int(N), int(K), float(alpha),
                                           A or None, int(lda), B or None, int(ldb), float(beta), C or None,
                                           int(ldc), stream or None)


def mi_sgemm_with_config(config, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                         stream=0) -> int:
    return load_library().mi_sgemm_with_config(
        int(config), _ch(transA), _ch(transB), int(M), int(N), int(K), float(alpha), A or None,
        int(lda), B or None, int(ldb), float(beta), C or None, int(ldc), stream or None)


def mi_sgemm_select_config(transA, transB, M, N, K) -> int:
    return load_library().mi_sgemm_select_config(_ch(transA), _ch(transB), int(M), int(N), int(K))


def mi_sgemm_config_count() -> int:
    return load_library().mi_sgemm_config_count()


def mi_sgemm_config_name(config) -> str | None:
    r = load_library().mi_sgemm_config_name(int(config))
    return None if r is None else r.decode()


def mi_sgemm_status_string(status) -> str:
    return load_library().mi_sgemm_status_string(int(status)).decode()


def mi_sgemm_release_workspace(stream=0) -> int:
    """C ABI mi_sgemm_release_workspace (integer stream handle); returns the status code."""
    return load_library().mi_sgemm_release_workspace(stream or None)


def mi_clock_probe(iters, stamps, stream=0):
    """C ABI mi_clock_probe (measurement aid): enqueue the probe writing to the
    device buffer `stamps` (int address); returns (status, wall_clock_khz)."""
    khz = ctypes.c_int(0)
    rc = load_library().mi_clock_probe(int(iters), stamps or None, ctypes.byref(khz), stream or None)
    return rc, khz.value


def config_names() -> list[str]:
    return [mi_sgemm_config_name(i) for i in range(mi_sgemm_config_count())]


def _ld(t) -> int:
    """Leading dimension of a 2-D tensor whose rows are contiguous (stride(1) == 1).

    With more than one row it is the row stride, which must be at least the
    row length: a smaller one (rows that overlap, or stride 0 from expand())
    cannot be described by a leading dimension, and passing the row length
    instead would make the kernels address elements the tensor does not hold.
    Such tensors raise ValueError before anything is launched. A single row
    has no row stride to honour, so its row length (at least 1) is passed.
    """
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    rows, cols = int(t.shape[0]), int(t.shape[1])
    if cols > 1 and t.stride(1) != 1:
        raise ValueError("rows must be contiguous (stride(1) == 1); pass op 'T' for transposes")
    if rows <= 1:
        return max(cols, 1)
    ld = int(t.stride(0))
    if ld < max(cols, 1):
        raise ValueError(f"row stride {ld} is smaller than the row length {cols} (overlapping or broadcast "
                         "rows have no leading dimension); pass a tensor with distinct rows, e.g. .contiguous()")
    return ld


def _overlaps(x, y) -> bool:
    """Whether two 2-D tensors with contiguous rows share any element's memory
    (C must not overlap A or B). Row i of x covers bytes [x0 + i*sx, x0 + i*sx + wx);
    for each row of x the rows of y that could intersect it form one index
    range, so the test is exact (padding between rows is not counted) and
    linear in the rows of x. The row strides are the leading dimensions of
    _ld, so a tensor with overlapping or broadcast rows raises ValueError."""
    import numpy as np

    if x.numel() == 0 or y.numel() == 0:
        return False
    es = x.element_size()

    def rows(t):
        return t.data_ptr(), _ld(t) * es, t.shape[1] * es, t.shape[0]

    x0, sx, wx, rx = rows(x)
    y0, sy, wy, ry = rows(y)
    if x0 + (rx - 1) * sx + wx <= y0 or y0 + (ry - 1) * sy + wy <= x0:
        return False
    start = x0 + sx * np.arange(rx, dtype=np.int64)
    # Rows j of y with y0 + j*sy < start + wx and y0 + j*sy + wy > start.
    j_hi = np.minimum((start + wx - y0 - 1) // sy, ry - 1)
    j_lo = np.maximum((start - y0 - wy) // sy + 1, 0)
    return bool(np.any(j_lo <= j_hi))


def sgemm(transA: str, transB: str, alpha: float, A, B, beta: float, C, stream=None, config=None):
    """C <- alpha*op(A)@op(B) + beta*C on float32 device tensors (row-major views).

    A is the stored matrix (M x K for 'N', K x M for 'T'); likewise B. C is
    M x N. Each tensor must have contiguous rows; its row stride is passed as
    the leading dimension. Work is enqueued on ``stream`` (default: the current
    torch stream of C's device); returns C.
    """
    import torch

    for name, t in (("A", A), ("B", B), ("C", C)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor")
    if not (A.device == B.device == C.device):
        raise ValueError(f"A, B and C must be on one device (got {A.device}, {B.device}, {C.device})")
    lda, ldb, ldc = _ld(A), _ld(B), _ld(C)
    if _overlaps(C, A) or _overlaps(C, B):
        raise ValueError("C must not overlap A or B")
    ta = transA in ("T", "t", "C", "c")
    tb = transB in ("T", "t", "C", "c")
    M, N = int(C.shape[0]), int(C.shape[1])
    K = int(A.shape[0] if ta else A.shape[1])
    am = int(A.shape[1] if ta else A.shape[0])
    bk = int(B.shape[1] if tb else B.shape[0])
    bn = int(B.shape[0] if tb else B.shape[1])
    if am != M or bk != K or bn != N:
        raise ValueError(f"shape mismatch: op(A) {am}x{K}, op(B) {bk}x{bn}, C {M}x{N}")
    if stream is None:
        stream = torch.cuda.current_stream(C.device).cuda_stream
    args = (transA, transB, M, N, K, alpha, A.data_ptr(), lda, B.data_ptr(), ldb, beta,
            C.data_ptr(), ldc, stream)
    rc = mi_sgemm(*args) if config is None else mi_sgemm_with_config(config, *args)
    if rc != 0:
        raise MisgemmError(rc)
    return C
