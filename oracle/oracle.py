"""CPU oracle for single-precision GEMM -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this module.  The product path (the HIP library and its Python
binding) never imports, links or calls anything under ``oracle/``, and this
module imports nothing from the product package.

The arithmetic lives in ``oracle_sgemm.c`` (plain C, fp64 accumulation, one
rounding to fp32); this file only builds it with gcc and marshals numpy arrays.
The problem it states is the one all four pages share:
``C = alpha * A @ B + beta * C`` on row-major fp32 matrices ("Warp Tiling: A
Third Level of Tiling", section "The Kernel"; "Shared Memory Tiling", kernel
listing).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle_sgemm.c")
LIB = os.path.join(HERE, "liboracle_sgemm.so")

# -ffp-contract=off: no fused multiply-add anywhere, so the epilogue's fp64
# rounding is the one the C source spells out.  No -ffast-math.
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-std=c99", "-shared", "-fPIC"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle_sgemm.so``."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", *CFLAGS, SRC, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(LIB)
        i64, f32, vp = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
        lib.oracle_sgemm.argtypes = [i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64, vp, i64]
        lib.oracle_sgemm.restype = ctypes.c_int
        lib.oracle_sgemm_entries.argtypes = [i64, vp, vp, i64, i64, i64, f32, vp, i64, vp, i64,
                                             f32, vp, i64, vp, vp]
        lib.oracle_sgemm_entries.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _as_f32(a, name):
    if a is None:
        return None
    if a.dtype != np.float32 or not a.flags.c_contiguous:
        raise TypeError(f"{name} must be a C-contiguous float32 array")
    return a


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def sgemm_raw(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, want64=False):
    """Call the C oracle on flat float32 buffers.  C is updated in place.

    Returns ``(status, C64)`` where C64 (M x N, fp64, before the final
    rounding) is returned when ``want64`` and the call succeeded.
    """
    lib = _load()
    A = _as_f32(A, "A"); B = _as_f32(B, "B"); C = _as_f32(C, "C")
    C64 = np.empty((max(M, 0), max(N, 1)), dtype=np.float64) if want64 else None
    rc = lib.oracle_sgemm(M, N, K, ctypes.c_float(alpha), _ptr(A), lda, _ptr(B), ldb,
                          ctypes.c_float(beta), _ptr(C), ldc, _ptr(C64), max(N, 1))
    if C64 is not None:
        C64 = C64[:, :N]
    return rc, C64


def sgemm(A: np.ndarray, B: np.ndarray, C: np.ndarray, alpha: float = 1.0, beta: float = 0.0):
    """Oracle on tight row-major 2-D arrays (A: M x K, B: K x N, C: M x N).

    Returns ``(C_out32, C64)`` as new arrays; the inputs are not modified.
    Padded leading dimensions go through :func:`sgemm_raw`.
    """
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or C.shape != (M, N):
        raise ValueError("shape mismatch")
    Af = np.ascontiguousarray(A, dtype=np.float32)
    Bf = np.ascontiguousarray(B, dtype=np.float32)
    Cf = np.array(C, dtype=np.float32, order="C", copy=True)
    rc, C64 = sgemm_raw(M, N, K, alpha, Af, max(K, 1), Bf, max(N, 1), beta, Cf,
                        max(N, 1), want64=True)
    if rc != 0:
        raise RuntimeError(f"oracle_sgemm returned {rc}")
    return Cf, C64


def entries(rows, cols, A, B, Cin, alpha=1.0, beta=0.0):
    """Selected outputs (row[t], col[t]) as the textbook dot product in fp64.

    A (M x K), B (K x N), Cin (M x N) are C-contiguous float32.
    Returns ``(out32, out64)``.
    """
    lib = _load()
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    M, K = A.shape
    N = B.shape[1]
    A = _as_f32(A, "A"); B = _as_f32(B, "B"); Cin = _as_f32(Cin, "Cin")
    out32 = np.empty(rows.shape, dtype=np.float32)
    out64 = np.empty(rows.shape, dtype=np.float64)
    rc = lib.oracle_sgemm_entries(rows.size, _ptr(rows), _ptr(cols), M, N, K,
                                  ctypes.c_float(alpha), _ptr(A), max(K, 1), _ptr(B), max(N, 1),
                                  ctypes.c_float(beta), _ptr(Cin), max(N, 1), _ptr(out32),
                                  _ptr(out64))
    if rc != 0:
        raise RuntimeError(f"oracle_sgemm_entries returned {rc}")
    return out32, out64


def rel_error(C_test, C64, K, maxabs_A, maxabs_B):
    """Parity measure: max |C_test - C64| / (K * max|A| * max|B|).

    The pages verify each result against a vendor library without stating a
    criterion ("Autotuning: Searching the Tile-Shape Space", code listing of the
    sweep); this normalisation is the reading adopted for this project.  When
    the denominator is zero the caller must require exact equality instead, so
    this returns ``None`` then.
    """
    denom = float(K) * float(maxabs_A) * float(maxabs_B)
    if denom == 0.0:
        return None
    diff = np.abs(np.asarray(C_test, dtype=np.float64) - np.asarray(C64, dtype=np.float64))
    return float(diff.max()) / denom if diff.size else 0.0
