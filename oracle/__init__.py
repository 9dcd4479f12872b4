"""CPU oracle for the dense fp16 NT GEMM C = A @ B.T.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  The HIP
library never imports, links or calls it, and it shares no code with it.

The arithmetic lives in ``gemm_oracle.c`` (plain C, fp64, hand-written fp16
conversions); this module only builds that file with gcc and marshals numpy
arrays through ctypes.  The definition it follows (Tilus "Hopper matmul"
pages, "2. Multi-Stage Software Pipelining" / The Full Kernel, and
"6. Register Reallocation, Multicast, and a Persistent Kernel" / opening
paragraphs) is

    C[i, j] = fp16_rne( sum_k double(A[i, k]) * double(B[j, k]) )

one fp64 accumulator per element, k ascending, then one round-to-nearest-even.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_gemm.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile gemm_oracle.c into liboracle_gemm.so (gcc, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            i64, p = ctypes.c_int64, ctypes.c_void_p
            lib.oracle_gemm_f16_nt.argtypes = [i64, i64, i64, p, p, p, p, p, p, ctypes.c_int]
            lib.oracle_gemm_f16_nt.restype = None
            lib.oracle_gemm_f16_nt_sampled.argtypes = [i64, i64, i64, p, p, p, p, i64, p, p,
                                                       ctypes.c_int]
            lib.oracle_gemm_f16_nt_sampled.restype = None
            lib.oracle_f16_to_f64_array.argtypes = [p, p, i64]
            lib.oracle_f16_to_f64_array.restype = None
            lib.oracle_f64_to_f16_array.argtypes = [p, p, i64]
            lib.oracle_f64_to_f16_array.restype = None
            _lib = lib
    return _lib


def default_threads() -> int:
    """Host threads available to this process (its CPU affinity set)."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _as_f16(x: np.ndarray, name: str) -> np.ndarray:
    if x.dtype != np.float16:
        raise TypeError(f"{name} must be float16, got {x.dtype}")
    return np.ascontiguousarray(x)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def gemm(a: np.ndarray, b: np.ndarray, threads: int | None = None,
         return_sum: bool = False):
    """C = fp16_rne(A @ B.T) for fp16 A [M, K] and B [N, K].

    Returns the fp16 matrix C [M, N]; with ``return_sum`` also the unrounded
    fp64 sums [M, N].
    """
    a = _as_f16(a, "A")
    b = _as_f16(b, "B")
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"shape mismatch: A{a.shape} B{b.shape}")
    m, k = a.shape
    n = b.shape[0]
    lib = _load()
    c = np.empty((m, n), dtype=np.float16)
    s = np.empty((m, n), dtype=np.float64) if return_sum else None
    if m > 0 and n > 0:
        a_dbl = np.empty(max(1, m * k), dtype=np.float64)
        b_dbl = np.empty(max(1, n * k), dtype=np.float64)
        lib.oracle_gemm_f16_nt(m, n, k, _ptr(a), _ptr(b), _ptr(c),
                               _ptr(s) if s is not None else None,
                               _ptr(a_dbl), _ptr(b_dbl),
                               int(threads or default_threads()))
    return (c, s) if return_sum else c


def gemm_sampled(a: np.ndarray, b: np.ndarray, rows, cols,
                 threads: int | None = None, return_sum: bool = False):
    """The oracle evaluated only at positions (rows[t], cols[t])."""
    a = _as_f16(a, "A")
    b = _as_f16(b, "B")
    m, k = a.shape
    n = b.shape[0]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be 1-D and of equal length")
    if rows.size and (rows.min() < 0 or rows.max() >= m or cols.min() < 0 or cols.max() >= n):
        raise IndexError("sample position out of range")
    lib = _load()
    out = np.empty(rows.size, dtype=np.float16)
    s = np.empty(rows.size, dtype=np.float64) if return_sum else None
    lib.oracle_gemm_f16_nt_sampled(m, n, k, _ptr(a), _ptr(b), _ptr(rows), _ptr(cols),
                                   rows.size, _ptr(out),
                                   _ptr(s) if s is not None else None,
                                   int(threads or default_threads()))
    return (out, s) if return_sum else out


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """The oracle's fp16 -> fp64 decoding, applied elementwise to uint16 bits."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().oracle_f16_to_f64_array(_ptr(bits), _ptr(out), bits.size)
    return out


def f64_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """The oracle's fp64 -> fp16 round-to-nearest-even, as uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_f64_to_f16_array(_ptr(x), _ptr(out), x.size)
    return out
