"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle's tests.

Holds no arithmetic of the operator itself: it draws random numbers (SplitMix64,
Box-Muller, inverse-CDF Laplace, Fisher-Yates, Householder QR) and rounds them to the
16-bit storage type.  The native part is ``fq_synth.c``, built by ``synth.build``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .configs import WORKLOADS, Workload  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfqsynth.so")

F16 = 1
BF16 = 2
_DT = {"f16": F16, "fp16": F16, "float16": F16, "bf16": BF16, "bfloat16": BF16}
_DIST = {"gauss": 0, "laplace": 1}

_lib = None


def build(verbose: bool = False) -> str:
    """Compile fq_synth.c into libfqsynth.so next to it (gcc, -O2, no fast-math)."""
    import subprocess

    src = os.path.join(_HERE, "fq_synth.c")
    cmd = ["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           src, "-o", LIB_PATH + ".tmp", "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        i64, u64, ci, p = ctypes.c_int64, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p
        L.fqs_fill_x.argtypes = [p, i64, i64, ci, ci, ctypes.c_double, ctypes.c_double, u64, i64, i64, ci]
        L.fqs_fill_x.restype = ci
        L.fqs_orthogonal.argtypes = [p, p, i64, ci, u64, u64]
        L.fqs_orthogonal.restype = ci
        L.fqs_outlier_channels.argtypes = [i64, i64, u64, p]
        L.fqs_outlier_channels.restype = ci
        L.fqs_round.argtypes = [p, p, i64, ci]
        L.fqs_round.restype = ci
        _lib = L
    return _lib


def dtype_code(dt: str) -> int:
    return _DT[dt]


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def gen_x(M: int, N: int, dtype: str, dist: str = "gauss", outlier_frac: float = 0.0,
          outlier_scale: float = 1.0, seed: int = 0, k0: int = 0, k1: int = 1,
          out: np.ndarray | None = None, nthreads: int | None = None) -> np.ndarray:
    """Slices [k0, k1) of x[K, M, N] as raw uint16 bit patterns, shape [k1-k0, M, N]."""
    n = (k1 - k0) * M * N
    if out is None:
        out = np.empty((k1 - k0, M, N), dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags["C_CONTIGUOUS"] and out.size == n
    rc = lib().fqs_fill_x(out.ctypes.data, M, N, _DT[dtype], _DIST[dist], float(outlier_frac),
                          float(outlier_scale), seed, k0, k1, nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"fqs_fill_x failed ({rc})")
    return out


def gen_orthogonal(n: int, dtype: str, seed: int = 0, tensor_id: int = 2, with_f64: bool = False):
    """Haar-random orthogonal [n, n] rounded to dtype (uint16 bits); optionally the f64 matrix."""
    out = np.empty((n, n), dtype=np.uint16)
    q = np.empty((n, n), dtype=np.float64) if with_f64 else None
    rc = lib().fqs_orthogonal(out.ctypes.data, q.ctypes.data if q is not None else None, n,
                              _DT[dtype], seed, tensor_id)
    if rc != 0:
        raise ValueError(f"fqs_orthogonal failed ({rc})")
    return (out, q) if with_f64 else out


def outlier_channels(n: int, count: int, seed: int = 0) -> np.ndarray:
    out = np.empty(count, dtype=np.int64)
    rc = lib().fqs_outlier_channels(n, count, seed, out.ctypes.data)
    if rc != 0:
        raise ValueError(f"fqs_outlier_channels failed ({rc})")
    return out


def round_to(values, dtype: str) -> np.ndarray:
    """Round float64 values to the storage type (RNE through fp32); returns uint16 bits."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    rc = lib().fqs_round(v.ctypes.data, out.ctypes.data, v.size, _DT[dtype])
    if rc != 0:
        raise ValueError("fqs_round failed")
    return out


def make_inputs(w: "Workload", k0: int = 0, k1: int | None = None, nthreads: int | None = None):
    """(x, p1, p2) as uint16 arrays for workload w; p2 is None for a left-only workload."""
    k1 = w.K if k1 is None else k1
    x = gen_x(w.M, w.N, w.dtype, w.dist, w.outlier_frac, w.outlier_scale, w.seed, k0, k1,
              nthreads=nthreads)
    p1 = gen_orthogonal(w.M, w.dtype, w.seed, tensor_id=2)
    p2 = gen_orthogonal(w.N, w.dtype, w.seed, tensor_id=3) if w.two_sided else None
    return x, p1, p2
