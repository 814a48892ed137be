"""CPU oracle for the k-means assignment step (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It is a plain fp64 implementation of
the definition (see ``kmeans_oracle.c`` for the passages it follows and the
readings it adopts) and shares no code with the HIP path.

Inputs are bf16 bit patterns as ``uint16`` arrays, row-major ``[rows][D]``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "kmeans_oracle.c")
LIBRARY = os.path.join(_HERE, "libkmeans_oracle.so")

_lib = None


# gcc flags of the oracle build: generic x86-64 code (the library is built
# on one machine and may run on another host CPU), OpenMP over points.
BUILD_FLAGS = ("-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11")


def build(source: str = SOURCE, output: str = LIBRARY, extra_flags=()) -> str:
    """Compile the oracle with gcc (BUILD_FLAGS)."""
    cmd = ["gcc", *BUILD_FLAGS, *extra_flags, source, "-o", output + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


def load(path: str = LIBRARY):
    """Load (and return) the oracle library at ``path``."""
    lib = ctypes.CDLL(path)
    u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
    i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
    f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
    i64 = ctypes.c_int64
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_centroid_norms.argtypes = [u16p, i64, i64, f64p]
    lib.oracle_assign.argtypes = [u16p, u16p, i64, i64, i64, i32p,
                                  f64p, f64p, f64p]
    lib.oracle_score_for.argtypes = [u16p, u16p, i64, i64, i32p, f64p]
    lib.oracle_sqdist_for.argtypes = [u16p, u16p, i64, i64, i32p, f64p]
    i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
    lib.oracle_update.argtypes = [u16p, i32p, u16p, i64, i64, i64, i64p, f64p, u16p]
    lib.oracle_bf16_from_double_array.argtypes = [f64p, i64, u16p]
    for f in ("oracle_centroid_norms", "oracle_assign", "oracle_score_for",
              "oracle_sqdist_for", "oracle_update",
              "oracle_bf16_from_double_array"):
        getattr(lib, f).restype = None
    return lib


def _get():
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY) or (
                os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE)):
            build()
        _lib = load()
    return _lib


def _bits(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16 or a.ndim != 2:
        raise TypeError("expected a 2-D uint16 array of bf16 bit patterns")
    return a


def num_threads(lib=None) -> int:
    return (lib or _get()).oracle_num_threads()


def centroid_norms(C, lib=None) -> np.ndarray:
    """fp64 ``n_k = sum_j c_kj^2``."""
    C = _bits(C)
    out = np.empty(C.shape[0], dtype=np.float64)
    (lib or _get()).oracle_centroid_norms(C, C.shape[0], C.shape[1], out)
    return out


def assign(X, C, lib=None) -> dict:
    """Full fp64 assignment: labels, best score, runner-up score, distance."""
    X, C = _bits(X), _bits(C)
    N, D = X.shape
    K = C.shape[0]
    if C.shape[1] != D:
        raise ValueError("X and C disagree on D")
    labels = np.zeros(N, dtype=np.int32)
    best = np.full(N, np.nan)
    second = np.full(N, np.nan)
    dist = np.full(N, np.nan)
    (lib or _get()).oracle_assign(X, C, N, D, K, labels, best, second, dist)
    return dict(labels=labels, best=best, second=second, dist=dist)


def score_for(X, C, labels, lib=None) -> np.ndarray:
    """fp64 ``s_i,labels[i]``."""
    X, C = _bits(X), _bits(C)
    labels = np.ascontiguousarray(labels, dtype=np.int32)
    out = np.empty(X.shape[0], dtype=np.float64)
    (lib or _get()).oracle_score_for(X, C, X.shape[0], X.shape[1], labels, out)
    return out


def sqdist_for(X, C, labels, lib=None) -> np.ndarray:
    """fp64 ``sum_j (x_ij - c_labels[i],j)^2``."""
    X, C = _bits(X), _bits(C)
    labels = np.ascontiguousarray(labels, dtype=np.int32)
    out = np.empty(X.shape[0], dtype=np.float64)
    (lib or _get()).oracle_sqdist_for(X, C, X.shape[0], X.shape[1], labels, out)
    return out


def bf16_from_double(a, lib=None) -> np.ndarray:
    """fp64 values -> bf16 bit patterns (nearest, ties to even)."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    (lib or _get()).oracle_bf16_from_double_array(a.ravel(), a.size, out.ravel())
    return out


def update(X, labels, C_old, lib=None) -> dict:
    """Centroid update from ``labels``: per-cluster counts (int64), fp64
    means ``[K][D]`` and the new bf16 centroids ``[K][D]`` (an empty
    cluster keeps its old row; labels outside ``[0, K)`` are ignored)."""
    X, C_old = _bits(X), _bits(C_old)
    N, D = X.shape
    K = C_old.shape[0]
    if C_old.shape[1] != D:
        raise ValueError("X and C disagree on D")
    labels = np.ascontiguousarray(labels, dtype=np.int32)
    if labels.shape != (N,):
        raise ValueError("labels must have one entry per point")
    counts = np.zeros(K, dtype=np.int64)
    means = np.zeros((K, D), dtype=np.float64)
    C_new = np.zeros((K, D), dtype=np.uint16)
    (lib or _get()).oracle_update(X, labels, C_old, N, D, K, counts, means, C_new)
    return dict(counts=counts, means=means, C_new=C_new)
