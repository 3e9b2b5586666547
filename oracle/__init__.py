"""CPU oracle for batched potrf / posv -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, loads or calls it, and this package never
imports the product path.

The arithmetic lives in ``potrf_oracle.c`` (plain C, no FMA contraction, no
fast-math); this wrapper only marshals numpy buffers through ctypes and builds
the shared object with gcc when it is missing.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "potrf_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

_DT = {np.dtype(np.float32): 0, np.dtype(np.float64): 1,
       np.dtype(np.complex64): 2, np.dtype(np.complex128): 3}
_UPLO = {"L": 0, "U": 1}

_lib = None

COMPILE_FLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                 "-shared", "-pthread", "-Wall"]


def compile_source(src: str, out: str) -> str:
    """Compile an oracle C source into a shared object (used by build())."""
    tmp = out + f".tmp{os.getpid()}"
    subprocess.run(["gcc", *COMPILE_FLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile potrf_oracle.c into liboracle.so with gcc."""
    if force or not os.path.exists(_LIB_PATH):
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


def open_library(path: str):
    """ctypes handle of an oracle shared object with its signatures set."""
    lib = ctypes.CDLL(path)
    i64, vp, i32p = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
    lib.oracle_potrf.argtypes = [ctypes.c_int, ctypes.c_int, i64, vp, i64, i64, i64,
                                 i32p, ctypes.c_int]
    lib.oracle_potrf.restype = ctypes.c_int
    lib.oracle_posv.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, vp, i64, i64,
                                vp, i64, i64, i64, i32p, ctypes.c_int]
    lib.oracle_posv.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = open_library(_LIB_PATH)
    return _lib


def _uplo(u: str) -> int:
    return _UPLO[u.upper()[0]]


def default_threads() -> int:
    return max(1, os.cpu_count() or 1)


def potrf(buf: np.ndarray, uplo: str, n: int, batch: int, lda: int | None = None,
          stride: int | None = None, nthreads: int | None = None, lib=None) -> np.ndarray:
    """Factor a column-major batch buffer in place; returns info (int32[batch])."""
    lda = n if lda is None else lda
    stride = lda * n if stride is None else stride
    if not buf.flags.c_contiguous or buf.size < batch * stride:
        raise ValueError("buffer must be contiguous and hold batch * stride elements")
    info = np.zeros(batch, dtype=np.int32)
    rc = (lib or _load()).oracle_potrf(_DT[buf.dtype], _uplo(uplo), n, buf.ctypes.data, lda, stride,
                              batch, info.ctypes.data, nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_potrf rejected its arguments (rc={rc})")
    return info


def posv(abuf: np.ndarray, bbuf: np.ndarray, uplo: str, n: int, nrhs: int, batch: int,
         lda: int | None = None, strideA: int | None = None, ldb: int | None = None,
         strideB: int | None = None, nthreads: int | None = None, lib=None) -> np.ndarray:
    """Factor A and solve A X = B in place (column-major buffers); returns info."""
    lda = n if lda is None else lda
    strideA = lda * n if strideA is None else strideA
    ldb = n if ldb is None else ldb
    strideB = ldb * nrhs if strideB is None else strideB
    if abuf.dtype != bbuf.dtype:
        raise ValueError("A and B must share a dtype")
    for b_, s_ in ((abuf, strideA), (bbuf, strideB)):
        if not b_.flags.c_contiguous or b_.size < batch * s_:
            raise ValueError("buffers must be contiguous and large enough")
    info = np.zeros(batch, dtype=np.int32)
    rc = (lib or _load()).oracle_posv(_DT[abuf.dtype], _uplo(uplo), n, nrhs, abuf.ctypes.data, lda,
                             strideA, bbuf.ctypes.data, ldb, strideB, batch, info.ctypes.data,
                             nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_posv rejected its arguments (rc={rc})")
    return info


def potrf_matrices(a: np.ndarray, uplo: str = "L", nthreads: int | None = None, lib=None):
    """Convenience: factor (batch, n, n) math-orientation matrices.

    Returns (factor, info) where factor is (batch, n, n) holding the whole
    buffer after the call (the unreferenced triangle is passed through).
    """
    from synthetic import to_colmajor, from_colmajor
    batch, n, _ = a.shape
    buf = to_colmajor(a)
    info = potrf(buf, uplo, n, batch, nthreads=nthreads, lib=lib)
    return from_colmajor(buf, n, n, batch), info


def posv_matrices(a: np.ndarray, b: np.ndarray, uplo: str = "L",
                  nthreads: int | None = None, lib=None):
    """Convenience: (batch, n, n) and (batch, n, nrhs) -> (factor, X, info)."""
    from synthetic import to_colmajor, from_colmajor
    batch, n, _ = a.shape
    nrhs = b.shape[2]
    abuf = to_colmajor(a)
    bbuf = to_colmajor(b)
    info = posv(abuf, bbuf, uplo, n, nrhs, batch, nthreads=nthreads, lib=lib)
    return from_colmajor(abuf, n, n, batch), from_colmajor(bbuf, n, nrhs, batch), info
