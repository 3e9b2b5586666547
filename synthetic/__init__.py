"""Seeded synthetic inputs for batched potrf / posv.

This module is shared by the tests, the benchmark and the smoke check: it is the
only code both the CPU oracle's callers and the HIP path's callers use.  It holds
no part of the factorisation or solve arithmetic -- only random draws, the
positive-definite generator, and column-major layout helpers.

Generator (the same recipe for every workload):
  1. G is drawn in float64 from ``numpy.random.default_rng(seed)``, chunk by
     chunk of 64 matrices: real G ~ N(0, 1); complex G = X + iY with X, Y drawn
     in that order, each ~ N(0, 1/2).
  2. A = G G^H / n + I in float64.  Its eigenvalues are >= 1, so every Schur
     pivot of A is >= 1 (interlacing), and A is well conditioned.
  3. The strictly lower triangle is mirrored to the upper one exactly
     (A(c, i) = conj(A(i, c))) and the imaginary part of the diagonal is 0.
  4. A is rounded to the element type.
Planted failures: items b with b % every == 0 get A(k, k) <- -A(k, k) for
k ~ U{0..n-1} drawn from ``default_rng([seed, 1])``; the leading k x k block is
unchanged and the k-th Schur pivot becomes <= -1, so info = k + 1 exactly.
Right-hand sides: B ~ N(0, 1) (complex: (X + iY) / sqrt(2)) from
``default_rng([seed, 2])``.

Layout: a batch buffer is a flat array of ``batch * stride`` elements; matrix b's
element (i, c) lives at ``b * stride + c * ld + i`` (column-major, counts in
elements).  Math-orientation arrays have shape (batch, rows, cols).
"""
from __future__ import annotations

import numpy as np

DTYPES = {
    "f32": np.dtype(np.float32),
    "f64": np.dtype(np.float64),
    "c64": np.dtype(np.complex64),
    "c128": np.dtype(np.complex128),
}

SENTINEL_REAL = -999.0
SENTINEL_IMAG = 777.0


def np_dtype(dt) -> np.dtype:
    """Map 'f32' / 'f64' / 'c64' / 'c128' (or a numpy dtype) to a numpy dtype."""
    if isinstance(dt, str):
        return DTYPES[dt]
    return np.dtype(dt)


def dtype_name(dt) -> str:
    d = np_dtype(dt)
    for k, v in DTYPES.items():
        if v == d:
            return k
    raise ValueError(f"unsupported dtype {dt}")


def is_complex(dt) -> bool:
    return np_dtype(dt).kind == "c"


def real_dtype(dt) -> np.dtype:
    d = np_dtype(dt)
    return np.dtype(np.float32) if d in (np.float32, np.complex64) else np.dtype(np.float64)


def _draw_g(rng, count, n, cplx):
    if cplx:
        x = rng.standard_normal((count, n, n))
        y = rng.standard_normal((count, n, n))
        return (x + 1j * y) * np.sqrt(0.5)
    return rng.standard_normal((count, n, n))


def spd_matrices(n: int, batch: int, dtype, seed: int, chunk: int = 64) -> np.ndarray:
    """Hermitian positive-definite matrices, shape (batch, n, n), math orientation."""
    d = np_dtype(dtype)
    cplx = d.kind == "c"
    rng = np.random.default_rng(seed)
    out = np.empty((batch, n, n), dtype=d)
    eye = np.eye(n)
    low = np.tril(np.ones((n, n), dtype=bool), -1)
    for b0 in range(0, batch, chunk):
        cnt = min(chunk, batch - b0)
        g = _draw_g(rng, cnt, n, cplx)
        gh = np.conj(np.swapaxes(g, 1, 2)) if cplx else np.swapaxes(g, 1, 2)
        a = np.matmul(g, gh) / n + eye
        # mirror the strictly lower triangle to the upper one, exactly
        at = np.swapaxes(a, 1, 2)
        a = np.where(low[None], a, np.conj(at) if cplx else at)
        if cplx:
            idx = np.arange(n)
            a[:, idx, idx] = a[:, idx, idx].real
        out[b0:b0 + cnt] = a.astype(d)
    return out


def plant_failures(a: np.ndarray, seed: int, every: int = 64) -> np.ndarray:
    """Negate one diagonal entry of items b % every == 0 (in place).

    Returns the expected info array (int32): k + 1 for planted items, else 0.
    """
    batch, n, _ = a.shape
    rng = np.random.default_rng([seed, 1])
    info = np.zeros(batch, dtype=np.int32)
    for b in range(0, batch, every):
        k = int(rng.integers(0, n))
        a[b, k, k] = -a[b, k, k]
        info[b] = k + 1
    return info


def rhs(n: int, nrhs: int, batch: int, dtype, seed: int) -> np.ndarray:
    """Right-hand sides, shape (batch, n, nrhs)."""
    d = np_dtype(dtype)
    rng = np.random.default_rng([seed, 2])
    if d.kind == "c":
        x = rng.standard_normal((batch, n, nrhs))
        y = rng.standard_normal((batch, n, nrhs))
        return ((x + 1j * y) * np.sqrt(0.5)).astype(d)
    return rng.standard_normal((batch, n, nrhs)).astype(d)


def sentinel(dtype):
    d = np_dtype(dtype)
    if d.kind == "c":
        return d.type(complex(SENTINEL_REAL, SENTINEL_IMAG))
    return d.type(SENTINEL_REAL)


def nan_value(dtype):
    d = np_dtype(dtype)
    if d.kind == "c":
        return d.type(complex(np.nan, np.nan))
    return d.type(np.nan)


def to_colmajor(m: np.ndarray, ld: int | None = None, stride: int | None = None,
                fill=0) -> np.ndarray:
    """Flatten (batch, rows, cols) into a column-major batch buffer.

    Padding (rows ld..., and the tail of each stride) is set to ``fill``.
    """
    batch, rows, cols = m.shape
    ld = rows if ld is None else ld
    stride = ld * cols if stride is None else stride
    if ld < rows or stride < ld * cols:
        raise ValueError("ld / stride too small")
    buf = np.full(batch * stride, fill, dtype=m.dtype)
    view = buf.reshape(batch, stride)[:, : ld * cols].reshape(batch, cols, ld)
    view[:, :, :rows] = np.swapaxes(m, 1, 2)
    return buf


def from_colmajor(buf: np.ndarray, rows: int, cols: int, batch: int,
                  ld: int | None = None, stride: int | None = None) -> np.ndarray:
    """Inverse of ``to_colmajor``: returns (batch, rows, cols)."""
    ld = rows if ld is None else ld
    stride = ld * cols if stride is None else stride
    view = np.asarray(buf).reshape(batch, stride)[:, : ld * cols].reshape(batch, cols, ld)
    return np.ascontiguousarray(np.swapaxes(view[:, :, :rows], 1, 2))


def referenced_mask(n: int, uplo: str) -> np.ndarray:
    """Boolean (n, n) mask of the triangle potrf reads and writes."""
    low = np.tril(np.ones((n, n), dtype=bool))
    return low if uplo.upper().startswith("L") else low.T


def poison(m: np.ndarray, uplo: str, value) -> np.ndarray:
    """Copy of (batch, n, n) with the unreferenced triangle set to ``value``."""
    n = m.shape[1]
    out = m.copy()
    out[:, ~referenced_mask(n, uplo)] = value
    return out


def layout(n: int, ncols: int | None = None, padded: bool = False):
    """(ld, stride) for the natural layout, or the padded one ld = n + 7,
    stride = ld * ncols + 13."""
    ncols = n if ncols is None else ncols
    if padded:
        ld = n + 7
        return ld, ld * ncols + 13
    return n, n * ncols
