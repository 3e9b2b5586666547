"""Comparison helpers shared by the oracle pins and the GPU parity tests.

Everything is evaluated in float64 / complex128, per matrix, and reported as the
maximum over items (a batch aggregate would hide one bad item).
"""
from __future__ import annotations

import numpy as np

from synthetic import np_dtype, real_dtype, referenced_mask

# Tolerances on the relative Frobenius error against the oracle, per element type.
TOL = {"f32": 1e-4, "c64": 1e-4, "f64": 1e-11, "c128": 1e-11}
RESIDUAL_BOUND = 10.0


def eps_of(dt) -> float:
    return float(np.finfo(real_dtype(dt)).eps)


def lower_factor(f: np.ndarray, uplo: str) -> np.ndarray:
    """L (batch, n, n) in complex128/float64 from a potrf result buffer."""
    f = f.astype(np.complex128 if np.iscomplexobj(f) else np.float64)
    if uplo.upper().startswith("L"):
        return np.tril(f)
    u = np.triu(f)
    return np.conj(np.swapaxes(u, 1, 2))


def factor_residual(a: np.ndarray, f: np.ndarray, uplo: str, items=None) -> np.ndarray:
    """Per-item ||A - L L^H||_F / (||A||_F n eps)."""
    n = a.shape[1]
    eps = eps_of(a.dtype)
    idx = np.arange(a.shape[0]) if items is None else np.asarray(items)
    if idx.size == 0:
        return np.zeros(0)
    aa = a[idx].astype(np.complex128 if np.iscomplexobj(a) else np.float64)
    ll = lower_factor(f[idx], uplo)
    r = aa - np.matmul(ll, np.conj(np.swapaxes(ll, 1, 2)))
    num = np.linalg.norm(r, axis=(1, 2))
    den = np.linalg.norm(aa, axis=(1, 2)) * n * eps
    return num / den


def solve_residual(a: np.ndarray, x: np.ndarray, b: np.ndarray, items=None) -> np.ndarray:
    """Per-item ||B - A X||_F / (||A||_F ||X||_F n eps)."""
    n = a.shape[1]
    eps = eps_of(a.dtype)
    idx = np.arange(a.shape[0]) if items is None else np.asarray(items)
    if idx.size == 0:
        return np.zeros(0)
    wide = np.complex128 if np.iscomplexobj(a) else np.float64
    aa, xx, bb = a[idx].astype(wide), x[idx].astype(wide), b[idx].astype(wide)
    r = bb - np.matmul(aa, xx)
    num = np.linalg.norm(r, axis=(1, 2))
    den = np.linalg.norm(aa, axis=(1, 2)) * np.linalg.norm(xx, axis=(1, 2)) * n * eps
    return num / den


def rel_err_triangle(got: np.ndarray, ref: np.ndarray, uplo: str, items=None) -> np.ndarray:
    """Per-item relative Frobenius error over the referenced triangle."""
    n = ref.shape[1]
    m = referenced_mask(n, uplo)
    idx = np.arange(ref.shape[0]) if items is None else np.asarray(items)
    if idx.size == 0:
        return np.zeros(0)
    wide = np.complex128 if np.iscomplexobj(ref) else np.float64
    g = got[idx][:, m].astype(wide)
    r = ref[idx][:, m].astype(wide)
    return np.linalg.norm(g - r, axis=1) / np.linalg.norm(r, axis=1)


def rel_err(got: np.ndarray, ref: np.ndarray, items=None) -> np.ndarray:
    """Per-item relative Frobenius error over whole (batch, rows, cols) arrays."""
    idx = np.arange(ref.shape[0]) if items is None else np.asarray(items)
    if idx.size == 0:
        return np.zeros(0)
    wide = np.complex128 if np.iscomplexobj(ref) else np.float64
    g = got[idx].reshape(len(idx), -1).astype(wide)
    r = ref[idx].reshape(len(idx), -1).astype(wide)
    return np.linalg.norm(g - r, axis=1) / np.linalg.norm(r, axis=1)


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    """Bitwise equality (NaN payloads included)."""
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    return a.shape == b.shape and a.dtype == b.dtype and \
        np.array_equal(a.view(np.uint8), b.view(np.uint8))


def dtype_key(dt) -> str:
    d = np_dtype(dt)
    return {np.float32: "f32", np.float64: "f64", np.complex64: "c64",
            np.complex128: "c128"}[d.type]
