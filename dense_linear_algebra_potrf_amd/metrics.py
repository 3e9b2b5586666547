"""Throughput models for batched potrf / posv (host-side bookkeeping only).

Algorithmic flops: n^3/3 per real potrf and 4n^3/3 per complex potrf; posv adds
2 n^2 nrhs (x4 for complex).  The real convention reproduces the 1.26 TFLOP/s
the BatchLAS perf_potrf page prints for float n = 155, batch 4096 at 4049 us
(section 'CTA kernel measured against cuSOLVER').

Algorithmic bytes: every distinct 128-byte line of the batch buffer that holds a
referenced element is read once and written once, plus 4 bytes of info per
matrix (plus the lines of B, read and written, for posv).  With the natural
layout at small n every line holds a referenced element, so this equals the
footprint 2 n^2 s that the perf_small_n_baseline page's 'DRAM roof' uses
(section 'The potrf n = 8 finding').
"""
from __future__ import annotations

import numpy as np

LINE = 128
ELEM_BYTES = {"f32": 4, "f64": 8, "c64": 8, "c128": 16}
COMPLEX = {"f32": False, "f64": False, "c64": True, "c128": True}

# MI355X published peaks
HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"f32": 157.3, "c64": 157.3, "f64": 78.6, "c128": 78.6}


def potrf_flops(n: int, dt: str) -> float:
    return (4.0 if COMPLEX[dt] else 1.0) * n ** 3 / 3.0


def posv_flops(n: int, nrhs: int, dt: str) -> float:
    return potrf_flops(n, dt) + (4.0 if COMPLEX[dt] else 1.0) * 2.0 * n * n * nrhs


def referenced_lines(n: int, ncols: int, ld: int, stride: int, batch: int, es: int,
                     uplo: str | None) -> int:
    """Distinct 128-byte lines touched by the referenced elements of a batch buffer.

    uplo None means every element of the n x ncols block is referenced (B of posv).
    """
    b = np.arange(batch, dtype=np.int64)[:, None]
    c = np.arange(ncols, dtype=np.int64)[None, :]
    if uplo is None:
        r0 = np.zeros_like(c)
        r1 = np.full_like(c, n)
    elif uplo.upper().startswith("L"):
        r0, r1 = c, np.full_like(c, n)          # rows c..n-1 of column c
    else:
        r0, r1 = np.zeros_like(c), c + 1        # rows 0..c of column c
    start = (b * stride + c * ld + r0) * es
    end = (b * stride + c * ld + r1) * es       # exclusive
    first = (start // LINE).ravel()
    last = ((end - 1) // LINE).ravel()
    nlines = int(last.max()) + 2
    diff = np.zeros(nlines, dtype=np.int32)
    np.add.at(diff, first, 1)
    np.add.at(diff, last + 1, -1)
    return int(np.count_nonzero(np.cumsum(diff) > 0))


def potrf_bytes(n: int, batch: int, dt: str, uplo: str = "L", ld: int | None = None,
                stride: int | None = None) -> int:
    """Algorithmic bytes of one potrf call over the whole batch."""
    ld = n if ld is None else ld
    stride = ld * n if stride is None else stride
    lines = referenced_lines(n, n, ld, stride, batch, ELEM_BYTES[dt], uplo)
    return 2 * LINE * lines + 4 * batch


def posv_bytes(n: int, nrhs: int, batch: int, dt: str, uplo: str = "L") -> int:
    es = ELEM_BYTES[dt]
    a_lines = referenced_lines(n, n, n, n * n, batch, es, uplo)
    b_lines = referenced_lines(n, nrhs, n, n * nrhs, batch, es, None)
    return 2 * LINE * (a_lines + b_lines) + 4 * batch


def footprint_bytes(n: int, batch: int, dt: str) -> int:
    """Whole matrices read and written (the pages' DRAM-roof convention)."""
    return 2 * n * n * ELEM_BYTES[dt] * batch
