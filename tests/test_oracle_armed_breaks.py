"""Armed breaks: plant a plausible mistake in a copy of the oracle's C source,
build it, and check that the pins go red.  This shows the pins can fail; the
shipped oracle is never modified (the mutants live in pytest's tmp_path)."""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import synthetic as syn
from tests.test_oracle_pins import exact_product, integer_factor

SRC = os.path.join(os.path.dirname(oracle.__file__), "potrf_oracle.c")

# (name, old text, new text) -- each replacement must hit the source exactly once
BREAKS = [
    ("stale pivot: the original diagonal instead of the Schur value",
     "R d = *s_at_##SUF(A, lda, upper, j, j) - s;",
     "R d = *s_at_##SUF(A, lda, upper, j, j) - 0 * s;"),
    ("complex update uses a transpose instead of a conjugate transpose",
     "t.re -= a.re * b.re + a.im * b.im;",
     "t.re -= a.re * b.re - a.im * b.im;"),
    ("zero and NaN pivots accepted (d < 0 instead of !(d > 0))",
     "        R d = s_get_##SUF(A, lda, upper, j, j).re - s;                          \\\n        if (!(d > 0)) {",
     "        R d = s_get_##SUF(A, lda, upper, j, j).re - s;                          \\\n        if (d < 0) {"),
    ("transposed operand in the real update",
     "                     *s_at_##SUF(A, lda, upper, j, p);",
     "                     *s_at_##SUF(A, lda, upper, p, j);"),
    ("dropped term in the real forward solve",
     "            for (int64_t p = 0; p < i; ++p)                                     \\\n                t -= *s_at_##SUF(Am, lda, upper, i, p) * b[p];",
     "            for (int64_t p = 1; p < i; ++p)                                     \\\n                t -= *s_at_##SUF(Am, lda, upper, i, p) * b[p];"),
    ("missing conj in the complex backward solve",
     "                t.re -= l.re * x.re + l.im * x.im;",
     "                t.re -= l.re * x.re - l.im * x.im;"),
]


def _pins_fail(lib) -> list[str]:
    """Run a compact set of pins against a (possibly broken) oracle library."""
    failures = []
    rng = np.random.default_rng(5)
    for dt in ("f32", "c128"):
        d = syn.np_dtype(dt)
        l0s = np.stack([integer_factor(9, syn.is_complex(dt), rng) for _ in range(3)])
        a = np.stack([exact_product(l) for l in l0s])
        for uplo in ("L", "U"):
            f, info = oracle.potrf_matrices(a.astype(d), uplo, lib=lib)
            want = l0s if uplo == "L" else np.conj(np.swapaxes(l0s, 1, 2))
            view = np.tril if uplo == "L" else np.triu
            if not ((info == 0).all() and np.array_equal(view(f), view(want.astype(d)))):
                failures.append(f"integer factor {dt} {uplo}")
        x0 = rng.integers(-2, 3, size=(3, 9, 2)).astype(a.dtype)
        if syn.is_complex(dt):
            x0 = x0 + 1j * rng.integers(-2, 3, size=(3, 9, 2))
        _, x, info = oracle.posv_matrices(a.astype(d), np.matmul(a, x0).astype(d), "L", lib=lib)
        if not ((info == 0).all() and np.array_equal(x, x0.astype(d))):
            failures.append(f"integer solve {dt}")
        stale = np.array([[[1, .75, .75], [.75, 1, -.75], [.75, -.75, 1]]], dtype=d)
        _, info = oracle.potrf_matrices(stale, "L", lib=lib)
        if info[0] != 3:
            failures.append(f"stale pivot {dt}")
        one = np.array([0.0, np.nan, 2.0], dtype=d).reshape(3, 1, 1)
        _, info = oracle.potrf_matrices(one, "L", lib=lib)
        if list(info) != [1, 1, 0]:
            failures.append(f"1x1 pivots {dt}")
    return failures


def test_shipped_oracle_passes_the_compact_pins():
    assert _pins_fail(None) == []


@pytest.mark.parametrize("name,old,new", BREAKS, ids=[b[0] for b in BREAKS])
def test_planted_break_turns_a_pin_red(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"break '{name}' no longer matches the source"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new))
    so = oracle.compile_source(str(mutant), str(tmp_path / "libmutant.so"))
    lib = oracle.open_library(so)
    assert _pins_fail(lib), f"no pin caught: {name}"
