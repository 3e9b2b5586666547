"""Pins for the CPU oracle, checked against things other than the oracle itself.

Each group catches a different class of mistake:
  * exact recovery of an integer factor L0 from A = L0 L0^H (closed form: every
    partial sum is an integer below 2^24, every division exact, every square
    root of a perfect square) -- catches a dropped term, a wrong sign, a wrong
    index, a missing conj, a transposed operand, in fp32 and fp64;
  * brute force on tiny inputs against exact integer arithmetic (Sylvester's
    criterion: the first failing Schur pivot is the first leading minor <= 0);
  * LAPACK (scipy's ?potrf / ?posv) on the same inputs;
  * invariants: Upper = Lower^H, batch permutation, padded layouts, the other
    triangle and padding untouched, planted failures at a known column;
  * the error bound: residual <= 10 n eps ||A||.
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest
import scipy.linalg.lapack as lapack

import oracle
import synthetic as syn
from tests._checks import (RESIDUAL_BOUND, bits_equal, factor_residual, rel_err,
                           rel_err_triangle, solve_residual)

DTS = ["f32", "f64", "c64", "c128"]
UPLOS = ["L", "U"]


def integer_factor(n: int, cplx: bool, rng) -> np.ndarray:
    """Random lower-triangular integer (Gaussian-integer) L0 with diag in 1..4."""
    l0 = np.tril(rng.integers(-4, 5, size=(n, n)), -1).astype(np.complex128 if cplx else np.float64)
    if cplx:
        l0 = l0 + 1j * np.tril(rng.integers(-4, 5, size=(n, n)), -1)
    l0[np.arange(n), np.arange(n)] = rng.integers(1, 5, size=n)
    return l0


def exact_product(l0: np.ndarray) -> np.ndarray:
    """A = L0 L0^H with Python-integer arithmetic (exact), as float64/complex128."""
    n = l0.shape[0]
    re = [[int(l0[i, j].real) for j in range(n)] for i in range(n)]
    im = [[int(l0[i, j].imag) for j in range(n)] for i in range(n)]
    a_re = np.zeros((n, n))
    a_im = np.zeros((n, n))
    for i in range(n):
        for j in range(n):
            sr = si = 0
            for p in range(n):
                # (re_ip + i im_ip)(re_jp - i im_jp)
                sr += re[i][p] * re[j][p] + im[i][p] * im[j][p]
                si += im[i][p] * re[j][p] - re[i][p] * im[j][p]
            assert abs(sr) < 2 ** 23 and abs(si) < 2 ** 23
            a_re[i, j] = sr
            a_im[i, j] = si
    if np.iscomplexobj(l0):
        return a_re + 1j * a_im
    return a_re


def full_factor_view(f: np.ndarray, uplo: str) -> np.ndarray:
    """The referenced triangle of a result, as L (Lower) or U (Upper)."""
    return np.tril(f) if uplo == "L" else np.triu(f)


# ----------------------------------------------------------------------------- P1
@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("uplo", UPLOS)
@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 13, 17, 32])
def test_integer_factor_is_recovered_exactly(dt, uplo, n):
    rng = np.random.default_rng(1000 + n)
    cplx = syn.is_complex(dt)
    batch = 6
    l0s = np.stack([integer_factor(n, cplx, rng) for _ in range(batch)])
    a = np.stack([exact_product(l) for l in l0s]).astype(syn.np_dtype(dt))
    f, info = oracle.potrf_matrices(a, uplo)
    assert (info == 0).all()
    want = l0s if uplo == "L" else np.conj(np.swapaxes(l0s, 1, 2))
    want = want.astype(syn.np_dtype(dt))
    got = full_factor_view(f, uplo)
    # exact values (a signed zero in an imaginary part is an arithmetic artefact)
    assert np.array_equal(got, full_factor_view(want, uplo)), "factor of an integer L0 must be exact"


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("uplo", UPLOS)
@pytest.mark.parametrize("n", [1, 4, 11, 16])
def test_integer_solution_is_recovered_exactly(dt, uplo, n):
    rng = np.random.default_rng(2000 + n)
    cplx = syn.is_complex(dt)
    batch, nrhs = 4, 3
    l0s = np.stack([integer_factor(n, cplx, rng) for _ in range(batch)])
    a = np.stack([exact_product(l) for l in l0s])
    x0 = rng.integers(-2, 3, size=(batch, n, nrhs)).astype(a.dtype)
    if cplx:
        x0 = x0 + 1j * rng.integers(-2, 3, size=(batch, n, nrhs))
    b = np.matmul(a, x0)                       # exact: small integers in float64
    assert np.abs(b).max() < 2 ** 22
    d = syn.np_dtype(dt)
    f, x, info = oracle.posv_matrices(a.astype(d), b.astype(d), uplo)
    assert (info == 0).all()
    assert np.array_equal(x, x0.astype(d)), "posv of A = L0 L0^H, B = A X0 must return X0 exactly"


# ----------------------------------------------------------------------------- P2
@pytest.mark.parametrize("dt", DTS)
def test_one_by_one(dt):
    d = syn.np_dtype(dt)
    vals = [4.0, 2.0, 1e-3, 0.0, -0.0, -1.0, np.nan, np.inf * -1]
    a = np.array(vals, dtype=d).reshape(-1, 1, 1)
    f, info = oracle.potrf_matrices(a, "L")
    for k, v in enumerate(vals):
        ok = v > 0
        assert info[k] == (0 if ok else 1)
        if ok:
            assert f[k, 0, 0] == np.sqrt(syn.real_dtype(dt).type(v))


@pytest.mark.parametrize("dt", DTS)
def test_two_by_two_against_exact_rationals(dt):
    from fractions import Fraction
    rng = np.random.default_rng(7)
    d = syn.np_dtype(dt)
    for _ in range(50):
        a11 = float(rng.uniform(0.5, 4))
        a21 = float(rng.uniform(-1, 1))
        a22 = float(rng.uniform(0.5, 4))
        m = np.array([[[a11, a21], [a21, a22]]], dtype=d)
        f, info = oracle.potrf_matrices(m, "L")
        fa11, fa21, fa22 = (Fraction(float(np.real(m[0, 0, 0]))), Fraction(float(np.real(m[0, 1, 0]))),
                            Fraction(float(np.real(m[0, 1, 1]))))
        det = fa11 * fa22 - fa21 * fa21
        assert info[0] == (0 if det > 0 else 2)
        tol = 8 * float(np.finfo(syn.real_dtype(dt)).eps)
        l11 = float(fa11) ** 0.5
        l21 = float(fa21) / l11
        l22 = float(det / fa11) ** 0.5          # l22^2 = det(A) / a11
        got = np.real(f[0])
        assert abs(got[0, 0] - l11) <= tol * l11
        assert abs(got[1, 0] - l21) <= tol * max(1.0, abs(l21))
        assert abs(got[1, 1] - l22) <= 4 * tol * l22 / min(1.0, float(det / fa11))


@pytest.mark.parametrize("dt", DTS)
def test_three_by_three_textbook_example(dt):
    d = syn.np_dtype(dt)
    a = np.array([[[4, 2, -2], [2, 10, 5], [-2, 5, 21]]], dtype=d)
    f, info = oracle.potrf_matrices(a, "L")
    assert info[0] == 0
    assert np.array_equal(np.tril(f[0]), np.array([[2, 0, 0], [1, 3, 0], [-1, 2, 4]], dtype=d))


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("uplo", UPLOS)
def test_stale_pivot_trap(dt, uplo):
    """Unit diagonal, not positive definite: only the updated pivot d3 = -3.5 fails."""
    d = syn.np_dtype(dt)
    a = np.array([[[1, .75, .75], [.75, 1, -.75], [.75, -.75, 1]]], dtype=d)
    buf = syn.to_colmajor(a)
    info = oracle.potrf(buf, uplo, 3, 1)
    assert info[0] == 3
    f = syn.from_colmajor(buf, 3, 3, 1)
    assert np.real(f[0, 2, 2]) == pytest.approx(-3.5, rel=1e-5)


def _leading_minors_int(m):
    """Exact leading principal minors of a 3x3 (or 2x2) Hermitian Gaussian-integer matrix."""
    n = len(m)
    out = []
    for k in range(1, n + 1):
        if k == 1:
            out.append(m[0][0])
        elif k == 2:
            out.append(m[0][0] * m[1][1] - m[0][1] * m[1][0])
        else:
            a = m
            out.append(a[0][0] * (a[1][1] * a[2][2] - a[1][2] * a[2][1])
                       - a[0][1] * (a[1][0] * a[2][2] - a[1][2] * a[2][0])
                       + a[0][2] * (a[1][0] * a[2][1] - a[1][1] * a[2][0]))
    return out


def _sylvester_info(m):
    """First k with a leading minor <= 0 (1-based), 0 if none; None if borderline (== 0)."""
    for k, det in enumerate(_leading_minors_int(m), start=1):
        det = det.real if isinstance(det, complex) else det
        if det <= 0:
            return None if det == 0 else k
    return 0


@pytest.mark.parametrize("dt", ["f32", "f64"])
@pytest.mark.parametrize("n", [2, 3])
def test_info_exhaustive_small_integer_matrices(dt, n):
    """Every symmetric n x n matrix with entries in -3..3: info follows Sylvester."""
    vals = range(-3, 4)
    pos = [(i, j) for i in range(n) for j in range(i + 1)]
    mats, expect = [], []
    for entries in itertools.product(vals, repeat=len(pos)):
        m = [[0] * n for _ in range(n)]
        for (i, j), v in zip(pos, entries):
            m[i][j] = m[j][i] = v
        e = _sylvester_info(m)
        if e is None:
            continue
        mats.append(m)
        expect.append(e)
    a = np.array(mats, dtype=syn.np_dtype(dt))
    _, info = oracle.potrf_matrices(a, "L")
    assert np.array_equal(info, np.array(expect, dtype=np.int32))
    assert len(mats) >= 0.5 * 7 ** len(pos)


@pytest.mark.parametrize("dt", ["c64", "c128"])
def test_info_exhaustive_small_hermitian_matrices(dt):
    """3x3 Hermitian with diag in -3..3 and off-diagonals in {-1,0,1} + i{-1,0,1}."""
    gauss = [complex(r, i) for r in (-1, 0, 1) for i in (-1, 0, 1)]
    mats, expect = [], []
    for d0, d1, d2 in itertools.product(range(-3, 4), repeat=3):
        for a10, a20, a21 in itertools.product(gauss, repeat=3):
            m = [[complex(d0), a10.conjugate(), a20.conjugate()],
                 [a10, complex(d1), a21.conjugate()],
                 [a20, a21, complex(d2)]]
            e = _sylvester_info(m)
            if e is None:
                continue
            mats.append(m)
            expect.append(e)
    a = np.array(mats, dtype=syn.np_dtype(dt))
    _, info = oracle.potrf_matrices(a, "L")
    assert np.array_equal(info, np.array(expect, dtype=np.int32))
    _, info_u = oracle.potrf_matrices(a, "U")
    assert np.array_equal(info_u, np.array(expect, dtype=np.int32))


# ----------------------------------------------------------------------------- P3
_LAPACK_POTRF = {"f32": lapack.spotrf, "f64": lapack.dpotrf, "c64": lapack.cpotrf, "c128": lapack.zpotrf}
_LAPACK_POSV = {"f32": lapack.sposv, "f64": lapack.dposv, "c64": lapack.cposv, "c128": lapack.zposv}
_LAPACK_TOL = {"f32": 2e-5, "c64": 2e-5, "f64": 1e-13, "c128": 1e-13}


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("uplo", UPLOS)
@pytest.mark.parametrize("n", [1, 7, 17, 33, 64])
def test_potrf_matches_lapack(dt, uplo, n):
    batch = 40
    a = syn.spd_matrices(n, batch, dt, seed=300 + n)
    want_info = syn.plant_failures(a, seed=300 + n, every=8)
    f, info = oracle.potrf_matrices(a, uplo)
    assert np.array_equal(info, want_info)
    ref = np.empty_like(a)
    for b in range(batch):
        c, inf = _LAPACK_POTRF[dt](a[b], lower=(uplo == "L"), clean=0)
        assert inf == info[b]
        ref[b] = c
    ok = np.where(info == 0)[0]
    assert rel_err_triangle(f, ref, uplo, ok).max() <= _LAPACK_TOL[dt]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("uplo", UPLOS)
@pytest.mark.parametrize("n,nrhs", [(1, 1), (9, 2), (32, 4), (40, 7)])
def test_posv_matches_lapack(dt, uplo, n, nrhs):
    batch = 24
    a = syn.spd_matrices(n, batch, dt, seed=400 + n)
    want_info = syn.plant_failures(a, seed=400 + n, every=5)
    b = syn.rhs(n, nrhs, batch, dt, seed=400 + n)
    f, x, info = oracle.posv_matrices(a, b, uplo)
    assert np.array_equal(info, want_info)
    for k in range(batch):
        c, xr, inf = _LAPACK_POSV[dt](a[k], b[k], lower=(uplo == "L"))
        assert inf == info[k]
        if inf == 0:
            assert rel_err(x[k:k + 1], xr[None]).max() <= 10 * _LAPACK_TOL[dt]
        else:
            assert bits_equal(x[k], b[k]), "B must be unchanged for a failed item"


# ----------------------------------------------------------------------------- P4
@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("n", [8, 17, 33])
def test_planted_failure_reports_its_column(dt, n):
    """A = G G^H/n + I with A(k,k) negated: d_k <= -1, so info = k + 1 for every k."""
    a = syn.spd_matrices(n, n, dt, seed=500 + n)
    for k in range(n):
        a[k, k, k] = -a[k, k, k]
    for uplo in UPLOS:
        _, info = oracle.potrf_matrices(a, uplo)
        assert np.array_equal(info, np.arange(1, n + 1, dtype=np.int32))


@pytest.mark.parametrize("dt", DTS)
def test_first_failure_wins(dt):
    n = 12
    a = syn.spd_matrices(n, 3, dt, seed=9)
    a[0, 3, 3] *= -1
    a[0, 9, 9] *= -1
    a[1, 0, 0] = syn.nan_value(dt)
    a[2, 11, 11] = 0
    a[2, 5, 5] *= -1
    _, info = oracle.potrf_matrices(a, "L")
    assert list(info) == [4, 1, 6]


@pytest.mark.parametrize("dt", DTS)
def test_failed_item_keeps_leading_columns(dt):
    """After a failure at column j, columns < j equal the factor of the leading block."""
    n, k = 10, 6
    a = syn.spd_matrices(n, 1, dt, seed=11)
    good, info_good = oracle.potrf_matrices(a, "L")
    bad = a.copy()
    bad[0, k, k] = -bad[0, k, k]
    f, info = oracle.potrf_matrices(bad, "L")
    assert info_good[0] == 0 and info[0] == k + 1
    assert bits_equal(f[0][:, :k], good[0][:, :k])


@pytest.mark.parametrize("dt", DTS)
def test_upper_is_conjugate_transpose_of_lower(dt):
    n = 21
    a = syn.spd_matrices(n, 5, dt, seed=12)
    fl, il = oracle.potrf_matrices(a, "L")
    fu, iu = oracle.potrf_matrices(a, "U")
    assert (il == 0).all() and (iu == 0).all()
    # equal values: conj() of a real diagonal gives -0 imaginary parts in the reference
    assert np.array_equal(np.triu(fu), np.triu(np.conj(np.swapaxes(fl, 1, 2))))


@pytest.mark.parametrize("dt", DTS)
def test_batch_permutation_and_threads(dt):
    n, batch = 9, 37
    a = syn.spd_matrices(n, batch, dt, seed=13)
    syn.plant_failures(a, seed=13, every=6)
    f1, i1 = oracle.potrf_matrices(a, "L", nthreads=1)
    perm = np.random.default_rng(1).permutation(batch)
    f2, i2 = oracle.potrf_matrices(a[perm], "L", nthreads=5)
    assert bits_equal(f2, f1[perm]) and np.array_equal(i2, i1[perm])


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("uplo", UPLOS)
def test_padding_and_other_triangle_untouched(dt, uplo):
    n, batch = 11, 9
    a = syn.spd_matrices(n, batch, dt, seed=14)
    plain = syn.to_colmajor(a)
    info_plain = oracle.potrf(plain, uplo, n, batch)
    for fill in (syn.nan_value(dt), syn.sentinel(dt)):
        lda, stride = syn.layout(n, padded=True)
        src = syn.poison(a, uplo, fill)
        buf = syn.to_colmajor(src, lda, stride, fill=fill)
        before = buf.copy()
        info = oracle.potrf(buf, uplo, n, batch, lda, stride)
        assert np.array_equal(info, info_plain)
        got = syn.from_colmajor(buf, n, n, batch, lda, stride)
        want = syn.from_colmajor(plain, n, n, batch)
        mask = syn.referenced_mask(n, uplo)
        assert bits_equal(got[:, mask], want[:, mask])
        # everything outside the referenced triangle is bit-identical to the input
        touched = np.zeros(buf.size, dtype=bool)
        tv = touched.reshape(batch, stride)[:, : lda * n].reshape(batch, n, lda)
        tv[:, :, :n] = np.swapaxes(np.broadcast_to(mask, (batch, n, n)), 1, 2)
        assert bits_equal(buf[~touched], before[~touched])


@pytest.mark.parametrize("dt", DTS)
def test_diagonal_is_real_positive(dt):
    n = 16
    a = syn.spd_matrices(n, 8, dt, seed=15)
    if syn.is_complex(dt):
        idx = np.arange(n)
        a[:, idx, idx] += 1j * 5.0          # the imaginary part of the diagonal is ignored
    for uplo in UPLOS:
        f, info = oracle.potrf_matrices(a, uplo)
        assert (info == 0).all()
        dg = f[:, np.arange(n), np.arange(n)]
        assert (np.real(dg) > 0).all()
        if syn.is_complex(dt):
            assert (np.imag(dg) == 0).all() and not np.signbit(np.imag(dg)).any()


# ----------------------------------------------------------------------------- P5
@pytest.mark.parametrize("dt,n,batch", [("f32", 8, 64), ("f32", 17, 64), ("f32", 33, 64),
                                        ("c64", 64, 16), ("f64", 128, 4), ("c128", 48, 8),
                                        ("f64", 512, 1)])
def test_residual_and_forward_error_bounds(dt, n, batch):
    a = syn.spd_matrices(n, batch, dt, seed=600 + n)
    for uplo in UPLOS:
        f, info = oracle.potrf_matrices(a, uplo)
        assert (info == 0).all()
        assert factor_residual(a, f, uplo).max() <= RESIDUAL_BOUND
        # forward error against a float64 LAPACK factor of the same rounded input
        wide = np.complex128 if syn.is_complex(dt) else np.float64
        ref = np.stack([np.linalg.cholesky(a[b].astype(wide)) for b in range(batch)])
        if uplo == "U":
            ref = np.conj(np.swapaxes(ref, 1, 2))
        kappa = 5.0                                   # generator's condition number
        bound = 4 * n * float(np.finfo(syn.real_dtype(dt)).eps) * kappa
        assert rel_err_triangle(f, ref, uplo).max() <= bound


@pytest.mark.parametrize("dt", DTS)
def test_solve_residual_bound(dt):
    n, nrhs, batch = 32, 4, 32
    a = syn.spd_matrices(n, batch, dt, seed=700)
    b = syn.rhs(n, nrhs, batch, dt, seed=700)
    for uplo in UPLOS:
        _, x, info = oracle.posv_matrices(a, b, uplo)
        assert (info == 0).all()
        assert solve_residual(a, x, b).max() <= RESIDUAL_BOUND


def test_generator_condition_number():
    """kappa_2(A) of the generator stays below 5.5 at the workload sizes."""
    for dt, n in (("f32", 8), ("f32", 17), ("f32", 33), ("c64", 64), ("f64", 256)):
        a = syn.spd_matrices(n, 4, dt, seed=42)
        ev = np.linalg.eigvalsh(a.astype(np.complex128 if syn.is_complex(dt) else np.float64))
        assert (ev[:, 0] >= 1 - 1e-5).all()
        assert (ev[:, -1] / ev[:, 0]).max() < 5.5
