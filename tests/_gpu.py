"""Helpers for the GPU parity tests: run the HIP path through the C ABI and the
CPU oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import json
import os
import sys

import numpy as np

import oracle
import synthetic as syn
from tests._checks import (RESIDUAL_BOUND, TOL, bits_equal, factor_residual, rel_err,
                           rel_err_triangle, solve_residual)


def announce(*parts):
    print("[case]", *parts, file=sys.stderr, flush=True)


def record_error(kind: str, label: str, dt: str, uplo: str, n: int, batch: int, **errs):
    """Print the observed worst-case errors of a parity case, and append them to
    the JSON-lines file named by BATCHLAS_PARITY_LOG when that is set."""
    vals = {k: float(v) for k, v in errs.items()}
    print("[errors]", kind, label, dt, uplo, f"n={n}", f"batch={batch}",
          " ".join(f"{k}={v:.3e}" for k, v in vals.items()), file=sys.stderr, flush=True)
    path = os.environ.get("BATCHLAS_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(dict(kind=kind, label=label, dt=dt, uplo=uplo, n=n, batch=batch,
                                    **vals)) + "\n")


def torch_dtype(dt):
    import torch
    return {"f32": torch.float32, "f64": torch.float64, "c64": torch.complex64,
            "c128": torch.complex128}[syn.dtype_name(dt)]


def gpu_potrf(buf: np.ndarray, uplo: str, n: int, batch: int, lda: int, stride: int,
              family: str = "auto", with_info: bool = True):
    import torch
    import dense_linear_algebra_potrf_amd as bl
    t = torch.from_numpy(buf.copy()).cuda()
    info = bl.potrf(t, uplo, None if with_info else False, n=n, lda=lda, stride=stride,
                    batch=batch, family=family)
    torch.cuda.synchronize()
    return t.cpu().numpy(), (info.cpu().numpy() if with_info else None)


def gpu_posv(abuf, bbuf, uplo, n, nrhs, batch, lda, strideA, ldb, strideB, family="auto"):
    import torch
    import dense_linear_algebra_potrf_amd as bl
    ta = torch.from_numpy(abuf.copy()).cuda()
    tb = torch.from_numpy(bbuf.copy()).cuda()
    info = bl.posv(ta, tb, uplo, n=n, nrhs=nrhs, lda=lda, strideA=strideA, ldb=ldb,
                   strideB=strideB, batch=batch, family=family)
    torch.cuda.synchronize()
    return ta.cpu().numpy(), tb.cpu().numpy(), info.cpu().numpy()


def check_potrf(a: np.ndarray, uplo: str, family: str = "auto", padded: bool = False,
                fill=None, expect_info=None, tol_scale: float = 1.0, label: str = ""):
    """Run GPU and oracle on the same input and assert parity.  Returns (gpu, oracle, info)."""
    batch, n, _ = a.shape
    dt = syn.dtype_name(a.dtype)
    announce("potrf", label, dt, uplo, f"n={n}", f"batch={batch}", family,
             "padded" if padded else "packed", "fill" if fill is not None else "")
    lda, stride = syn.layout(n, padded=padded)
    src = a if fill is None else syn.poison(a, uplo, fill)
    buf = syn.to_colmajor(src, lda, stride, fill=0 if fill is None else fill)
    ref = buf.copy()
    info_ref = oracle.potrf(ref, uplo, n, batch, lda, stride)
    out, info = gpu_potrf(buf, uplo, n, batch, lda, stride, family)
    # info: bit-exact on every item
    assert np.array_equal(info, info_ref), \
        f"info mismatch at items {np.nonzero(info != info_ref)[0][:10]}"
    if expect_info is not None:
        assert np.array_equal(info, expect_info)
    got = syn.from_colmajor(out, n, n, batch, lda, stride)
    want = syn.from_colmajor(ref, n, n, batch, lda, stride)
    ok = np.nonzero(info_ref == 0)[0]
    tol = TOL[dt] * tol_scale
    if ok.size:
        err = rel_err_triangle(got, want, uplo, ok)
        worst = int(ok[np.argmax(err)])
        res = factor_residual(a, got, uplo, ok)
        if label.startswith("config"):
            record_error("potrf", label, dt, uplo, n, batch, factor_rel=err.max(),
                         residual=res.max())
        assert err.max() <= tol, f"factor rel err {err.max():.3e} > {tol} (item {worst})"
        assert res.max() <= RESIDUAL_BOUND, f"residual {res.max():.2f} > {RESIDUAL_BOUND}"
    # failed items: the leading info-1 columns are the leading block's factor
    for b in np.nonzero(info_ref > 0)[0][:64]:
        k = int(info_ref[b]) - 1
        if k == 0:
            continue
        g = got[b][:, :k] if uplo == "L" else got[b][:k, :]
        w = want[b][:, :k] if uplo == "L" else want[b][:k, :]
        m = syn.referenced_mask(n, uplo)
        m = m[:, :k] if uplo == "L" else m[:k, :]
        wv, gv = w[m].astype(np.complex128), g[m].astype(np.complex128)
        e = np.linalg.norm(gv - wv) / max(np.linalg.norm(wv), 1e-300)
        assert e <= tol, f"failed item {b}: leading columns differ ({e:.3e})"
    # the other triangle and the padding are bit-identical to the input
    touched = np.zeros(buf.size, dtype=bool)
    tv = touched.reshape(batch, stride)[:, : lda * n].reshape(batch, n, lda)
    tv[:, :, :n] = np.swapaxes(np.broadcast_to(syn.referenced_mask(n, uplo), (batch, n, n)), 1, 2)
    assert bits_equal(out[~touched], buf[~touched]), "wrote outside the referenced triangle"
    return got, want, info


def check_posv(a, b, uplo, family="auto", padded=False, label=""):
    batch, n, _ = a.shape
    nrhs = b.shape[2]
    dt = syn.dtype_name(a.dtype)
    announce("posv", label, dt, uplo, f"n={n}", f"nrhs={nrhs}", f"batch={batch}", family)
    lda, strideA = syn.layout(n, padded=padded)
    ldb, strideB = syn.layout(n, nrhs, padded=padded)
    abuf = syn.to_colmajor(syn.poison(a, uplo, syn.sentinel(dt)), lda, strideA,
                           fill=syn.sentinel(dt))
    bbuf = syn.to_colmajor(b, ldb, strideB, fill=syn.sentinel(dt))
    aref, bref = abuf.copy(), bbuf.copy()
    info_ref = oracle.posv(aref, bref, uplo, n, nrhs, batch, lda, strideA, ldb, strideB)
    aout, bout, info = gpu_posv(abuf, bbuf, uplo, n, nrhs, batch, lda, strideA, ldb, strideB,
                                family)
    assert np.array_equal(info, info_ref), \
        f"info mismatch at items {np.nonzero(info != info_ref)[0][:10]}"
    ok = np.nonzero(info_ref == 0)[0]
    x = syn.from_colmajor(bout, n, nrhs, batch, ldb, strideB)
    xr = syn.from_colmajor(bref, n, nrhs, batch, ldb, strideB)
    fa = syn.from_colmajor(aout, n, n, batch, lda, strideA)
    far = syn.from_colmajor(aref, n, n, batch, lda, strideA)
    tol = TOL[dt]
    if ok.size:
        ferr = rel_err_triangle(fa, far, uplo, ok).max()
        xerr = rel_err(x, xr, ok).max()
        sres = solve_residual(a, x, b, ok).max()
        if label.startswith("config"):
            record_error("posv", label, dt, uplo, n, batch, factor_rel=ferr, x_rel=xerr,
                         residual=sres)
        assert ferr <= tol, f"factor rel err {ferr:.3e} > {tol}"
        # X at the same stated tolerance: with kappa(A) <= 5 the solves add about
        # n u kappa (2e-5 at fp32 n = 32) to the factor's error
        assert xerr <= tol, f"solution rel err {xerr:.3e} > {tol}"
        assert sres <= RESIDUAL_BOUND, f"solve residual {sres:.2f} > {RESIDUAL_BOUND}"
    bad = np.nonzero(info_ref > 0)[0]
    if bad.size:
        assert bits_equal(x[bad], b[bad].astype(x.dtype)), "B changed for a failed item"
    # padding of A and B untouched
    assert bits_equal(bout.reshape(batch, strideB)[:, ldb * nrhs:],
                      bbuf.reshape(batch, strideB)[:, ldb * nrhs:])
    return x, xr, info
