"""GPU parity of the tiny family's folded window against the CPU oracle: fp64
and cfloat at orders 33..64, two matrices per wavefront, lane q holding rows q
and 63 - q of its matrix (rows at or beyond n hold the identity); Upper moves
the matrix through LDS in slabs of whole cache lines.

Same bar as the other families: info bit-exact on every item, the referenced
triangle within 1e-4 (cfloat) or 1e-11 (fp64) relative Frobenius error per
item, the other triangle and the padding untouched.  The cases aim at what is
particular to the window: failures on either side of the fold (rows 31 and 32
are the short and the long row of lane 31), Schur pivots that only fail after
updates across it, a second matrix of the pair that does not exist (odd
batches, batch 1), batches beyond the launch's grid cap, strides whose pair of
matrices overflows the 31-bit offsets (then the one-wavefront window serves),
and thousands of distinct items.  Every order and the padded layouts are in
the tiny family's tests (test_gpu_potrf).
"""
from __future__ import annotations

import numpy as np
import pytest

import synthetic as syn
from tests._gpu import announce, check_potrf

pytestmark = pytest.mark.gpu

UPLOS = ["L", "U"]
DTS = ["f64", "c64"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    import dense_linear_algebra_potrf_amd as bl
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bl.load_library()
    yield
    torch.cuda.empty_cache()


def _bits(t):
    import torch
    return t.view(torch.int64)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("uplo", UPLOS)
@pytest.mark.parametrize("n", [33, 48, 64])
def test_fold_info_first_failure_nan_and_stale_pivot(dt, uplo, n):
    """The first failing column wins; NaN and zero pivots fail; a pivot that
    goes non-positive only in its Schur complement fails at that column, here
    with the chain crossing the fold (rows 30, 31 short, row 32 long)."""
    import dense_linear_algebra_potrf_amd as bl
    r = bl.route(dt, uplo, n, 9, family="tiny")
    assert (r["lanes_per_matrix"], r["rows_per_lane"], r["matrices_per_wave"]) == (32, 2, 2)
    a = syn.spd_matrices(n, 9, dt, seed=71 + n)
    a[0, 3, 3] *= -1
    a[0, n - 2, n - 2] *= -1                  # two plants: the first wins
    a[1, 0, 0] = syn.nan_value(dt)            # NaN pivot in the first column
    a[2, 32, 32] = syn.nan_value(dt)          # the first long row's own pivot
    a[3, n - 1, n - 1] = -a[3, n - 1, n - 1]  # last column
    stale = np.eye(n)
    idx = [30, 31, 32]
    stale[np.ix_(idx, idx)] = [[1, .75, .75], [.75, 1, -.75], [.75, -.75, 1]]
    a[4] = stale.astype(a.dtype)              # unit diagonal: only the Schur pivot of column 33 fails
    a[5, 31, 31] = 0                          # exact zero pivot on the last short row
    a[6, 16, 16] *= -1
    stale2 = np.eye(n)
    idx2 = [n - 3, n - 2, n - 1]
    stale2[np.ix_(idx2, idx2)] = [[1, .75, .75], [.75, 1, -.75], [.75, -.75, 1]]
    a[7] = stale2.astype(a.dtype)             # the chain at the last rows (long rows only)
    _, _, info = check_potrf(a, uplo, family="tiny", label="fold-info")
    assert list(info) == [4, 1, 33, n, 33, 32, 17, n, 0]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("uplo", UPLOS)
def test_fold_small_and_odd_batches(dt, uplo):
    """Batches of 1, 2, 3 and 129: the last pair's second matrix is missing
    whenever the batch is odd; nothing of it is read or written (the padded
    layout keeps sentinels around every matrix)."""
    for n in (33, 47, 64):
        for batch in (1, 2, 3, 129):
            a = syn.spd_matrices(n, batch, dt, seed=n * 7 + batch)
            want = syn.plant_failures(a, seed=batch, every=3)
            check_potrf(a, uplo, family="tiny", expect_info=want, label="fold-batch")
            check_potrf(a, uplo, family="tiny", padded=True, fill=syn.sentinel(dt),
                        label="fold-batch-padded")


@pytest.mark.parametrize("dt,uplo,n", [("c64", "U", 33), ("c64", "L", 48), ("f64", "L", 33),
                                       ("f64", "U", 40)])
def test_fold_batch_beyond_the_grid_cap_is_uniform(dt, uplo, n):
    """More pairs than the launch's workgroups (2^19): every workgroup loops
    over several pairs, and the odd batch leaves the last pair half empty.
    Identical items give the solo result bit for bit; compared on the device."""
    import torch
    import dense_linear_algebra_potrf_amd as bl
    batch = (1 << 20) + 5
    r = bl.route(dt, uplo, n, batch, family="tiny")
    assert r["grid"] == 1 << 19 and r["matrices_per_wave"] == 2
    one = syn.spd_matrices(n, 1, dt, seed=3 * n)
    solo = torch.from_numpy(syn.to_colmajor(one)).cuda()
    bl.potrf(solo, uplo, n=n, batch=1, family="tiny")
    announce("fold beyond grid cap", dt, uplo, f"n={n}", f"batch={batch}")
    many = torch.from_numpy(syn.to_colmajor(one)).cuda().repeat(batch)
    info = bl.potrf(many, uplo, n=n, batch=batch, family="tiny")
    torch.cuda.synchronize()
    assert int((info != 0).sum()) == 0
    assert torch.equal(_bits(many).view(batch, -1), _bits(solo).view(1, -1).expand(batch, -1))
    del many, info
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dt,uplo", [("c64", "L"), ("f64", "U")])
def test_fold_stride_beyond_a_pair_uses_the_one_wavefront_window(dt, uplo):
    """A stride whose pair of matrices overflows the 31-bit buffer offsets
    while one matrix fits: the route keeps the tiny family's one-wavefront
    window (64 lanes per matrix), and the result matches the oracle."""
    import torch
    import dense_linear_algebra_potrf_amd as bl
    import oracle
    from tests._checks import TOL, rel_err_triangle
    n, batch = 40, 2
    stride = (1 << 31) // 16 + 64                  # 2 stride elements > 2^31 bytes > stride elements
    r = bl.route(dt, uplo, n, batch, stride=stride)
    assert r["family"] == "tiny" and r["lanes_per_matrix"] == 64, r
    a = syn.spd_matrices(n, batch, dt, seed=17)
    syn.plant_failures(a, seed=5, every=2)
    dense = syn.to_colmajor(a)
    announce("fold stride fallback", dt, uplo, f"n={n}", f"stride={stride}")
    t = torch.zeros(stride * (batch - 1) + n * n, dtype=torch.float64 if dt == "f64" else torch.complex64,
                    device="cuda")
    for b in range(batch):
        t[b * stride:b * stride + n * n] = torch.from_numpy(dense[b * n * n:(b + 1) * n * n]).cuda()
    info = bl.potrf(t, uplo, n=n, batch=batch, stride=stride)
    torch.cuda.synchronize()
    got = np.concatenate([t[b * stride:b * stride + n * n].cpu().numpy() for b in range(batch)])
    ref = dense.copy()
    want_info = oracle.potrf(ref, uplo, n, batch, n, n * n)
    assert list(info.cpu().numpy()) == list(want_info)
    g = syn.from_colmajor(got, n, n, batch, n, n * n)
    w = syn.from_colmajor(ref, n, n, batch, n, n * n)
    ok = np.asarray(want_info) == 0
    assert float(rel_err_triangle(g[ok], w[ok], uplo).max(initial=0.0)) <= TOL[dt]
    del t
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dt,uplo,n,batch", [("c64", "U", 64, 4096), ("c64", "L", 40, 2049),
                                              ("f64", "L", 48, 4096), ("f64", "U", 64, 2047)])
def test_fold_batch_of_distinct_items_matches_the_oracle_at_every_item(dt, uplo, n, batch):
    """Thousands of distinct matrices (cfloat Upper n = 64: the secondary
    workload's shape): every item against the oracle, in chunks."""
    import torch
    import dense_linear_algebra_potrf_amd as bl
    import oracle
    from tests._checks import TOL, rel_err_triangle
    a = syn.spd_matrices(n, batch, dt, seed=1010 + n)
    buf = syn.to_colmajor(a)
    announce("fold distinct", dt, uplo, f"n={n}", f"batch={batch}")
    t = torch.from_numpy(buf).cuda()
    info = bl.potrf(t, uplo, n=n, batch=batch)
    torch.cuda.synchronize()
    assert int((info != 0).sum()) == 0
    out = t.cpu().numpy()
    worst = 0.0
    for c0 in range(0, batch, 512):
        m = min(512, batch - c0)
        ref = buf[c0 * n * n:(c0 + m) * n * n].copy()
        assert (oracle.potrf(ref, uplo, n, m, n, n * n) == 0).all()
        got = syn.from_colmajor(out[c0 * n * n:(c0 + m) * n * n], n, n, m, n, n * n)
        want = syn.from_colmajor(ref, n, n, m, n, n * n)
        worst = max(worst, float(rel_err_triangle(got, want, uplo).max()))
    assert worst <= TOL[dt], worst
