"""GPU parity of the tiny family's folded window against the CPU oracle: a
window of NB rows on NB / 2 lanes per matrix, lane q holding rows q and
NB - 1 - q (rows at or beyond n hold the identity); Upper moves the matrix
through LDS in slabs of whole (or half) cache lines.  NB = 64 (two matrices
per wavefront) serves fp64 at 49..64, cfloat at 57..64 and fp32 Lower at
49..64; NB = 56 (28 lanes of a 32-lane group, two matrices per wavefront)
cfloat at 49..56; NB = 48 (24 lanes of a 32-lane group) fp64 and cfloat at
33..48 and fp32 at 35..48; NB = 128 (one matrix per wavefront) fp32 Upper at
97..128; NB = 34 (17 lanes per matrix, three matrices per wavefront) fp32
Lower at 34; NB = 32 (16 lanes, four matrices per wavefront) cdouble Lower at
17..32, fp64 at 25..32 and fp32 Upper at 25..32.

Same bar as the other families: info bit-exact on every item, the referenced
triangle within 1e-4 (cfloat) or 1e-11 (fp64) relative Frobenius error per
item, the other triangle and the padding untouched.  The cases aim at what is
particular to the window: failures on either side of the fold (rows NB/2 - 1
and NB/2 are the short and the long row of the last lane), Schur pivots that
only fail after updates across it, a second matrix of the pair that does not exist (odd
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
# (dtype, triangle, orders) served by the folded window
ROUTES = [("f64", uplo, (25, 32, 33, 48, 49, 56, 57, 64)) for uplo in UPLOS] + \
         [("c64", uplo, (33, 48, 49, 56, 57, 64)) for uplo in UPLOS] + \
         [("f32", "L", (34, 35, 48, 49, 64)), ("f32", "U", (25, 32, 35, 48, 97, 112, 128)),
          ("c128", "L", (17, 24, 32))]


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


def _route_cases():
    return [(dt, uplo, n) for dt, uplo, orders in ROUTES for n in orders]


@pytest.mark.parametrize("dt,uplo,n", _route_cases())
def test_fold_info_first_failure_nan_and_stale_pivot(dt, uplo, n):
    """The first failing column wins; NaN and zero pivots fail; a pivot that
    goes non-positive only in its Schur complement fails at that column, here
    with the chain crossing the fold (rows h - 2, h - 1 short, row h long, for
    h = NB/2)."""
    import dense_linear_algebra_potrf_amd as bl
    r = bl.route(dt, uplo, n, 9, family="tiny")
    h = r["lanes_per_matrix"]                 # NB / 2
    assert h in (16, 17, 24, 28, 32, 64) and (r["rows_per_lane"], r["matrices_per_wave"]) == (2, 64 // h)
    a = syn.spd_matrices(n, 9, dt, seed=71 + n)
    a[0, 3, 3] *= -1
    a[0, n - 2, n - 2] *= -1                  # two plants: the first wins
    a[1, 0, 0] = syn.nan_value(dt)            # NaN pivot in the first column
    a[2, h, h] = syn.nan_value(dt)            # the first long row's own pivot
    a[3, n - 1, n - 1] = -a[3, n - 1, n - 1]  # last column
    stale = np.eye(n)
    idx = [h - 2, h - 1, h]
    stale[np.ix_(idx, idx)] = [[1, .75, .75], [.75, 1, -.75], [.75, -.75, 1]]
    a[4] = stale.astype(a.dtype)              # unit diagonal: only the Schur pivot of column h + 1 fails
    a[5, h - 1, h - 1] = 0                    # exact zero pivot on the last short row
    a[6, 16, 16] *= -1
    stale2 = np.eye(n)
    idx2 = [n - 3, n - 2, n - 1]
    stale2[np.ix_(idx2, idx2)] = [[1, .75, .75], [.75, 1, -.75], [.75, -.75, 1]]
    a[7] = stale2.astype(a.dtype)             # the chain at the last rows (long rows only)
    _, _, info = check_potrf(a, uplo, family="tiny", label="fold-info")
    assert list(info) == [4, 1, h + 1, n, h + 1, h, 17, n, 0]


@pytest.mark.parametrize("dt,uplo,orders", ROUTES)
def test_fold_small_and_odd_batches(dt, uplo, orders):
    """Batches of 1, 2, 3 and 129: with two matrices per wavefront the last
    one's second matrix is missing whenever the batch is odd; nothing of it is
    read or written (the padded layout keeps sentinels around every matrix)."""
    lo, hi = orders[0], orders[-1]
    for n in (lo, (lo + hi) // 2 | 1, hi):
        for batch in (1, 2, 3, 129):
            a = syn.spd_matrices(n, batch, dt, seed=n * 7 + batch)
            want = syn.plant_failures(a, seed=batch, every=3)
            check_potrf(a, uplo, family="tiny", expect_info=want, label="fold-batch")
            check_potrf(a, uplo, family="tiny", padded=True, fill=syn.sentinel(dt),
                        label="fold-batch-padded")


@pytest.mark.parametrize("dt,uplo,n", [("c64", "U", 33), ("c64", "L", 48), ("f64", "L", 33),
                                       ("f64", "U", 40), ("f32", "L", 40), ("f32", "U", 100),
                                       ("f32", "L", 34), ("c128", "L", 20), ("c64", "U", 52),
                                       ("f64", "U", 28)])
def test_fold_batch_beyond_the_grid_cap_is_uniform(dt, uplo, n):
    """More wavefronts of matrices than the launch's workgroups (2^19): every
    workgroup loops over several, and with two matrices per wavefront the odd
    batch leaves the last one half empty.  Identical items give the solo
    result bit for bit; compared on the device."""
    import torch
    import dense_linear_algebra_potrf_amd as bl
    mpw = bl.route(dt, uplo, n, 1000, family="tiny")["matrices_per_wave"]
    batch = mpw * (1 << 19) + 5            # (odd: the last wavefront partly empty)
    r = bl.route(dt, uplo, n, batch, family="tiny")
    assert r["grid"] == 1 << 19 and r["grid"] * r["matrices_per_wave"] < batch
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


@pytest.mark.parametrize("dt,uplo", [("c64", "L"), ("f64", "U"), ("f32", "L")])
def test_fold_stride_beyond_a_pair_uses_the_one_wavefront_window(dt, uplo):
    """A stride whose pair of matrices overflows the 31-bit buffer offsets
    while one matrix fits: the route keeps the tiny family's one-wavefront
    window (64 lanes per matrix), and the result matches the oracle."""
    import torch
    import dense_linear_algebra_potrf_amd as bl
    import oracle
    from tests._checks import TOL, rel_err_triangle
    n, batch = 40, 2
    es = 4 if dt == "f32" else 8
    stride = (1 << 31) // (2 * es) + 64            # 2 stride elements > 2^31 bytes > stride elements
    r = bl.route(dt, uplo, n, batch, stride=stride)
    assert r["family"] == "tiny" and r["lanes_per_matrix"] == 64, r
    a = syn.spd_matrices(n, batch, dt, seed=17)
    syn.plant_failures(a, seed=5, every=2)
    dense = syn.to_colmajor(a)
    announce("fold stride fallback", dt, uplo, f"n={n}", f"stride={stride}")
    tdt = {"f32": torch.float32, "f64": torch.float64, "c64": torch.complex64}[dt]
    t = torch.zeros(stride * (batch - 1) + n * n, dtype=tdt, device="cuda")
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
                                              ("f64", "L", 48, 4096), ("f64", "U", 64, 2047),
                                              ("f32", "L", 64, 4095), ("f32", "U", 128, 2048),
                                              ("f32", "L", 34, 16383), ("c128", "L", 32, 2047),
                                              ("c64", "U", 56, 4096), ("f64", "L", 32, 8191)])
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
