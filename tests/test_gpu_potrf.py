"""GPU parity of batched potrf against the CPU oracle, through the C ABI.

info must match bit-exactly on every item; the referenced triangle must match
within 1e-4 (fp32, complex-float) or 1e-11 (fp64, complex-double) relative
Frobenius error per item; the other triangle and all padding must be
bit-identical to the input (NaN pass: not read; sentinel pass: not written).
"""
from __future__ import annotations

import numpy as np
import pytest

import synthetic as syn
from tests._gpu import announce, check_potrf, gpu_potrf
from tests._checks import bits_equal

pytestmark = pytest.mark.gpu

DTS = ["f32", "f64", "c64", "c128"]
UPLOS = ["L", "U"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    import dense_linear_algebra_potrf_amd as bl
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bl.load_library()          # fails loudly if the HIP library is missing
    yield


def runnable(family, dt, n, uplo="L", batch=64):
    import dense_linear_algebra_potrf_amd as bl
    try:
        bl.route(dt, uplo, n, batch, family=family)
        return True
    except bl.BatchlasError:
        return False


def max_order(family, dt, limit=600):
    return max([n for n in (1, 2, 4, 8, 16, 17, 24, 32, 33, 48, 64, 96, 128, 142, 200, 256, 512)
                if n <= limit and runnable(family, dt, n)] or [0])


# ---------------------------------------------------------------- every order, tiny family
@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("uplo", UPLOS)
def test_tiny_every_order(dt, uplo):
    top = max(n for n in range(1, 65) if runnable("tiny", dt, n, uplo))
    for n in range(1, top + 1):
        a = syn.spd_matrices(n, 203, dt, seed=10 * n + (uplo == "U"))
        want = syn.plant_failures(a, seed=n, every=7)
        check_potrf(a, uplo, family="tiny", expect_info=want, label="every-order")


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("uplo", UPLOS)
def test_tiny_poison_and_padding(dt, uplo):
    for n in (1, 5, 8, 13, 16, 33, 40, 64):
        if not runnable("tiny", dt, n, uplo):
            continue
        a = syn.spd_matrices(n, 77, dt, seed=n)
        syn.plant_failures(a, seed=n, every=9)
        for fill in (syn.nan_value(dt), syn.sentinel(dt)):
            check_potrf(a, uplo, family="tiny", padded=True, fill=fill, label="poison")


# ---------------------------------------------------------------- LDS family
@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("uplo", UPLOS)
def test_lds_orders(dt, uplo):
    """Every order from 1 to 40, then a ragged sample up to the family's top order."""
    top = max(n for n in range(1, 200) if runnable("lds", dt, n, uplo))
    assert top >= 64
    orders = list(range(1, 41)) + [47, 48, 49, 63, 64, 65, 77, 95, 96, top]
    for n in sorted(set(k for k in orders if k <= top)):
        a = syn.spd_matrices(n, 37, dt, seed=30 * n + (uplo == "U"))
        want = syn.plant_failures(a, seed=n, every=5)
        check_potrf(a, uplo, family="lds", expect_info=want, label="lds-orders")


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("uplo", UPLOS)
def test_lds_poison_and_padding(dt, uplo):
    for n in (3, 33, 64):
        a = syn.spd_matrices(n, 23, dt, seed=n)
        syn.plant_failures(a, seed=n, every=4)
        for fill in (syn.nan_value(dt), syn.sentinel(dt)):
            check_potrf(a, uplo, family="lds", padded=True, fill=fill, label="lds-poison")


@pytest.mark.parametrize("dt", ["f32", "c64"])
def test_lds_packed_batch_is_independent(dt):
    """16384 identical items plus a ragged tail (several workgroups resident per
    compute unit) give the solo result bit for bit; compared on the device."""
    import torch
    import dense_linear_algebra_potrf_amd as bl
    n = 50
    one = torch.from_numpy(syn.to_colmajor(syn.spd_matrices(n, 1, dt, seed=5))).cuda()
    solo = one.clone()
    bl.potrf(solo, "U", n=n, batch=1, family="lds")
    batch = 16384 + 3
    announce("lds saturating", dt, n, batch)
    many = one.repeat(batch)
    info = bl.potrf(many, "U", n=n, batch=batch, family="lds")
    torch.cuda.synchronize()
    assert int((info != 0).sum()) == 0
    iv = torch.int64 if many.element_size() >= 8 else torch.int32
    assert torch.equal(many.view(iv).view(batch, -1), solo.view(iv).view(1, -1).expand(batch, -1))


@pytest.mark.parametrize("planted", [False, True])
def test_config_cfloat_upper_n64_b16384(planted):
    a = syn.spd_matrices(64, 16384, "c64", seed=1004)
    want = syn.plant_failures(a, seed=1004, every=64) if planted else np.zeros(16384, np.int32)
    check_potrf(a, "U", expect_info=want, label="config c64 U n=64 b16384")


def test_config_cfloat_upper_n64_b16384_lds_route():
    a = syn.spd_matrices(64, 16384, "c64", seed=1004)
    want = syn.plant_failures(a, seed=1004, every=64)
    check_potrf(a, "U", family="lds", expect_info=want, label="config c64 U n=64 via lds")


def test_config_fp32_n33_b16384_lds_route():
    a = syn.spd_matrices(33, 16384, "f32", seed=1022)
    want = syn.plant_failures(a, seed=1022, every=64)
    check_potrf(a, "L", family="lds", expect_info=want, label="config n=33 via lds")


# ---------------------------------------------------------------- info semantics
@pytest.mark.parametrize("family", ["tiny", "lds"])
@pytest.mark.parametrize("dt", DTS)
def test_info_first_failure_nan_and_stale_pivot(family, dt):
    n = 12
    if not runnable(family, dt, n):
        pytest.skip("family does not serve this order")
    a = syn.spd_matrices(n, 6, dt, seed=9)
    a[0, 3, 3] *= -1
    a[0, 9, 9] *= -1                      # two plants: the first wins
    a[1, 0, 0] = syn.nan_value(dt)        # NaN pivot
    a[2, 11, 11] = 0
    a[2, 5, 5] *= -1
    a[3, n - 1, n - 1] = -a[3, n - 1, n - 1]   # last column
    stale = np.eye(n)
    stale[:3, :3] = [[1, .75, .75], [.75, 1, -.75], [.75, -.75, 1]]
    a[4] = stale.astype(a.dtype)          # unit diagonal, only the Schur pivot fails
    for uplo in UPLOS:
        _, _, info = check_potrf(a, uplo, family=family, label="info")
        assert list(info) == [4, 1, 6, n, 3, 0]


@pytest.mark.parametrize("dt", DTS)
def test_null_info_is_allowed(dt):
    n = 8
    a = syn.spd_matrices(n, 40, dt, seed=3)
    buf = syn.to_colmajor(a)
    out, _ = gpu_potrf(buf, "L", n, 40, n, n * n, with_info=False)
    with_info, info = gpu_potrf(buf, "L", n, 40, n, n * n)
    assert (info == 0).all() and bits_equal(out, with_info)


# ---------------------------------------------------------------- packing invariants
@pytest.mark.parametrize("dt", ["f32", "c64", "f64"])
@pytest.mark.parametrize("n", [5, 8, 17, 32])
def test_packed_batch_is_independent_and_saturating_batch_is_uniform(dt, n):
    if not runnable("tiny", dt, n):
        pytest.skip("order not served by tiny")
    one = syn.spd_matrices(n, 1, dt, seed=21)
    solo = syn.to_colmajor(one)
    solo_out, solo_info = gpu_potrf(solo, "L", n, 1, n, n * n, family="tiny")
    batch = 16384 + 3                     # saturating, with a ragged tail
    many = np.repeat(one, batch, axis=0)
    announce("saturating", dt, n, batch)
    out, info = gpu_potrf(syn.to_colmajor(many), "L", n, batch, n, n * n, family="tiny")
    assert (info == 0).all() and solo_info[0] == 0
    res = out.reshape(batch, n * n)
    assert bits_equal(res, np.broadcast_to(solo_out.reshape(1, n * n), res.shape))


@pytest.mark.parametrize("dt", DTS)
def test_upper_equals_conjugate_transpose_of_lower(dt):
    n = 16 if dt == "c128" else 24
    if not runnable("tiny", dt, n):
        pytest.skip("order not served by tiny")
    a = syn.spd_matrices(n, 50, dt, seed=31)
    lo, _ = gpu_potrf(syn.to_colmajor(a), "L", n, 50, n, n * n)
    up, _ = gpu_potrf(syn.to_colmajor(a), "U", n, 50, n, n * n)
    lo = syn.from_colmajor(lo, n, n, 50)
    up = syn.from_colmajor(up, n, n, 50)
    assert np.array_equal(np.triu(up), np.triu(np.conj(np.swapaxes(np.tril(lo), 1, 2))))


# ---------------------------------------------------------------- the workload configurations
def test_config_fp32_n8_b1024_planted():
    a = syn.spd_matrices(8, 1024, "f32", seed=1001)
    want = syn.plant_failures(a, seed=1001, every=64)
    assert (want > 0).sum() == 16
    check_potrf(a, "L", expect_info=want, label="config n=8 b1024")


@pytest.mark.parametrize("planted", [False, True])
def test_config_fp32_n17_b32768(planted):
    a = syn.spd_matrices(17, 32768, "f32", seed=1021)
    want = syn.plant_failures(a, seed=1021, every=64) if planted else np.zeros(32768, np.int32)
    check_potrf(a, "L", expect_info=want, label="config n=17 b32768")


@pytest.mark.parametrize("planted", [False, True])
def test_config_fp32_n33_b16384(planted):
    a = syn.spd_matrices(33, 16384, "f32", seed=1022)
    want = syn.plant_failures(a, seed=1022, every=64) if planted else np.zeros(16384, np.int32)
    check_potrf(a, "L", expect_info=want, label="config n=33 b16384")


def test_config_fp32_n8_saturating_planted():
    batch = 1 << 20
    a = syn.spd_matrices(8, batch, "f32", seed=1011, chunk=4096)
    want = syn.plant_failures(a, seed=1011, every=64)
    check_potrf(a, "L", expect_info=want, label="n=8 b2^20")
