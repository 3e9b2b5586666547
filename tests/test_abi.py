"""The C ABI without a GPU: the library loads, exports every declared symbol,
validates arguments in the documented order before touching the GPU, and its
host-only route query agrees with the families' tables.  Also the build gate:
no kernel uses scratch memory."""
from __future__ import annotations

import ctypes
import json
import os
import re
import subprocess
import sys

import pytest

import dense_linear_algebra_potrf_amd as bl
from dense_linear_algebra_potrf_amd import build as blbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "batchlas.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bl.LIB_PATH):
        blbuild.build(incremental=True, verbose=False)
    return bl.load_library()


def declared_functions() -> set[str]:
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(batchlas_[a-z_]+)\s*\(", text))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert names == set(bl.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", bl.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (batchlas_\w+)", out))
    assert names <= exported


def test_version_and_status_strings(lib):
    assert lib.batchlas_version() >= 100
    for code in range(6):
        assert lib.batchlas_status_string(code)
    assert lib.batchlas_status_string(99) == b"unknown status"


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


@pytest.mark.parametrize("args,status,msg", [
    (dict(n=0), 1, "n must be"),
    (dict(n=-3), 1, "n must be"),
    (dict(batch=0), 1, "batch must be"),
    (dict(lda=7), 1, "lda must be"),
    (dict(stride=63), 1, "strideA"),
    (dict(A=None), 2, "A is NULL"),
    (dict(dt=7), 1, "dtype"),
    (dict(uplo=2), 1, "uplo"),
    (dict(stride=1 << 62, batch=1 << 10), 1, "overflows"),
    # order: n is checked before lda, lda before the pointer
    (dict(n=0, lda=0, A=None), 1, "n must be"),
    (dict(lda=1, A=None), 1, "lda must be"),
])
def test_potrf_validation(lib, args, status, msg):
    a = dict(dt=0, uplo=0, n=8, A=FAKE, lda=8, stride=64, batch=4)
    a.update(args)
    st = lib.batchlas_potrf(a["dt"], a["uplo"], a["n"], a["A"], a["lda"], a["stride"], a["batch"],
                            None, None)
    assert st == status
    assert msg in lib.batchlas_last_error().decode()


@pytest.mark.parametrize("args,status,msg", [
    (dict(nrhs=0), 1, "nrhs must be"),
    (dict(ldb=3), 1, "ldb must be"),
    (dict(strideB=15), 1, "strideB"),
    (dict(B=None), 2, "B is NULL"),
])
def test_posv_validation(lib, args, status, msg):
    a = dict(dt=0, uplo=0, n=8, nrhs=2, A=FAKE, lda=8, strideA=64, B=FAKE, ldb=8, strideB=16,
             batch=4)
    a.update(args)
    st = lib.batchlas_posv(a["dt"], a["uplo"], a["n"], a["nrhs"], a["A"], a["lda"], a["strideA"],
                           a["B"], a["ldb"], a["strideB"], a["batch"], None, None)
    assert st == status
    assert msg in lib.batchlas_last_error().decode()


def test_unknown_family_is_rejected(lib):
    st = lib.batchlas_potrf_family(42, 0, 0, 8, FAKE, 8, 64, 4, None, None)
    assert st == 1


def test_route_tiny_geometry_invariants(lib):
    for dt in ("f32", "f64", "c64", "c128"):
        for n in range(1, 34):
            try:
                r = bl.route(dt, "L", n, 1000, family="tiny")
            except bl.BatchlasError as e:
                assert e.status_name == "NOT_SUPPORTED"
                continue
            P, R, G = r["lanes_per_matrix"], r["rows_per_lane"], r["matrices_per_wave"]
            if P > 64:      # the wide window: one matrix over several wavefronts
                assert dt == "c128" and n == 33 and G == 1 and P == r["block_threads"]
                continue
            # up to 64 // P matrices per wavefront (fewer where measured faster)
            assert P * R >= n and 1 <= G <= 64 // P
            assert r["grid"] * G * (r["block_threads"] // 64) >= 1000
            assert r["family"] == "tiny"


def test_route_auto_picks_by_size(lib):
    assert bl.route("f32", "L", 8, 1024)["family"] == "tiny"
    assert bl.route("f32", "L", 17, 32768)["family"] == "tiny"
    assert bl.route("c128", "U", 16, 64)["family"] == "tiny"
    # the tiny range (with its wide window) ends at the measured cut of each type;
    # the blocked family takes the orders above it
    for dt, top in (("f32", 192), ("f64", 128), ("c64", 192), ("c128", 192)):
        assert bl.route(dt, "L", top, 16384)["family"] == "tiny"
        assert bl.route(dt, "U", top + 1, 16384)["family"] == "blocked", dt
    for dt, n in (("c64", 65), ("c64", 96), ("c128", 33), ("c128", 64), ("c128", 65)):
        assert bl.route(dt, "U", n, 16384)["family"] == "tiny", (dt, n)
    assert bl.route("c64", "L", 512, 64)["family"] == "blocked"
    assert bl.route("c128", "L", 256, 64)["family"] == "blocked"
    # a stride beyond the tiny family's 31-bit offsets goes to the LDS family up
    # to its cut (64 for cdouble), then to the blocked family
    big = (1 << 31) // 16 + 1
    assert bl.route("c128", "L", 40, 4, stride=big)["family"] == "lds"
    assert bl.route("c128", "L", 65, 4, stride=big)["family"] == "blocked"


def test_posv_auto_routes_beyond_the_window_to_split(lib):
    assert bl.route("f32", "L", 32, 64, nrhs=4)["family"] == "posv_tiny"
    assert bl.route("f32", "L", 32, 64, nrhs=5)["family"] == "posv_split"
    assert bl.route("f64", "U", 200, 64, nrhs=1)["family"] == "posv_split"
    assert bl.route("c64", "U", 512, 64, nrhs=3)["family"] == "posv_split"
    with pytest.raises(bl.BatchlasError) as e:
        bl.route("c128", "L", 600, 4, nrhs=1)      # no potrf family for this shape
    assert e.value.status_name == "NOT_SUPPORTED"


def test_route_beyond_every_family_is_not_supported(lib):
    for dt, n in (("c128", 513), ("c64", 513), ("f64", 513), ("f32", 1000)):
        with pytest.raises(bl.BatchlasError) as e:
            bl.route(dt, "L", n, 4)
        assert e.value.status_name == "NOT_SUPPORTED"


def _route_in_subprocess(env_extra: dict, code: str) -> str:
    env = dict(os.environ, **env_extra)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                         cwd=ROOT)
    return out.stdout.strip() + out.stderr.strip()


def test_environment_pin_is_read_and_a_bad_pin_is_an_error(lib):
    code = ("import dense_linear_algebra_potrf_amd as bl\n"
            "try:\n    print(bl.route('f32','L',8,64)['family'])\n"
            "except bl.BatchlasError as e:\n    print('ERR', e)\n")
    assert _route_in_subprocess({"BATCHLAS_POTRF_ROUTE": "tiny"}, code).endswith("tiny")
    res = _route_in_subprocess({"BATCHLAS_POTRF_ROUTE": "native:tiny"}, code)
    assert "ERR INVALID_VALUE" in res and "does not parse" in res


# Kernels allowed a bounded spill, with the reason.  The fp64 blocked kernels
# keep two 64-column superblocks (128 registers) in accumulators from the GEMM
# through the two-stage solve; the compiler spills about 80 bytes per lane at
# the GEMM loops' boundaries (none inside them).  That schedule measured 3%
# faster (fp64 n=512, b1024) than keeping one superblock with no spill.
# Dynamic register indexing would show as far more scratch than this.
SPILL_ALLOWANCE = {"potrf_blocked_kernelIdLb": 96}


def test_no_kernel_uses_scratch(lib):
    res = json.load(open(blbuild.RESOURCES))
    assert res, "resource report is empty"

    def allowed(name, nbytes):
        return any(key in name and nbytes <= bound for key, bound in SPILL_ALLOWANCE.items())

    bad = {k: v for k, v in res.items()
           if v.get("scratch_bytes", 0) != 0 and not allowed(k, v["scratch_bytes"])}
    assert not bad, f"kernels with scratch (dynamic register indexing?): {sorted(bad)}"


def test_counter_digest_follows_the_family_sources(tmp_path, monkeypatch):
    """A committed counter run stays attached while its kernel family's sources
    are unchanged: a change elsewhere (another family) keeps the digest, a change
    in the family's own file or a shared header moves it."""
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    csrc = tmp_path / "dense_linear_algebra_potrf_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in ("tiny_impl.hpp", "blocked_impl.hpp", "common.hpp", "api.cpp"):
        (csrc / name).write_text(name)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    tiny0, all0 = bench.source_digest("tiny"), bench.source_digest()
    (csrc / "blocked_impl.hpp").write_text("changed")
    assert bench.source_digest("tiny") == tiny0
    assert bench.source_digest() != all0
    (csrc / "tiny_impl.hpp").write_text("changed")
    tiny1 = bench.source_digest("tiny")
    assert tiny1 != tiny0
    (csrc / "common.hpp").write_text("changed")
    assert bench.source_digest("tiny") != tiny1


def test_route_wide_window_geometry(lib):
    """fp32 orders 65..192: one matrix per workgroup.  Up to 128, two
    wavefronts holding a row per lane; above, one wavefront per tile of 64 rows
    x 32 columns below the diagonal.  At most 2^20 workgroups."""
    def tile_waves(n):
        w, rb = 0, 0
        while 64 * rb < n:
            w += -(-min(64 * (rb + 1), n) // 32)
            rb += 1
        return w
    assert (tile_waves(129), tile_waves(160), tile_waves(192)) == (11, 11, 12)
    for uplo in ("L", "U"):
        for n in (65, 96, 97, 128, 129, 160, 192):
            if uplo == "U" and 97 <= n <= 128:
                continue                  # the folded window (below)
            threads = 128 if n <= 128 else 64 * tile_waves(n)
            for batch in (1, 1000, (1 << 20) + 5):
                r = bl.route("f32", uplo, n, batch, family="tiny")
                assert r["family"] == "tiny"
                assert r["block_threads"] == threads <= 768
                assert (r["lanes_per_matrix"], r["rows_per_lane"], r["matrices_per_wave"]) == \
                    (threads, 1, 1)
                assert r["panel"] == (0 if n <= 128 else 32)
                assert r["grid"] == min(batch, 1 << 20)
                tile = 128 * 33 * 4 if uplo == "U" and n <= 128 else 0   # the rows layout's slab tile
                assert r["lds_bytes"] == 2 * (192 + 4) * 4 + tile
    # fp64 takes the tiles layout at every order of the window
    for n in (65, 128, 192):
        r = bl.route("f64", "U", n, 1000, family="tiny")
        assert r["block_threads"] == 64 * tile_waves(n) and r["panel"] == 32
        assert r["lds_bytes"] == 2 * (192 + 4) * 8
    for n in (65, 192):
        r = bl.route("c64", "L", n, 1000, family="tiny")
        assert r["block_threads"] == 64 * tile_waves(n) and r["lds_bytes"] == 2 * (192 + 4) * 8
    for n in (33, 64, 65, 192):
        r = bl.route("c128", "L", n, 1000, family="tiny")
        assert r["block_threads"] == 64 * tile_waves(n) and r["lds_bytes"] == 2 * (192 + 4) * 16
    for dt in ("f32", "f64", "c64", "c128"):
        with pytest.raises(bl.BatchlasError) as e:
            bl.route(dt, "L", 193, 64, family="tiny")
        assert e.value.status_name == "NOT_SUPPORTED"
    # the layout bound: every offset of one matrix within 2^31 bytes
    with pytest.raises(bl.BatchlasError):
        bl.route("f32", "L", 100, 4, family="tiny", lda=(1 << 29) // 100 + 1)


def test_route_folded_window_geometry(lib):
    """fp64 and cfloat orders 33..64: two matrices per wavefront, 32 lanes x 2
    rows each (rows q and 63 - q), one wavefront per workgroup, a grid of pairs
    capped at 2^19; Upper adds the slab tile to the pivot buffers.  A stride
    whose pair of matrices leaves the 31-bit offsets falls back to the
    one-wavefront window; fp32 keeps that window at these orders."""
    for dt, es in (("f64", 8), ("c64", 8)):
        for uplo in ("L", "U"):
            for n in (33, 40, 48, 49, 56, 57, 63, 64):
                for batch in (1, 2, 1001, (1 << 20) + 5):
                    r = bl.route(dt, uplo, n, batch)
                    assert r["family"] == "tiny", (dt, n)
                    # up to 48: the 48-row window (24 lanes of a 32-lane group);
                    # cfloat 49..56 the 56-row window (28 lanes)
                    half = 24 if n <= 48 else 28 if dt == "c64" and n <= 56 else 32
                    assert (r["lanes_per_matrix"], r["rows_per_lane"], r["matrices_per_wave"]) == \
                        (half, 2, 2)
                    assert r["block_threads"] == 64
                    assert r["grid"] == min((batch + 1) // 2, 1 << 19)
                    sr = 128 // es if half != 28 else 64 // es      # slab rows: a line, or half
                    lds = 2 * 2 * 68 * es + (2 * 64 * (sr + 1) * es if uplo == "U" else 0)
                    assert r["lds_bytes"] == lds
        top = (1 << 31) // es // 2                  # largest stride whose pair fits, with margin
        assert bl.route(dt, "L", 40, 4, stride=top - 1)["lanes_per_matrix"] == 24
        r = bl.route(dt, "L", 40, 4, stride=top + 64)
        assert r["family"] == "tiny" and r["lanes_per_matrix"] == 64 and r["matrices_per_wave"] == 1
    # fp64 25..32: the 32-row window (16 lanes, four matrices per wavefront)
    for uplo in ("L", "U"):
        for n in (25, 28, 32):
            r = bl.route("f64", uplo, n, 1001)
            assert (r["lanes_per_matrix"], r["rows_per_lane"], r["matrices_per_wave"]) == (16, 2, 4)
            assert r["grid"] == 251
            assert r["lds_bytes"] == 2 * 4 * 36 * 8 + (4 * 32 * 17 * 8 if uplo == "U" else 0)
    assert bl.route("f64", "L", 24, 1001)["lanes_per_matrix"] == 8
    for n in (25, 32):                    # fp32: Upper only (Lower keeps its 16 x 2 window)
        r = bl.route("f32", "U", n, 1001)
        assert (r["lanes_per_matrix"], r["rows_per_lane"], r["matrices_per_wave"]) == (16, 2, 4)
        assert r["lds_bytes"] == 2 * 4 * 36 * 4 + 4 * 32 * 17 * 4
        assert bl.route("f32", "L", n, 1001)["lanes_per_matrix"] == 16
        assert bl.route("f32", "L", n, 1001)["matrices_per_wave"] == 4
    assert bl.route("c64", "L", 32, 1001)["lanes_per_matrix"] == 8
    # cdouble Lower 17..32: the 32-row window (16 lanes, four matrices per
    # wavefront); Upper keeps 32 x 1
    for n in (17, 24, 32):
        r = bl.route("c128", "L", n, 1001)
        assert (r["lanes_per_matrix"], r["rows_per_lane"], r["matrices_per_wave"]) == (16, 2, 4)
        assert r["grid"] == 251 and r["lds_bytes"] == 2 * 4 * 36 * 16
        assert bl.route("c128", "U", n, 1001)["lanes_per_matrix"] == 32
    # the neighbours: order 32 in a smaller register window, 65 in the wide window
    assert bl.route("f64", "L", 32, 1000)["matrices_per_wave"] > 2
    assert bl.route("f64", "L", 65, 1000)["block_threads"] > 64
    # fp32: the folded window for Lower at 34..64 (Upper keeps 64 x 1; order 33
    # has its own window) and for Upper at 97..128, one matrix per wavefront
    # (Lower keeps the rows layout)
    for n in (35, 48, 49, 64):
        r = bl.route("f32", "L", n, 1001)
        assert (r["lanes_per_matrix"], r["rows_per_lane"], r["matrices_per_wave"]) == \
            (24 if n <= 48 else 32, 2, 2)
        assert r["grid"] == 501 and r["lds_bytes"] == 2 * 2 * 68 * 4
        assert bl.route("f32", "U", n, 1000)["lanes_per_matrix"] == (24 if n <= 48 else 64)
    r = bl.route("f32", "L", 34, 1000)    # the 34-row window: 17 lanes, three matrices per wavefront
    assert (r["lanes_per_matrix"], r["rows_per_lane"], r["matrices_per_wave"]) == (17, 2, 3)
    assert r["grid"] == 334 and r["lds_bytes"] == 2 * 4 * 38 * 4
    for uplo in ("L", "U"):               # order 33 keeps its 11 x 3 window
        assert bl.route("f32", uplo, 33, 1000)["lanes_per_matrix"] == 11
    for n in (97, 112, 128):
        for batch in (1, 1000, (1 << 20) + 5):
            r = bl.route("f32", "U", n, batch)
            assert r["family"] == "tiny" and r["block_threads"] == 64
            assert (r["lanes_per_matrix"], r["rows_per_lane"], r["matrices_per_wave"]) == (64, 2, 1)
            assert r["grid"] == min(batch, 1 << 19)
            assert r["lds_bytes"] == (2 * 132 + 128 * 33) * 4
        assert bl.route("f32", "L", n, 1000)["block_threads"] == 128
    assert bl.route("f32", "U", 96, 1000)["block_threads"] == 128


def test_tiny_grid_is_capped_for_huge_batches(lib):
    """A batch of 2^30 matrices of order 4 (16 per wavefront) would need 2^26
    one-wavefront workgroups; the tiny family launches it in slices of at most
    2^24 workgroups, and the route reports the first slice's grid."""
    r = bl.route("f32", "L", 4, 1 << 30, family="tiny")
    assert r["grid"] == 1 << 24
    assert r["grid"] * r["matrices_per_wave"] * (r["block_threads"] // 64) < (1 << 30)
    small = bl.route("f32", "L", 4, 1000, family="tiny")
    assert small["grid"] * small["matrices_per_wave"] >= 1000
