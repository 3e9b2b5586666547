"""Batches holding more than 2^31 elements, for every family.

Index arithmetic that silently wraps at 2^31 elements (32-bit element offsets)
is a known failure of batched kernels (the perf_level3 page, section
"Level-3: scratch expansions and their ceilings").  Each case replicates one
matrix past that point and checks, on the device, that every copy gives the
solo result bit for bit and that info is 0 everywhere, including the last
item, which lies beyond 2^31 elements from the base.
"""
from __future__ import annotations

import numpy as np
import pytest

import synthetic as syn
from tests._gpu import announce

pytestmark = pytest.mark.gpu

TWO31 = 1 << 31


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
    return t.view(torch.int64) if t.element_size() >= 8 or t.is_complex() else t.view(torch.int32)


def _replicas(buf: np.ndarray, batch: int):
    import torch
    return torch.from_numpy(buf).cuda().repeat(batch)


# (dtype, uplo, n, family); the batch is the smallest with more than 2^31 elements, plus a tail
CASES = [
    ("f32", "L", 8, "tiny"),       # packed window, 8 matrices per wavefront
    ("f32", "L", 33, "tiny"),      # per-row window, 4 matrices per wavefront
    ("c64", "U", 64, "tiny"),      # one matrix per wavefront, slab-transposed loads
    ("f32", "U", 80, "lds"),
    ("f64", "L", 512, "blocked"),
]


@pytest.mark.parametrize("dt,uplo,n,family", CASES)
def test_potrf_beyond_2_31_elements(dt, uplo, n, family):
    import torch
    import dense_linear_algebra_potrf_amd as bl
    batch = TWO31 // (n * n) + 3
    assert batch * n * n > TWO31
    announce("large", dt, uplo, f"n={n}", f"batch={batch}", family)
    one = syn.to_colmajor(syn.spd_matrices(n, 1, dt, seed=n))
    solo = _replicas(one, 1)
    bl.potrf(solo, uplo, n=n, batch=1, family=family)
    many = _replicas(one, batch)
    info = bl.potrf(many, uplo, n=n, batch=batch, family=family)
    torch.cuda.synchronize()
    assert int((info != 0).sum()) == 0
    assert torch.equal(_bits(many).view(batch, -1), _bits(solo).view(1, -1).expand(batch, -1))
    del many, info
    torch.cuda.empty_cache()


def test_posv_tiny_beyond_2_31_elements():
    import torch
    import dense_linear_algebra_potrf_amd as bl
    n, nrhs = 32, 4
    batch = TWO31 // (n * n) + 3
    announce("large posv", f"n={n}", f"nrhs={nrhs}", f"batch={batch}")
    a1 = syn.to_colmajor(syn.spd_matrices(n, 1, "f32", seed=3))
    b1 = syn.to_colmajor(syn.rhs(n, nrhs, 1, "f32", seed=3))
    sa, sb = _replicas(a1, 1), _replicas(b1, 1)
    bl.posv(sa, sb, "L", n=n, nrhs=nrhs, batch=1, family="posv_tiny")
    ma, mb = _replicas(a1, batch), _replicas(b1, batch)
    info = bl.posv(ma, mb, "L", n=n, nrhs=nrhs, batch=batch, family="posv_tiny")
    torch.cuda.synchronize()
    assert int((info != 0).sum()) == 0
    assert torch.equal(_bits(ma).view(batch, -1), _bits(sa).view(1, -1).expand(batch, -1))
    assert torch.equal(_bits(mb).view(batch, -1), _bits(sb).view(1, -1).expand(batch, -1))
    del ma, mb, info
    torch.cuda.empty_cache()


def test_tiny_batch_sliced_over_several_launches():
    """Order 2 packs 16 matrices per wavefront; 2^28 + 5 matrices need more than
    2^24 workgroups, so the batch runs as two launches over consecutive slices.
    Every item, on both sides of the slice boundary, must equal the solo result."""
    import torch
    import dense_linear_algebra_potrf_amd as bl
    n, batch = 2, (1 << 28) + 5
    assert bl.route("f32", "L", n, batch, family="tiny")["grid"] == 1 << 24
    announce("sliced", f"n={n}", f"batch={batch}")
    one = syn.to_colmajor(syn.spd_matrices(n, 1, "f32", seed=2))
    solo = _replicas(one, 1)
    bl.potrf(solo, "L", n=n, batch=1, family="tiny")
    many = _replicas(one, batch)
    info = bl.potrf(many, "L", n=n, batch=batch, family="tiny")
    torch.cuda.synchronize()
    assert int((info != 0).sum()) == 0
    assert torch.equal(_bits(many).view(batch, -1), _bits(solo).view(1, -1).expand(batch, -1))
    del many, info
    torch.cuda.empty_cache()
