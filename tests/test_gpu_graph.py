"""The library's calls inside a captured HIP graph: one call per family is
captured once and replayed several times, each replay on a fresh copy of the
input made eagerly between replays, and every replay must give the eager
result bit for bit (the kernels are deterministic).  The bench times its
launches this way."""
from __future__ import annotations

import numpy as np
import pytest

import synthetic as syn
from tests._gpu import announce, torch_dtype

pytestmark = pytest.mark.gpu

CASES = [("f32", "L", 33, 4096, "tiny"), ("c64", "U", 64, 512, "tiny"),
         ("f32", "L", 128, 2048, "tiny"), ("c64", "U", 160, 256, "tiny"),
         ("f32", "U", 48, 300, "lds"), ("f64", "L", 300, 40, "blocked"),
         # the folded windows: 48 rows (odd batch), 128 rows (one matrix per
         # wavefront), 32 rows (four), 34 rows (three), 56 rows
         ("f64", "L", 40, 1001, "tiny"), ("f32", "U", 112, 513, "tiny"),
         ("c128", "L", 24, 999, "tiny"), ("f32", "L", 34, 3001, "tiny"),
         ("c64", "L", 52, 777, "tiny")]


@pytest.mark.parametrize("dt,uplo,n,batch,family", CASES)
def test_graph_replays_match_eager(dt, uplo, n, batch, family):
    import torch
    import dense_linear_algebra_potrf_amd as bl
    announce("graph", dt, uplo, f"n={n}", f"batch={batch}", family)
    a = syn.spd_matrices(n, batch, dt, seed=n + batch)
    syn.plant_failures(a, seed=n, every=9)
    src = torch.from_numpy(syn.to_colmajor(a)).cuda()
    eager = src.clone()
    info_e = bl.potrf(eager, uplo, n=n, batch=batch, family=family)
    torch.cuda.synchronize()
    work = src.clone()
    info = torch.zeros(batch, dtype=torch.int32, device="cuda")
    bl.potrf(work, uplo, info, n=n, batch=batch, family=family)   # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bl.potrf(work, uplo, info, n=n, batch=batch, family=family)
    torch.cuda.synchronize()
    for rep in range(3):
        work.copy_(src)
        info.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(info, info_e), f"replay {rep}: info differs"
        assert np.array_equal(work.cpu().numpy().view(np.uint8), eager.cpu().numpy().view(np.uint8)), \
            f"replay {rep}: factor differs"
