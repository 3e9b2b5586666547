"""Benchmark for batched potrf / posv on one MI355X.

`python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--no-secondary]`

A step is one call of the library on one batch of synthetic input that is
already resident in HBM.  Since potrf works in place, every step gets its own
freshly prepared copy of the input (copies are made before the timed region,
and together they exceed the 256 MB MALL, so each step starts from HBM).
W untimed steps, then exactly K timed steps bracketed by synchronisation; rank
0 prints ONE JSON line.

The headline workload is fp32 Lower potrf, n = 33, batch 16384 (matrices/s,
HBM GB/s and its fraction of the 8 TB/s peak).  Secondary lines cover the
other workloads (n = 8, 17; posv n = 32 nrhs = 4; complex-float Upper n = 64;
fp64 n = 512 in GFLOP/s against the 78.6 TFLOP/s FP64 peak).

The roofline of the dominant kernel uses the algorithmic bytes (or flops) of
one launch divided by the launch's average duration, measured with HIP events
on the stream the kernel runs on.  The CPU baseline times the oracle on the
host cores on a bounded sample of the same workload.

Modes for profiling: --mode copy runs a plain device copy of known size (the
calibration for FETCH_SIZE / WRITE_SIZE counters).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from dense_linear_algebra_potrf_amd import metrics  # noqa: E402  (host-side byte and flop models)

METRIC = "batched potrf matrices/s + GB/s (% HBM peak) fp32 n=33; GFLOP/s fp64 n=512"

CONFIGS = {
    "potrf_f32_L_n8_b1024": dict(op="potrf", dt="f32", uplo="L", n=8, batch=1024, seed=1001, plant=64),
    "potrf_f32_L_n8_b1048576": dict(op="potrf", dt="f32", uplo="L", n=8, batch=1 << 20, seed=1011, plant=64),
    "potrf_f32_L_n17_b32768": dict(op="potrf", dt="f32", uplo="L", n=17, batch=32768, seed=1021),
    "potrf_f32_L_n33_b16384": dict(op="potrf", dt="f32", uplo="L", n=33, batch=16384, seed=1022),
    "posv_f32_L_n32_r4_b16384": dict(op="posv", dt="f32", uplo="L", n=32, nrhs=4, batch=16384, seed=1003),
    "potrf_c64_U_n64_b16384": dict(op="potrf", dt="c64", uplo="U", n=64, batch=16384, seed=1004),
    "potrf_f64_L_n512_b1024": dict(op="potrf", dt="f64", uplo="L", n=512, batch=1024, seed=1005),
    # beyond the listed workloads: mid orders (the tiny family's wide window, one
    # per layout) and the complex blocked path at the largest order
    "potrf_f32_L_n128_b8192": dict(op="potrf", dt="f32", uplo="L", n=128, batch=8192, seed=1006),
    "potrf_f64_L_n96_b8192": dict(op="potrf", dt="f64", uplo="L", n=96, batch=8192, seed=1008),
    "potrf_c64_L_n128_b4096": dict(op="potrf", dt="c64", uplo="L", n=128, batch=4096, seed=1009),
    "potrf_c64_L_n512_b1024": dict(op="potrf", dt="c64", uplo="L", n=512, batch=1024, seed=1007),
}
PRIMARY = "potrf_f32_L_n33_b16384"
SECONDARY = ["potrf_f32_L_n17_b32768", "potrf_f32_L_n8_b1024", "potrf_f32_L_n8_b1048576",
             "posv_f32_L_n32_r4_b16384", "potrf_c64_U_n64_b16384", "potrf_f64_L_n512_b1024",
             "potrf_f32_L_n128_b8192", "potrf_f64_L_n96_b8192", "potrf_c64_L_n128_b4096",
             "potrf_c64_L_n512_b1024"]


def describe(cfg: dict) -> str:
    kind = {"f32": "s", "f64": "d", "c64": "c", "c128": "z"}[cfg["dt"]] + cfg["op"]
    s = f"{kind} {'lower' if cfg['uplo'] == 'L' else 'upper'} n={cfg['n']}"
    if cfg["op"] == "posv":
        s += f" nrhs={cfg['nrhs']}"
    return s + f" batch={cfg['batch']}, column-major lda=n stride=n*n, A = G G^H/n + I (seed {cfg['seed']})"


# The sources each route's kernels are built from: a counter run stays valid
# while these are unchanged (with no family given, every source counts).
FAMILY_SOURCES = {
    "tiny": ("tiny", "wide", "fold"),
    "posv_tiny": ("tiny", "posv"),
    "lds": ("lds",),
    "blocked": ("blocked",),
    "posv_split": ("tiny", "wide", "fold", "lds", "blocked", "potrs"),
}
COMMON_SOURCES = ("common.hpp", "families.hpp", "api.cpp")


def source_digest(family: str | None = None) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_linear_algebra_potrf_amd", "csrc")
    prefixes = FAMILY_SOURCES.get(family) if family else None
    for name in sorted(os.listdir(csrc)):
        if prefixes is not None and not (name.startswith(prefixes) or name in COMMON_SOURCES):
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def make_input(cfg: dict):
    """Host buffers (column-major) for a workload."""
    import numpy as np
    import synthetic as syn
    a = syn.spd_matrices(cfg["n"], cfg["batch"], cfg["dt"], cfg["seed"],
                         chunk=64 if cfg["n"] >= 128 else 4096)
    if cfg.get("plant"):
        syn.plant_failures(a, cfg["seed"], every=cfg["plant"])
    abuf = syn.to_colmajor(a)
    del a
    bbuf = None
    if cfg["op"] == "posv":
        bbuf = syn.to_colmajor(syn.rhs(cfg["n"], cfg["nrhs"], cfg["batch"], cfg["dt"], cfg["seed"]))
    return abuf, bbuf


def bench_config(name: str, steps: int, warmup: int, use_graph: bool = True) -> dict:
    import torch
    import dense_linear_algebra_potrf_amd as bl
    from dense_linear_algebra_potrf_amd import metrics

    cfg = CONFIGS[name]
    abuf, bbuf = make_input(cfg)
    dev = torch.device("cuda:0")
    pa = torch.from_numpy(abuf).to(dev)
    pb = torch.from_numpy(bbuf).to(dev) if bbuf is not None else None
    n, batch, dt, uplo = cfg["n"], cfg["batch"], cfg["dt"], cfg["uplo"]
    nrhs = cfg.get("nrhs", 0)
    # one fresh copy per step (potrf works in place); then a 1 GiB flush so that
    # the timed steps start from HBM, not from the 256 MB MALL or the L2s
    per_copy = pa.numel() * pa.element_size() + (pb.numel() * pb.element_size() if pb is not None else 0)
    if (steps + warmup) * per_copy > (96 << 30):
        raise SystemExit(f"{name}: {steps + warmup} copies of {per_copy >> 20} MiB do not fit")
    work_a = [pa.clone() for _ in range(steps + warmup)]
    work_b = [pb.clone() for _ in range(steps + warmup)] if pb is not None else None
    info = torch.empty(batch, dtype=torch.int32, device=dev)
    route = bl.route(dt, uplo, n, batch, nrhs=nrhs)
    stream = torch.cuda.current_stream()

    def launch(i):
        if cfg["op"] == "potrf":
            bl.potrf(work_a[i], uplo, info, n=n, batch=batch)
        else:
            bl.posv(work_a[i], work_b[i], uplo, info, n=n, nrhs=nrhs, batch=batch)

    for k in range(warmup):
        launch(k)
    torch.cuda.synchronize()
    # The K timed calls are captured into one HIP graph (capture records the
    # launches without running them) and replayed once: the kernels then run
    # back to back, where a Python loop of short kernels would leave the GPU
    # idle between launches.  Each call has its own input copy, so the single
    # replay factors K fresh batches.
    graph = None
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for k in range(steps):
                launch(warmup + k)
        torch.cuda.synchronize()
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    flush.fill_(7)
    del flush
    # Two events bracket the whole timed region on the launch stream: an event
    # between launches would itself open a gap of several microseconds.  Every
    # family is a single launch per call, so the region's time over K is the
    # average duration of the dominant kernel.
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for k in range(steps):
            launch(warmup + k)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [ev0.elapsed_time(ev1) / steps]
    del graph
    # correctness guard on the last step: info must be as planted
    info_h = info.cpu().numpy()
    if cfg.get("plant"):
        bad = int((info_h != 0).sum())
        expect = len(range(0, batch, cfg["plant"]))
        assert bad == expect, f"{name}: {bad} failed items, expected {expect}"
    else:
        assert (info_h == 0).all(), f"{name}: unexpected info"

    ms_step = wall * 1e3 / steps
    ms_kernel = kern_ms[0]
    if cfg["op"] == "potrf":
        byts = metrics.potrf_bytes(n, batch, dt, uplo)
        flops = metrics.potrf_flops(n, dt) * batch
    else:
        byts = metrics.posv_bytes(n, nrhs, batch, dt, uplo)
        flops = metrics.posv_flops(n, nrhs, dt) * batch
    peak_tf = metrics.PEAK_TFLOPS[dt]
    res = {
        "workload": describe(cfg),
        "family": route["family"],
        "geometry": {k: route[k] for k in ("lanes_per_matrix", "rows_per_lane", "matrices_per_wave",
                                           "block_threads", "panel", "grid")},
        "ms_per_step": ms_step,
        "ms_per_call_events": ms_kernel,
        "matrices_per_s": batch / (ms_step * 1e-3),
        "gflops": flops / (ms_step * 1e-3) / 1e9,
        "gbs": byts / (ms_step * 1e-3) / 1e9,
        "hbm_frac": byts / (ms_step * 1e-3) / 1e9 / metrics.HBM_PEAK_GBS,
        "flop_frac": flops / (ms_step * 1e-3) / 1e12 / peak_tf,
        "alg_bytes_per_call": byts,
        "alg_flops_per_call": flops,
    }
    # roofline of the dominant kernel (one launch per call for the single-launch
    # families): the matrix-core peak of the element type where the algorithmic
    # flops per algorithmic byte exceed that peak's ridge against 8 TB/s, HBM
    # otherwise
    ridge = peak_tf * 1e12 / (metrics.HBM_PEAK_GBS * 1e9)
    bound = "mfma" if flops / byts > ridge else "hbm"
    if bound == "hbm":
        ach = byts / (ms_kernel * 1e-3) / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": ach, "peak": metrics.HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": ach / metrics.HBM_PEAK_GBS,
                           "traffic": None}
    else:
        ach = flops / (ms_kernel * 1e-3) / 1e12
        res["roofline"] = {"bound": "mfma", "achieved": ach, "peak": peak_tf, "unit": "TFLOP/s",
                           "frac": ach / peak_tf, "traffic": None}
    del work_a, work_b, pa, pb
    torch.cuda.empty_cache()
    return res


def attach_traffic(name: str, res: dict) -> None:
    """HBM traffic per launch from committed counter runs, if the kernels are unchanged."""
    path = os.path.join(ROOT, "profiles", f"{name}.counters.json")
    if not os.path.exists(path):
        return
    rec = json.load(open(path))
    if rec.get("source_digest") != source_digest(res.get("family")):
        return
    res["roofline"]["traffic"] = rec.get("traffic_bytes")


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def host_threads() -> int:
    """Host threads the oracle may use: the process's CPU share, at most 16 (the
    host CPU share of one GPU on the benchmark machines)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _oracle_rate(name: str, threads: int, cpu_seconds: float) -> tuple[float, int, int, float]:
    """(matrices/s, matrices done, matrices per pass, wall s) of the oracle on a
    sample of the workload, run for about cpu_seconds of CPU time (wall x threads)."""
    import oracle
    cfg = CONFIGS[name]
    n = cfg["n"]
    budget_s = cpu_seconds / threads
    # one pass is about 0.2 s of single-thread work at ~1 GFLOP/s, a multiple of the threads
    per = max(threads, min(cfg["batch"], int(2e8 // max(1, n ** 3)) * threads))
    sample = dict(cfg, batch=per)
    abuf, bbuf = make_input(sample)
    done, t = 0, 0.0
    while t < budget_s:
        a = abuf.copy()
        b = bbuf.copy() if bbuf is not None else None
        t0 = time.perf_counter()
        if cfg["op"] == "potrf":
            oracle.potrf(a, cfg["uplo"], n, per, nthreads=threads)
        else:
            oracle.posv(a, b, cfg["uplo"], n, cfg["nrhs"], per, nthreads=threads)
        t += time.perf_counter() - t0
        done += per
    return done / t, done, per, t


def cpu_baseline(name: str, cpu_seconds: float = 16.0) -> dict:
    """The oracle (as it stands: unblocked column Cholesky, no FMA contraction)
    on the host, on a bounded sample of the same workload: about cpu_seconds of
    CPU time on all host threads, and a quarter of that on one thread."""
    cfg = CONFIGS[name]
    threads = host_threads()
    rate, done, per, wall = _oracle_rate(name, threads, cpu_seconds)
    rate1, done1, _, wall1 = _oracle_rate(name, 1, cpu_seconds / 4)
    flops = metrics.potrf_flops(cfg["n"], cfg["dt"]) if cfg["op"] == "potrf" else \
        metrics.posv_flops(cfg["n"], cfg["nrhs"], cfg["dt"])
    return {"value": rate, "unit": "matrices/s", "cores": threads, "kind": "oracle",
            "gflops": rate * flops / 1e9,
            "value_1thread": rate1, "gflops_1thread": rate1 * flops / 1e9,
            "cpu_model": cpu_model(),
            "sample": f"{done} matrices ({per} per pass) of: {describe(cfg)}; {wall:.2f} s wall "
                      f"on {threads} threads; one thread: {done1} matrices in {wall1:.2f} s"}


def copy_mode(mib: int, reps: int) -> None:
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "copy", "bytes_each_way": mib << 20, "reps": reps}))


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=PRIMARY, choices=sorted(CONFIGS))
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--mode", default="bench", choices=["bench", "copy"])
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the timed calls from Python instead of one graph replay")
    a = ap.parse_args(argv)

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the batched factorisation has no cross-GPU step, "
              "so only --gpus 1 is supported (a batch shards by slicing it across GPUs).",
              file=sys.stderr)
        return 2
    if a.mode == "copy":
        copy_mode(a.copy_mib, max(1, a.steps))
        return 0

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    import dense_linear_algebra_potrf_amd as bl
    bl.load_library()

    prim = bench_config(a.config, a.steps, a.warmup, use_graph=not a.no_graph)
    attach_traffic(a.config, prim)
    cfg = CONFIGS[a.config]
    out = {
        "metric": METRIC,
        "value": prim["matrices_per_s"],
        "unit": "matrices/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": prim["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dt"],
        "data": "synthetic",
        "config": {"workload": prim["workload"], "op": cfg["op"], "n": cfg["n"], "batch": cfg["batch"],
                   "uplo": cfg["uplo"], "family": prim["family"], "parallelism": "batch on 1 GPU"},
        "gbs": prim["gbs"],
        "hbm_frac": prim["hbm_frac"],
        "gflops": prim["gflops"],
        "roofline": prim["roofline"],
    }
    if not a.no_cpu:
        out["cpu_baseline"] = cpu_baseline(a.config)
    if not a.no_secondary:
        sec = {}
        for name in SECONDARY:
            if name == a.config:
                continue
            c = CONFIGS[name]
            try:
                bl.route(c["dt"], c["uplo"], c["n"], c["batch"], nrhs=c.get("nrhs", 0))
            except bl.BatchlasError as e:
                sec[name] = {"skipped": str(e)}
                continue
            r = bench_config(name, max(3, min(a.steps, 10)), max(1, min(a.warmup, 3)),
                             use_graph=not a.no_graph)
            attach_traffic(name, r)
            if not a.no_cpu:
                r["cpu_baseline"] = cpu_baseline(name, cpu_seconds=6.0)
            sec[name] = r
            print(f"[bench] {name}: {r['ms_per_step']:.4f} ms/step, {r['gbs']:.0f} GB/s, "
                  f"{r['gflops']:.0f} GFLOP/s", file=sys.stderr, flush=True)
        out["secondary"] = sec
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
