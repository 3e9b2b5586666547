"""Build the HIP library libbatchlas.so for gfx950 with hipcc.

Every source under csrc/ is compiled in parallel into _build/, then linked into
_lib/libbatchlas.so.  The compiler's per-kernel resource report (registers,
scratch, LDS, occupancy) is parsed into _lib/resource_usage.json; the test
suite gates on it (no kernel may use scratch memory).

Usage:  python -m dense_linear_algebra_potrf_amd.build [--incremental] [-j N]
"""
from __future__ import annotations

import argparse
import glob
import json
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libbatchlas.so")
RESOURCES = os.path.join(LIBDIR, "resource_usage.json")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 instructions off (their hand-written forms are avoided too)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _deps(src: str, seen: set | None = None) -> set:
    """The source and every local header it includes, transitively."""
    seen = set() if seen is None else seen
    if src in seen or not os.path.exists(src):
        return seen
    seen.add(src)
    for line in open(src, errors="replace"):
        m = re.match(r'\s*#\s*include\s+"([^"]+)"', line)
        if m:
            _deps(os.path.normpath(os.path.join(os.path.dirname(src), m.group(1))), seen)
    return seen


def _obj(src: str) -> str:
    return os.path.join(BUILD, os.path.basename(src) + ".o")


def _compile(src: str, incremental: bool) -> tuple[str, str]:
    obj = _obj(src)
    rep = obj + ".res.txt"
    if incremental and os.path.exists(obj) and os.path.exists(rep):
        newest = max(os.path.getmtime(p) for p in _deps(src))
        if os.path.getmtime(obj) >= newest:
            return src, open(rep).read()
    cmd = [hipcc(), *FLAGS, "-c", src, "-o", obj + ".tmp"]
    if src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    else:
        cmd = [hipcc(), *FLAGS, "-x", "hip", "--cuda-host-only", "-c", src, "-o", obj + ".tmp"]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in proc.stderr.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{err[-6000:]}")
    os.replace(obj + ".tmp", obj)
    with open(rep, "w") as f:
        f.write(err)
    return src, err


_KEYS = {
    "VGPRs": "vgprs", "AGPRs": "agprs", "SGPRs": "sgprs",
    "ScratchSize [bytes/lane]": "scratch_bytes", "Occupancy [waves/SIMD]": "occupancy",
    "LDS Size [bytes/block]": "lds_bytes",
}


def parse_resources(text: str) -> dict:
    out, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?): (-?\d+)", line)
        if m and cur is not None and m.group(1).strip() in _KEYS:
            out[cur][_KEYS[m.group(1).strip()]] = int(m.group(2))
    return out


def build(incremental: bool = False, jobs: int | None = None, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = _sources()
    jobs = jobs or min(16, os.cpu_count() or 4)
    # compile the slowest (kernel) sources first
    srcs.sort(key=lambda s: (not s.endswith(".hip"), -os.path.getsize(s)))
    reports = {}
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for src, rep in ex.map(lambda s: _compile(s, incremental), srcs):
            reports[src] = rep
            if verbose:
                print(f"[build] {os.path.basename(src)}", flush=True)
    tmp = LIB + f".tmp{os.getpid()}"
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
            *[_obj(s) for s in srcs]]
    proc = subprocess.run(link, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed:\n{proc.stderr[-4000:]}")
    os.replace(tmp, LIB)
    res = {}
    for rep in reports.values():
        res.update(parse_resources(rep))
    with open(RESOURCES, "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
    if verbose:
        print(f"[build] linked {LIB} ({len(res)} kernels)", flush=True)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--incremental", action="store_true")
    ap.add_argument("-j", type=int, default=None)
    a = ap.parse_args(argv)
    build(incremental=a.incremental, jobs=a.j)
    return 0


if __name__ == "__main__":
    sys.exit(main())
