"""rocprofv3 kernel statistics and hardware counters for the benchmark workloads.

`python -m dense_linear_algebra_potrf_amd.profile --raw DIR --out DIR [--config NAME ...]`

Run from the repository root on a machine with an MI355X.  For each workload of
bench.py it runs, each under rocprofv3 as its own process (the profiled program
is `python3 bench.py ...` itself):

  1. kernel statistics (`--kernel-trace --stats`), 20 timed calls;
  2. one counter pass per group below, each within the per-block limits of one
     pass (at most 8 SQ, 4 TCC, 2 TA and 2 GRBM counters), 3 timed calls;

plus the two passes of a plain 256 MiB device copy that calibrate FETCH_SIZE
and WRITE_SIZE (the factor that makes each read back the copy's known size).
It then writes, under --out, one Markdown summary per workload (named for the
kernel family and the workload) holding the commands, the per-kernel statistics
and the counter table, and a `<workload>.counters.json` with the calibrated
HBM traffic per launch that bench.py attaches to its roofline while the
family's sources are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from dense_linear_algebra_potrf_amd import metrics  # noqa: E402

PASS_TIMEOUT_S = 120
# GRBM_GUI_ACTIVE comes back summed over the chip's 8 accelerator complex dies
# (XCDs), each with its own graphics engine; the busy fractions below use the
# cycles of one of them.
XCDS = 8
SIMDS = 1024
CUS = 256

# counter groups, one rocprofv3 pass each
def counter_passes(dt: str, family: str) -> list[list[str]]:
    trans = "SQ_INSTS_VALU_TRANS_F64" if dt in ("f64", "c128") else "SQ_INSTS_VALU_TRANS_F32"
    passes = [
        ["FETCH_SIZE"],
        ["WRITE_SIZE", "TA_BUSY_avr", "GRBM_GUI_ACTIVE"],
        ["SQ_INSTS_VALU", trans, "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_ANY",
         "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAVES", "GRBM_GUI_ACTIVE"],
    ]
    if family == "blocked":
        passes.append(["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F64", "GRBM_GUI_ACTIVE"])
    if family in ("tiny", "posv_tiny"):
        # LDS against VALU: the register windows exchange every pivot column through LDS
        passes.append(["SQ_LDS_IDX_ACTIVE", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VALU",
                       "SQ_WAIT_INST_LDS", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE"])
    return passes


def bench_cmd(config: str | None, steps: int, warmup: int, copy: bool = False) -> list[str]:
    if copy:
        return ["python3", os.path.join(ROOT, "bench.py"), "--mode", "copy", "--copy-mib", "256",
                "--steps", str(steps)]
    return ["python3", os.path.join(ROOT, "bench.py"), "--config", config, "--no-secondary",
            "--no-cpu", "--steps", str(steps), "--warmup", str(warmup)]


def shown(cmd: list[str]) -> str:
    return " ".join("bench.py" if c.endswith("/bench.py") else c for c in cmd)


REPARSE = False      # rebuild the summaries from an earlier run's raw output


def run_rocprof(args: list[str], cmd: list[str], outdir: str) -> str:
    """Run `rocprofv3 <args> -d outdir -o run -- cmd` from /tmp; returns outdir."""
    outdir = os.path.abspath(outdir)
    if REPARSE:
        return outdir
    if os.path.exists(outdir):
        shutil.rmtree(outdir)
    full = ["rocprofv3", *args, "--output-format", "csv", "-d", outdir, "-o", "run", "--", *cmd]
    env = dict(os.environ, TMPDIR="/tmp")
    print("[profile]", " ".join(full), flush=True)
    proc = subprocess.run(full, cwd="/tmp", env=env, capture_output=True, text=True,
                          timeout=PASS_TIMEOUT_S)
    # the program's own last line must have been printed
    if proc.returncode != 0 and not proc.stdout.strip():
        raise RuntimeError(f"rocprofv3 failed ({proc.returncode}): {proc.stderr[-2000:]}")
    return outdir


def read_csv(outdir: str, suffix: str) -> list[dict]:
    rows = []
    for f in glob.glob(os.path.join(outdir, "**", f"*{suffix}"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def short_name(name: str) -> str:
    name = name.replace("void ", "").replace("bl::tiny_detail::", "").replace("bl::blocked_detail::", "")
    name = name.replace("bl::lds_detail::", "").replace("bl::potrs_detail::", "").replace("bl::", "")
    return name.split("(")[0]


def kernel_stats(outdir: str) -> list[dict]:
    rows = read_csv(outdir, "kernel_stats.csv")
    out = []
    for r in rows:
        out.append(dict(name=r["Name"], calls=int(r["Calls"]), avg_us=float(r["AverageNs"]) / 1e3,
                        min_us=float(r["MinNs"]) / 1e3, max_us=float(r["MaxNs"]) / 1e3,
                        share=float(r["Percentage"])))
    return sorted(out, key=lambda d: -d["share"])


def main_kernel(stats: list[dict]) -> str:
    for s in stats:
        if "potrf_" in s["name"] or "potrs_" in s["name"]:
            return s["name"]
    raise RuntimeError("no library kernel in the trace")


def counters(outdir: str, kernel: str) -> dict[str, float]:
    """Counter values per dispatch of `kernel`, averaged over its dispatches."""
    per: dict[str, dict[str, float]] = {}
    for r in read_csv(outdir, "counter_collection.csv"):
        if r["Kernel_Name"] != kernel:
            continue
        d = per.setdefault(r.get("Dispatch_Id", r.get("Correlation_Id")), {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    if not per:
        return {}
    names = set().union(*[set(v) for v in per.values()])
    return {n: sum(v.get(n, 0.0) for v in per.values()) / len(per) for n in names}


def calibrate(raw: str) -> tuple[float, float, list[str]]:
    """FETCH_SIZE and WRITE_SIZE factors from a plain 256 MiB device copy."""
    cmd = bench_cmd(None, 3, 0, copy=True)
    want_kib = 256 * 1024
    shown_cmds = []
    f = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        out = run_rocprof(["--pmc", ctr], cmd, os.path.join(raw, f"copy_{ctr}"))
        shown_cmds.append(f"rocprofv3 --pmc {ctr} --output-format csv -d <out> -o run -- {shown(cmd)}")
        vals = [float(r["Counter_Value"]) for r in read_csv(out, "counter_collection.csv")
                if r["Counter_Name"] == ctr and "copy" in r["Kernel_Name"].lower()]
        if not vals:
            names = sorted(set(r["Kernel_Name"] for r in read_csv(out, "counter_collection.csv")))
            raise RuntimeError(f"no {ctr} for the copy kernel among {names}")
        f[ctr] = want_kib / (sum(vals) / len(vals))
    return f["FETCH_SIZE"], f["WRITE_SIZE"], shown_cmds


def family_file_name(family: str, cfg: dict) -> str:
    op = cfg["op"]
    uplo = "lower" if cfg["uplo"] == "L" else "upper"
    head = family if family.startswith(op) else f"{op}_{family}"
    s = f"{head}_{cfg['dt']}_{uplo}_n{cfg['n']}"
    if op == "posv":
        s += f"_nrhs{cfg['nrhs']}"
    return s + f"_b{cfg['batch']}"


def profile_config(name: str, raw: str, outdir: str, ffac: float, wfac: float,
                   calib_cmds: list[str]) -> dict:
    cfg = bench.CONFIGS[name]
    stats_cmd = bench_cmd(name, 20, 5)
    sdir = run_rocprof(["--kernel-trace", "--stats"], stats_cmd, os.path.join(raw, f"{name}_stats"))
    stats = kernel_stats(sdir)
    kern = main_kernel(stats)
    family = "blocked" if "blocked" in kern else ("lds" if "lds" in kern else "tiny")
    if cfg["op"] == "posv":
        family = "posv_tiny" if "tiny" in kern else "posv_split"
    ctr_cmd = bench_cmd(name, 3, 1)
    vals: dict[str, float] = {}
    shown_cmds = [f"rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o run -- {shown(stats_cmd)}"]
    for i, group in enumerate(counter_passes(cfg["dt"], family)):
        out = run_rocprof(["--pmc", *group], ctr_cmd, os.path.join(raw, f"{name}_pmc{i}"))
        shown_cmds.append(f"rocprofv3 --pmc {' '.join(group)} --output-format csv -d <out> -o run -- "
                          f"{shown(ctr_cmd)}")
        vals.update(counters(out, kern))
    avg_us = next(s["avg_us"] for s in stats if s["name"] == kern)
    batch = cfg["batch"]
    if cfg["op"] == "potrf":
        alg = metrics.potrf_bytes(cfg["n"], batch, cfg["dt"], cfg["uplo"])
        flops = metrics.potrf_flops(cfg["n"], cfg["dt"]) * batch
    else:
        alg = metrics.posv_bytes(cfg["n"], cfg["nrhs"], batch, cfg["dt"], cfg["uplo"])
        flops = metrics.posv_flops(cfg["n"], cfg["nrhs"], cfg["dt"]) * batch
    fetch = vals.get("FETCH_SIZE", 0.0) * 1024 * ffac
    write = vals.get("WRITE_SIZE", 0.0) * 1024 * wfac
    rec = {"config": name, "kernel": short_name(kern), "family": family,
           "source_digest": bench.source_digest(family), "avg_kernel_us": avg_us,
           "alg_bytes": alg, "alg_flops": flops,
           "traffic_bytes": fetch + write, "fetch_bytes": fetch, "write_bytes": write,
           "fetch_factor": ffac, "write_factor": wfac, "counters": vals}
    fname = family_file_name(family, cfg)
    with open(os.path.join(outdir, f"{name}.counters.json"), "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    with open(os.path.join(outdir, fname + ".md"), "w") as f:
        f.write(summary_md(name, cfg, stats, kern, vals, rec, shown_cmds + calib_cmds))
    print(f"[profile] {name}: {short_name(kern)} {avg_us:.2f} us -> {fname}.md", flush=True)
    return rec


def summary_md(name, cfg, stats, kern, vals, rec, cmds) -> str:
    avg_us = rec["avg_kernel_us"]
    batch = cfg["batch"]
    gbs = rec["alg_bytes"] / (avg_us * 1e-6) / 1e9
    tfs = rec["alg_flops"] / (avg_us * 1e-6) / 1e12
    peak_tf = metrics.PEAK_TFLOPS[cfg["dt"]]
    lines = [f"# rocprofv3: {bench.describe(cfg)}", "",
             "Written by `python -m dense_linear_algebra_potrf_amd.profile --raw <raw> --out profiles`, which ran",
             "these commands, each from /tmp with TMPDIR=/tmp on one MI355X (the bench's own restore copies are",
             "the `__amd_rocclr_copyBuffer` rows, made outside the timed region; the last two commands",
             "calibrate FETCH_SIZE and WRITE_SIZE on a plain 256 MiB device copy):", "", "```"]
    lines += cmds
    lines += ["```", "", "| Kernel | Calls | Average (µs) | Min (µs) | Max (µs) | Share of GPU time |",
              "|---|---|---|---|---|---|"]
    for s in stats[:5]:
        lines.append(f"| `{short_name(s['name'])}` | {s['calls']} | {s['avg_us']:.2f} | {s['min_us']:.2f} | "
                     f"{s['max_us']:.2f} | {s['share']:.1f}% |")
    lines += ["", f"Algorithmic bytes per launch {rec['alg_bytes'] / 1e6:.1f} MB, flops per launch "
                  f"{rec['alg_flops'] / 1e9:.3f} GFLOP; at the average kernel duration that is "
                  f"{gbs:.0f} GB/s ({100 * gbs / metrics.HBM_PEAK_GBS:.1f}% of 8 TB/s) and {tfs:.2f} TFLOP/s "
                  f"({100 * tfs / peak_tf:.1f}% of {peak_tf} TFLOP/s).", ""]
    lines += ["Counters per dispatch of the library kernel (averaged over its dispatches):", "",
              "| Counter | Value | Derived |", "|---|---|---|"]
    gui = vals.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
    for k in sorted(vals):
        v = vals[k]
        derived = ""
        if k == "FETCH_SIZE":
            derived = f"{rec['fetch_bytes'] / 1e6:.1f} MB read (x{rec['fetch_factor']:.3f})"
        elif k == "WRITE_SIZE":
            derived = f"{rec['write_bytes'] / 1e6:.1f} MB written (x{rec['write_factor']:.3f})"
        elif k == "SQ_INSTS_VALU":
            derived = f"{v / batch:.0f} wave instructions per matrix"
        elif k.startswith("SQ_INSTS_VALU_TRANS"):
            derived = f"{v / batch:.0f} per matrix"
        elif k == "SQ_INSTS_LDS":
            derived = f"{v / batch:.0f} per matrix"
        elif k == "SQ_WAIT_INST_ANY" and vals.get("SQ_WAVE_CYCLES"):
            derived = f"{100 * v / vals['SQ_WAVE_CYCLES']:.0f}% of wave cycles waiting"
        elif k == "SQ_LDS_BANK_CONFLICT" and vals.get("SQ_INSTS_LDS"):
            derived = f"{v / vals['SQ_INSTS_LDS']:.2f} conflict cycles per LDS instruction"
        elif k == "TA_BUSY_avr" and gui:
            derived = f"address unit busy {100 * v / gui:.0f}% of GPU cycles"
        elif k == "SQ_VALU_MFMA_BUSY_CYCLES" and gui:
            derived = f"{100 * v / (gui * SIMDS):.0f}% of SIMD cycles on MFMA"
        elif k == "SQ_LDS_IDX_ACTIVE" and gui:
            derived = f"LDS busy {100 * v / (gui * CUS):.0f}% of CU cycles"
        elif k == "SQ_ACTIVE_INST_VALU" and gui:
            derived = f"VALU busy {100 * 4 * v / (gui * SIMDS):.0f}% of SIMD cycles"
        elif k == "SQ_ACTIVE_INST_LDS" and vals.get("SQ_INSTS_LDS"):
            derived = f"{4 * v / vals['SQ_INSTS_LDS']:.1f} cycles per LDS instruction"
        elif k == "SQ_WAIT_INST_LDS" and vals.get("SQ_WAVE_CYCLES"):
            derived = f"{100 * v / vals['SQ_WAVE_CYCLES']:.0f}% of wave cycles waiting to issue LDS"
        elif k == "SQ_BUSY_CU_CYCLES" and gui:
            derived = f"CU busy {100 * v / (gui * CUS):.0f}% of cycles"
        elif k == "GRBM_GUI_ACTIVE":
            derived = f"{v / XCDS:.0f} cycles per XCD"
        lines.append(f"| {k} | {v:.6g} | {derived} |")
    lines += ["", f"HBM traffic per launch {rec['traffic_bytes'] / 1e6:.1f} MB against {rec['alg_bytes'] / 1e6:.1f} MB "
                  f"algorithmic ({rec['traffic_bytes'] / rec['alg_bytes']:.2f}x).", ""]
    return "\n".join(lines)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--raw", required=True, help="directory for rocprofv3's raw output")
    ap.add_argument("--out", required=True, help="directory for the summaries")
    ap.add_argument("--config", action="append", choices=sorted(bench.CONFIGS))
    ap.add_argument("--reparse", action="store_true",
                    help="rebuild the summaries from the raw output of an earlier run")
    a = ap.parse_args(argv)
    global REPARSE
    REPARSE = a.reparse
    a.raw, a.out = os.path.abspath(a.raw), os.path.abspath(a.out)
    os.makedirs(a.raw, exist_ok=True)
    os.makedirs(a.out, exist_ok=True)
    ffac, wfac, calib_cmds = calibrate(a.raw)
    print(f"[profile] calibration: FETCH_SIZE x{ffac:.3f}, WRITE_SIZE x{wfac:.3f}", flush=True)
    for name in a.config or [bench.PRIMARY] + bench.SECONDARY:
        profile_config(name, a.raw, a.out, ffac, wfac, calib_cmds)
    return 0


if __name__ == "__main__":
    sys.exit(main())
