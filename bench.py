"""Benchmark of the attention forward pass on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = one full forward pass (fa_fwd) over the workload's tensors, which
are drawn (seeded) and uploaded to HBM before timing starts.  Prints ONE JSON
line on stdout.  Default workload: causal bf16, B=1, H_q=32, H_kv=8,
qL=kL=8192, D=128.

  value     algorithmic TFLOP/s of the timed steps (4*B*H_q*qL*kL*D, halved
            for causal), wall clock between two device synchronisations
  roofline  the kernel's achieved TFLOP/s from HIP events recorded around
            each launch on the launch stream, against the MI355X dense matrix
            peak for the dtype
  cpu_baseline  the fp64 CPU oracle, timed on this host on a bounded sample
            of the same workload's query rows
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X dense matrix peaks (TFLOP/s) and HBM bandwidth (GB/s), published
# figures: 256 CUs at 2.4 GHz.
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}
PEAK_HBM_GBS = 8000.0


PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "flashattention_forward_04_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sources(w) -> list:
    """The source files the kernels of workload w are compiled from (and the
    host code that chooses and launches them)."""
    common = ["fa_common.h", "fa_api.cpp"]
    if w.backward:
        return common + ["fa_bwd_bf16.h", f"fa_bwd_bf16_d{w.D}.hip"]
    kind = "bf16" if w.dtype == "bf16" else "f32"
    return common + [f"fa_fwd_{kind}.h", "fa_merge.h", f"fa_fwd_{kind}_d{w.D}.hip"]


def kernel_source_hash(w) -> str:
    """sha256 over the sources of w's kernels: a recorded traffic figure is
    only reported while the kernels it was measured on are unchanged."""
    import hashlib

    h = hashlib.sha256()
    for name in sorted(kernel_sources(w)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def recorded_traffic(w):
    """HBM bytes per launch recorded by --summarize for workload w, or None."""
    path = os.path.join(PROFILES, f"{w.name}.traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != kernel_source_hash(w):
        return None
    return rec.get("hbm_bytes_per_launch")


def _read_counter_csv(path, counter):
    """{kernel name: [per-dispatch values]} for one counter of a rocprofv3 CSV."""
    import csv

    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


# rocprofv3 passes of one profile (bench.py --profile).  The trace of record
# uses the protocol the benchmark line is measured with (5 warm-up launches,
# 20 timed); the steady-state trace lets the clock settle first.  Counters
# are taken in runs of their own, a few per pass, never beside a trace.
DRIVER_PROTOCOL = "--steps 20 --warmup 5"
STEADY_PROTOCOL = "--steps 100 --warmup 100"
N_XCD = 8       # MI355X: 8 XCDs (GRBM_GUI_ACTIVE is summed over them)
N_SIMD = 1024   # 256 CUs x 4 SIMDs
N_CU = 256


def counter_set(w):
    """The per-dispatch counters of the profile: clock, matrix-core busy
    cycles and operations, vector and transcendental instructions, LDS bank
    conflicts (one --pmc pass: 7 SQ counters and 1 GRBM)."""
    mops = "SQ_INSTS_VALU_MFMA_MOPS_BF16" if w.dtype == "bf16" else "SQ_INSTS_VALU_MFMA_MOPS_F32"
    return ["GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_WAVES", "SQ_INSTS_VALU",
            "SQ_INSTS_VALU_TRANS_F32", mops, "SQ_LDS_BANK_CONFLICT"]


def profile_commands(prof_dir, w):
    base = f" --workload {w.name}" if w.name != "causal_bf16_d128_8k" else ""
    counters = " ".join(counter_set(w))
    return {
        "copy_mib": 1024,
        "trace": f"rocprofv3 --kernel-trace --stats --output-format csv -d {prof_dir}/trace -o trace -- "
                 f"python3 bench.py {DRIVER_PROTOCOL} --no-cpu-baseline{base}",
        "steady": f"rocprofv3 --kernel-trace --stats --output-format csv -d {prof_dir}/steady -o steady -- "
                  f"python3 bench.py {STEADY_PROTOCOL} --no-cpu-baseline{base}",
        "counters": f"rocprofv3 --pmc {counters} --output-format csv -d {prof_dir}/counters -o counters -- "
                    f"python3 bench.py {DRIVER_PROTOCOL} --no-cpu-baseline{base}",
        "fetch": f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {prof_dir}/fetch -o fetch -- "
                 f"python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline{base}",
        "write": f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {prof_dir}/write -o write -- "
                 f"python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline{base}",
        "copyf": f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {prof_dir}/copyf -o copyf -- "
                 "python3 bench.py --copy-calibration-mib 1024",
        "copyw": f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {prof_dir}/copyw -o copyw -- "
                 "python3 bench.py --copy-calibration-mib 1024",
    }


def run_profile(prof_dir, w):
    """Run every rocprofv3 pass of the profile as a child process (this
    process never touches the GPU), each under a time limit of its own, then
    summarise.  Stops at the first pass that fails."""
    import shlex
    import subprocess

    cmds = profile_commands(prof_dir, w)
    limits = {"trace": 600, "steady": 300, "counters": 120, "fetch": 90, "write": 90, "copyf": 90, "copyw": 90}
    os.makedirs(prof_dir, exist_ok=True)
    for name in ("trace", "steady", "counters", "fetch", "write", "copyf", "copyw"):
        log(f"[profile] {w.name}: {name} pass")
        with open(os.path.join(prof_dir, f"{name}.log"), "w") as f:
            try:
                r = subprocess.run(shlex.split(cmds[name]), cwd=ROOT, stdout=f, stderr=subprocess.STDOUT,
                                   timeout=limits[name], env={**os.environ, "TMPDIR": "/tmp"})
            except subprocess.TimeoutExpired:
                raise SystemExit(f"[profile] {name} pass timed out after {limits[name]} s")
        if r.returncode != 0:
            raise SystemExit(f"[profile] {name} pass failed with status {r.returncode} "
                             f"(see {prof_dir}/{name}.log)")
    summarize(prof_dir, w, cmds)


def summarize(prof_dir, w, commands):
    """Write profiles/<workload>.md (+ .traffic.json) from rocprofv3 outputs.

    prof_dir holds the outputs of the passes in profile_commands: kernel
    traces under the benchmark's protocol (trace/) and after a long warm-up
    (steady/), one counter pass (counters/), FETCH_SIZE and WRITE_SIZE runs of
    the workload (fetch/, write/), and the same two counters on a device copy
    of known size (copyf/, copyw/).  FETCH_SIZE and WRITE_SIZE are KiB per
    dispatch; each is scaled by (known copy bytes / what the counter reads for
    that copy).
    """
    import csv
    import glob

    def one(pattern):
        hits = glob.glob(os.path.join(prof_dir, pattern))
        if not hits:
            raise FileNotFoundError(os.path.join(prof_dir, pattern))
        return hits[0]

    def trace_summary(sub, steps):
        stats = list(csv.DictReader(open(one(f"{sub}/*kernel_stats.csv"))))
        # the timed call's kernels: the backward workloads also run the
        # forward pass once, untimed, to produce O and L
        rows = [r for r in stats if "fa::" in r["Name"] and (("::bwd_" in r["Name"]) == bool(w.backward))]
        if not rows:
            raise RuntimeError(f"no fa:: kernel in the {sub} kernel-trace stats")
        # one call may launch more than one kernel (a split key range: the
        # partials, then their merge); the dominant one names the profile and
        # the per-call figures add up every kernel of the call
        rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
        trace = list(csv.DictReader(open(one(f"{sub}/*kernel_trace.csv"))))
        per = []
        for r in rows:
            disp = sorted((x for x in trace if x["Kernel_Name"] == r["Name"]), key=lambda x: int(x["Start_Timestamp"]))
            durs = [(int(x["End_Timestamp"]) - int(x["Start_Timestamp"])) / 1e3 for x in disp]
            timed = durs[-steps:]  # the timed steps are the last dispatches
            per.append((r, sum(timed) / len(timed), len(timed), durs))
        return per

    def n_steps(cmd):
        return int(cmd.split("--steps ")[1].split()[0])

    per_kernel = trace_summary("trace", n_steps(commands["trace"]))
    timed_us = sum(t for _, t, _, _ in per_kernel)
    n_timed = per_kernel[0][2]
    k = per_kernel[0][0]
    steady_us = None
    if glob.glob(os.path.join(prof_dir, "steady/*kernel_stats.csv")):
        steady = trace_summary("steady", n_steps(commands["steady"]))
        steady_us = sum(t for _, t, _, _ in steady)
    copy_bytes = commands["copy_mib"] << 20

    def scale(counter, sub_run, sub_copy):
        vals = _read_counter_csv(one(f"{sub_run}/*counter_collection.csv"), counter)
        kv = [v for n, v in vals.items() if "fa::" in n]
        per = sum(sum(x) / len(x) for x in kv) * 1024.0
        cvals = _read_counter_csv(one(f"{sub_copy}/*counter_collection.csv"), counter)
        cv = [v for n, v in cvals.items() if "copyBuffer" in n]
        cper = sum(cv[0]) / len(cv[0]) * 1024.0
        return per, cper, copy_bytes / cper

    f_raw, f_copy, f_factor = scale("FETCH_SIZE", "fetch", "copyf")
    w_raw, w_copy, w_factor = scale("WRITE_SIZE", "write", "copyw")
    fetch, write = f_raw * f_factor, w_raw * w_factor
    flops = w.flops()
    alg = algorithmic_bytes(w)
    peak = PEAK_TFLOPS[w.dtype]

    # ---- counters, per dispatch of the dominant kernel ----
    ctr_lines = []
    ctr_rec = None
    if glob.glob(os.path.join(prof_dir, "counters/*counter_collection.csv")):
        rows = list(csv.DictReader(open(one("counters/*counter_collection.csv"))))
        disp = {}
        for r in rows:
            if r["Kernel_Name"] != k["Name"]:
                continue
            d = disp.setdefault(int(r["Dispatch_Id"]), {"t0": int(r["Start_Timestamp"]), "t1": int(r["End_Timestamp"])})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        order = sorted(disp.values(), key=lambda d: d["t0"])
        mops = counter_set(w)[6]

        def derived(d):
            ns = d["t1"] - d["t0"]
            cyc = d["GRBM_GUI_ACTIVE"] / N_XCD  # GPU cycles of the dispatch
            return {"us": ns / 1e3, "ghz": cyc / ns, "cycles": cyc,
                    "mfma_busy": d["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * cyc),
                    "cu_busy": d["SQ_BUSY_CU_CYCLES"] / (N_CU * cyc),
                    "valu_per_wave": d["SQ_INSTS_VALU"] / max(1.0, d["SQ_WAVES"]),
                    "trans_per_wave": d["SQ_INSTS_VALU_TRANS_F32"] / max(1.0, d["SQ_WAVES"]),
                    "mfma_flop": d[mops] * 512,
                    "lds_conflict": d["SQ_LDS_BANK_CONFLICT"] / (N_CU * cyc)}

        der = [derived(d) for d in order]
        timed = der[-n_timed:]
        avg = {key: sum(x[key] for x in timed) / len(timed) for key in timed[0]}
        ctr_rec = avg
        ctr_lines = [
            "## Counters (one rocprofv3 --pmc pass under the benchmark's protocol)",
            "",
            "```",
            commands["counters"],
            "```",
            "",
            f"Clock = GRBM_GUI_ACTIVE / {N_XCD} XCDs / dispatch time; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
            f"({N_SIMD} SIMDs x cycles); CU busy = SQ_BUSY_CU_CYCLES / ({N_CU} CUs x cycles); matrix FLOP = "
            f"{mops} x 512; LDS conflict = SQ_LDS_BANK_CONFLICT / ({N_CU} CUs x cycles).  Timings under --pmc "
            "are serialised dispatches, so they differ from the trace above.",
            "",
            f"Averages over the {len(timed)} timed dispatches: clock {avg['ghz']:.3f} GHz"
            + (" (a dispatch this short is shorter than the counter window, so this overstates the clock and "
               "understates the busy fractions)" if avg["us"] < 150 else "") + ", "
            f"{avg['cycles'] / 1e6:.3f} M cycles, MFMA busy {avg['mfma_busy']:.3f}, CU busy {avg['cu_busy']:.3f}, "
            f"{avg['valu_per_wave']:.0f} VALU and {avg['trans_per_wave']:.0f} transcendental instructions per wave, "
            f"matrix FLOP {avg['mfma_flop']:.4g} ({avg['mfma_flop'] / flops:.3f}x the algorithmic {flops:.4g}), "
            f"LDS bank-conflict cycles {100 * avg['lds_conflict']:.2f} % of CU cycles.",
            "",
            f"At the measured clock the matrix peak is {peak * avg['ghz'] / 2.4:.1f} TFLOP/s "
            f"({peak} at 2.4 GHz).",
            "",
            "| dispatch | us | GHz | MFMA busy | CU busy | VALU/wave |",
            "|---|---|---|---|---|---|",
            *[f"| {i + 1}{' (timed)' if i >= len(der) - n_timed else ''} | {x['us']:.1f} | {x['ghz']:.3f} | "
              f"{x['mfma_busy']:.3f} | {x['cu_busy']:.3f} | {x['valu_per_wave']:.0f} |" for i, x in enumerate(der[:25])],
            "",
        ]

    os.makedirs(PROFILES, exist_ok=True)
    rec = {"workload": w.name, "kernel": k["Name"], "calls": int(k["Calls"]),
           "protocol": commands["trace"].split("bench.py ")[1],
           "timed_steps": n_timed, "timed_avg_us": timed_us, "steady_avg_us": steady_us,
           "kernels": [{"name": r["Name"], "timed_avg_us": t} for r, t, _, _ in per_kernel],
           "min_us": float(k["MinNs"]) / 1e3, "max_us": float(k["MaxNs"]) / 1e3,
           "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
           "hbm_bytes_per_launch": fetch + write, "algorithmic_bytes": alg,
           "fetch_scale": f_factor, "write_scale": w_factor, "counters": ctr_rec,
           "source_sha256": kernel_source_hash(w), "sources": sorted(kernel_sources(w))}
    with open(os.path.join(PROFILES, f"{w.name}.traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    first = per_kernel[0][3]
    lines = [
        f"# {k['Name']} -- {w.name}",
        "",
        f"Workload: {w.note}; B={w.B} H_q={w.Hq} H_kv={w.Hkv} qL={w.qL} kL={w.kL} D={w.D} {w.dtype} "
        f"causal={w.causal} mask={w.mask_kind}.  FLOP per launch {flops:.4g}; algorithmic bytes {alg:.4g}.",
        "",
        "## Kernel duration (rocprofv3 --kernel-trace --stats), the benchmark's protocol",
        "",
        "```",
        commands["trace"],
        "```",
        "",
        f"| kernel | calls | avg us (all) | avg us (last {n_timed} = timed steps) | min us | max us |",
        "|---|---|---|---|---|---|",
        *[f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {t:.1f} | "
          f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |" for r, t, _, _ in per_kernel],
        "",
        f"**Per call (every kernel above, timed steps): {timed_us:.1f} us, "
        f"{flops / (timed_us * 1e-6) / 1e12:.1f} TFLOP/s, {100 * flops / (timed_us * 1e-6) / 1e12 / peak:.1f} % of "
        f"{peak} TFLOP/s.**",
        "",
        "Dominant kernel, every dispatch in order (warm-up, then timed), us: " + " ".join(f"{x:.0f}" for x in first),
        "",
    ]
    if steady_us is not None:
        lines += [
            "## Steady state (same trace after a long warm-up)",
            "",
            "```",
            commands["steady"],
            "```",
            "",
            f"Per call: {steady_us:.1f} us, {flops / (steady_us * 1e-6) / 1e12:.1f} TFLOP/s, "
            f"{100 * flops / (steady_us * 1e-6) / 1e12 / peak:.1f} % of {peak} TFLOP/s.",
            "",
        ]
    lines += ctr_lines
    lines += [
        "## HBM traffic (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE; KiB per dispatch, summed over the call's kernels)",
        "",
        "```",
        commands["fetch"],
        commands["write"],
        commands["copyf"],
        commands["copyw"],
        "```",
        "",
        f"Copy calibration: a device copy of {copy_bytes} bytes reads FETCH_SIZE = {f_copy:.4g} B "
        f"(scale {f_factor:.3f}) and WRITE_SIZE = {w_copy:.4g} B (scale {w_factor:.3f}).",
        "",
        "| counter | raw bytes/launch | scaled bytes/launch |",
        "|---|---|---|",
        f"| FETCH_SIZE | {f_raw:.4g} | {fetch:.4g} |",
        f"| WRITE_SIZE | {w_raw:.4g} | {write:.4g} |",
        f"| total | | {fetch + write:.4g} ({(fetch + write) / alg:.2f}x algorithmic) |",
        "",
        f"At the timed average: algorithmic {alg / (timed_us * 1e-6) / 1e9:.0f} GB/s, measured "
        f"{(fetch + write) / (timed_us * 1e-6) / 1e9:.0f} GB/s, of {PEAK_HBM_GBS:.0f} GB/s HBM peak "
        f"(roofline bound: {roofline_bound(w)}"
        + (f"; {buffer_sets(w)} buffer sets rotated" if roofline_bound(w) == "hbm" else "") + ").",
        "",
        f"Kernel source sha256 {rec['source_sha256'][:16]}... over {', '.join(rec['sources'])}; bench.py reports "
        "this traffic only while it matches.",
        "",
    ]
    with open(os.path.join(PROFILES, f"{w.name}.md"), "w") as f:
        f.write("\n".join(lines))
    log(f"wrote profiles/{w.name}.md and .traffic.json")


def find_workload(W, name):
    every = {x.name: x for x in (*W.CONFIGS.values(), *W.SHORT_KL, *W.HEAD_DIMS, *W.SPLIT_KV, *W.DROPOUT,
                                 *W.WINDOW, *W.RAGGED, *W.BACKWARD)}
    if name not in every:
        raise SystemExit(f"unknown workload {name!r}; known: {', '.join(sorted(every))}")
    return every[name]


def roofline_bound(w) -> str:
    """'mfma' when the algorithmic flop per byte is above the ridge of the
    dtype's matrix peak and the HBM peak, 'hbm' below it."""
    ridge = PEAK_TFLOPS[w.dtype] * 1e12 / (PEAK_HBM_GBS * 1e9)
    return "mfma" if w.flops() / algorithmic_bytes(w) >= ridge else "hbm"


def buffer_sets(w) -> int:
    """Buffer sets rotated through for an HBM-bound workload: at least 3, and
    more than 256 MB of inputs and outputs in all."""
    return max(3, (512 << 20) // algorithmic_bytes(w) + 1)


def algorithmic_bytes(w) -> int:
    """Bytes every launch must move at least once: Q, K, V, O, L (and the
    mask); the backward pass reads Q, K, V, O, dO, L and writes dQ, dK, dV."""
    esz = 2 if w.dtype == "bf16" else 4
    qo = (5 if w.backward else 2) * w.B * w.Hq * w.qL * w.D * esz
    kv = (4 if w.backward else 2) * w.B * w.Hkv * w.kL * w.D * esz
    lse = w.B * w.Hq * w.qL * 4
    mask = 0
    if w.mask_kind == "additive":
        mask = w.B * w.Hq * w.qL * w.kL * esz
    elif w.mask_kind == "bool":
        mask = w.B * w.Hq * w.qL * w.kL
    return qo + kv + lse + mask


def cpu_baseline(w, q, k, v, mask, target_s: float):
    """Time the fp64 oracle on a uniform random sample of query rows.

    Row counts are calibrated so the timed run is about target_s seconds.
    FLOP per row = 4*D*(number of keys the row attends under the causal rule),
    the same accounting as the GPU metric.
    """
    import numpy as np

    from oracle import OracleLib

    lib = OracleLib()
    qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
    md, kind = None, "none"
    if mask is not None:
        kind = "bool" if w.mask_kind == "bool" else "additive"
        md = mask.double().numpy() if kind == "additive" else mask.numpy()
    total_rows = w.B * w.Hq * w.qL
    rng = np.random.default_rng(99)

    def run(n):
        rows = np.sort(rng.choice(total_rows, size=min(n, total_rows), replace=False)).astype(np.int64)
        i = rows % w.qL
        keys = np.minimum(i + 1, w.kL) if w.causal else np.full(rows.shape, w.kL)
        if w.window is not None:
            keys = np.maximum(0, keys - np.maximum(0, i - w.window + 1))
        flops = float(4.0 * w.D * keys.sum())
        t0 = time.perf_counter()
        lib.fwd(qd, kd, vd, scale=w.scale, causal=w.causal, mask=md, mask_kind=kind, rows=rows,
                dropout_p=w.dropout_p, seed=w.seed, window=w.window)
        return time.perf_counter() - t0, flops, rows.size

    dt, _, n = run(256)
    n2 = int(min(total_rows, max(256, 256 * target_s / max(dt, 1e-3))))
    dt, flops, n = run(n2)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": lib.threads(), "kind": "oracle",
            "sample": f"{n} query rows drawn uniformly from the {total_rows} rows of {w.name} "
                      f"(fp64, {dt:.1f} s, {flops / 1e9:.1f} GFLOP)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="causal_bf16_d128_8k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (a known-size kernel that "
                         "scales the FETCH_SIZE / WRITE_SIZE counters), then exit")
    ap.add_argument("--summarize", metavar="PROF_DIR", default=None,
                    help="only write profiles/<workload>.md from rocprofv3 outputs under PROF_DIR, then exit")
    ap.add_argument("--profile", metavar="PROF_DIR", default=None,
                    help="run every rocprofv3 pass of the workload's profile into PROF_DIR (as child "
                         "processes), then write profiles/<workload>.md")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              f"(the attention path needs no cross-GPU exchange; see the sharding notes in the docs).",
              file=sys.stderr)
        sys.exit(2)

    import workloads as W

    if args.summarize or args.profile:
        w = find_workload(W, args.workload)
        prof_dir = args.summarize or args.profile
        if args.profile:
            run_profile(prof_dir, w)
        else:
            summarize(prof_dir, w, profile_commands(prof_dir, w))
        return

    import torch

    import flashattention_forward_04_amd as fa

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n} bytes device-to-device 3 times")
        return

    w = find_workload(W, args.workload)
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name} ({getattr(props, 'gcnArchName', '?')}), {props.multi_processor_count} CUs")
    log(f"workload: {w.name}: {w.note}")

    q, k, v, mask = W.draw(w)
    bound = roofline_bound(w)
    # A workload bound by HBM is timed over several buffer sets in turn, more
    # than 256 MB in all, so that no launch finds its inputs in the 256 MB
    # Infinity Cache (MALL) or the L2 from the launch before.
    n_sets = buffer_sets(w) if bound == "hbm" else 1
    stream = torch.cuda.current_stream(dev)
    sets = []
    for _ in range(n_sets):
        out = (torch.empty((w.B, w.qL, w.Hq, w.D), dtype=q.dtype, device=dev).transpose(1, 2) if w.token_major_out
               else torch.empty((w.B, w.Hq, w.qL, w.D), dtype=q.dtype, device=dev))
        sets.append((q.to(dev), k.to(dev), v.to(dev), None if mask is None else mask.to(dev), out,
                     torch.empty((w.B, w.Hq, w.qL), dtype=torch.float32, device=dev)))
    if n_sets > 1:
        log(f"rotating {n_sets} buffer sets, {n_sets * algorithmic_bytes(w) / 1e6:.0f} MB of inputs and outputs")

    if w.backward:
        # the forward pass once (its O and L feed every backward step), then
        # the gradient buffers; a step is one fa_bwd call
        dod = W.draw_grad(w).to(dev)
        grads = []
        for qd, kd, vd, md, out, lse in sets:
            fa.fwd(qd, kd, vd, mask=md, causal=w.causal, scale=w.scale, out=out, lse=lse, stream=stream)
            grads.append((torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd), torch.empty_like(lse)))
        torch.cuda.synchronize()

    def step(i):
        qd, kd, vd, md, out, lse = sets[i % n_sets]
        if w.backward:
            dq, dk, dv, delta = grads[i % n_sets]
            fa.bwd(qd, kd, vd, out, dod, lse, mask=md, causal=w.causal, scale=w.scale, dq=dq, dk=dk, dv=dv,
                   delta=delta, stream=stream)
            return
        fa.fwd(qd, kd, vd, mask=md, causal=w.causal, scale=w.scale, out=out, lse=lse, stream=stream,
               dropout_p=w.dropout_p, seed=w.seed, window=w.window)

    # HIP events on the launch stream: around each warm-up call (they show
    # how the clock settles), and one pair around the timed region, whose
    # calls run back to back.  (An event pair per timed call costs the host
    # ~9 us per call; calls of a few tens of us would then be timed at the
    # host's pace, with the GPU idle between them.)
    def events(n):
        return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]

    wev = events(args.warmup)
    for i, (a, b) in enumerate(wev):
        a.record(stream)
        step(i)
        b.record(stream)
    ta, tb = events(1)[0]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ta.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    tb.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    warm_ms = [a.elapsed_time(b) for a, b in wev]
    log("per-launch us, warm-up: " + " ".join(f"{x * 1e3:.0f}" for x in warm_ms))
    kern_avg_ms = ta.elapsed_time(tb) / args.steps
    ms_per_step = wall * 1e3 / args.steps

    flops = w.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kern_avg_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    log(f"kernel avg {kern_avg_ms * 1e3:.1f} us over the {args.steps} timed calls; "
        f"{achieved:.1f} TFLOP/s = {100 * achieved / peak:.1f}% of {peak} TFLOP/s")
    nbytes = algorithmic_bytes(w)
    log(f"algorithmic bytes {nbytes / 1e6:.1f} MB -> {nbytes / (kern_avg_ms * 1e-3) / 1e9:.0f} GB/s "
        f"({100 * nbytes / (kern_avg_ms * 1e-3) / 1e9 / PEAK_HBM_GBS:.1f}% of HBM)")

    cpu = None
    if not args.no_cpu_baseline and not w.backward:
        cpu = cpu_baseline(w, q, k, v, mask, args.cpu_seconds)
        log(f"cpu baseline: {cpu}")

    gbs = nbytes / (kern_avg_ms * 1e-3) / 1e9
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
    roof.update({"traffic": recorded_traffic(w), "kernel_avg_us": round(kern_avg_ms * 1e3, 2)})
    metric = ("attention fwd TFLOP/s + % MFMA peak, bf16 D=128 causal qL=kL=8192" if w is W.HEADLINE
              else f"attention {'bwd' if w.backward else 'fwd'} TFLOP/s, {w.name}")
    res = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V)",
        "config": {"workload": w.name, "B": w.B, "H_q": w.Hq, "H_kv": w.Hkv, "qL": w.qL, "kL": w.kL, "D": w.D,
                   "causal": w.causal, "mask": w.mask_kind, "scale": w.scale,
                   **({"dropout": w.dropout_p} if w.dropout_p is not None else {}),
                   **({"window": w.window} if w.window is not None else {}),
                   **({"pass": "backward"} if w.backward else {}),
                   "o_layout": "token-major" if w.token_major_out else "head-major",
                   "flop_per_step": flops},
        "mfma_peak_frac": round(achieved / peak, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
