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


def kernel_source_hash() -> str:
    """sha256 over the kernel sources: a recorded traffic figure is only
    reported while the kernels it was measured on are unchanged."""
    import hashlib

    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h", ".cpp")):
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
    if rec.get("source_sha256") != kernel_source_hash():
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


def summarize(prof_dir, w, commands):
    """Write profiles/<workload>.md (+ .traffic.json) from rocprofv3 outputs.

    prof_dir holds the outputs of: a --kernel-trace --stats run (trace/),
    FETCH_SIZE and WRITE_SIZE runs of the workload (fetch/, write/), and the
    same two counters on a device copy of known size (copyf/, copyw/).
    The counters are KiB per dispatch; each is scaled by (known copy bytes /
    what the counter reads for that copy).
    """
    import csv
    import glob

    def one(pattern):
        hits = glob.glob(os.path.join(prof_dir, pattern))
        if not hits:
            raise FileNotFoundError(os.path.join(prof_dir, pattern))
        return hits[0]

    stats = list(csv.DictReader(open(one("trace/*kernel_stats.csv"))))
    fa_rows = [r for r in stats if "fa::" in r["Name"]]
    if not fa_rows:
        raise RuntimeError("no fa:: kernel in the kernel-trace stats")
    # one call may launch more than one kernel (a split key range: the
    # partials, then their merge); the dominant one names the profile and the
    # per-call figures add up every kernel of the call
    fa_rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    k = fa_rows[0]
    avg_us = float(k["AverageNs"]) / 1e3
    trace = list(csv.DictReader(open(one("trace/*kernel_trace.csv"))))

    def timed_avg(name):
        # the timed steps are the last `steps` dispatches of the kernel (the
        # earlier ones are bench.py's warm-up calls)
        disp = sorted((r for r in trace if r["Kernel_Name"] == name), key=lambda r: int(r["Start_Timestamp"]))
        timed = disp[-commands["steps"]:]
        return sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in timed) / len(timed) / 1e3, len(timed)

    per_kernel = [(r, *timed_avg(r["Name"])) for r in fa_rows]
    timed_us = sum(t for _, t, _ in per_kernel)
    n_timed = per_kernel[0][2]
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
    os.makedirs(PROFILES, exist_ok=True)
    rec = {"workload": w.name, "kernel": k["Name"], "calls": int(k["Calls"]), "avg_us": avg_us,
           "timed_steps": n_timed, "timed_avg_us": timed_us,
           "kernels": [{"name": r["Name"], "timed_avg_us": t} for r, t, _ in per_kernel],
           "min_us": float(k["MinNs"]) / 1e3, "max_us": float(k["MaxNs"]) / 1e3,
           "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
           "hbm_bytes_per_launch": fetch + write, "algorithmic_bytes": alg,
           "fetch_scale": f_factor, "write_scale": w_factor,
           "source_sha256": kernel_source_hash()}
    with open(os.path.join(PROFILES, f"{w.name}.traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    peak = PEAK_TFLOPS[w.dtype]
    lines = [
        f"# {k['Name']} -- {w.name}",
        "",
        f"Workload: {w.note}; B={w.B} H_q={w.Hq} H_kv={w.Hkv} qL={w.qL} kL={w.kL} D={w.D} {w.dtype} "
        f"causal={w.causal} mask={w.mask_kind}.  FLOP per launch {flops:.4g}; algorithmic bytes {alg:.4g}.",
        "",
        "## Kernel duration (rocprofv3 --kernel-trace --stats)",
        "",
        "```",
        commands["trace"],
        "```",
        "",
        f"| kernel | calls | avg us (all) | avg us (last {n_timed} = timed steps) | min us | max us |",
        "|---|---|---|---|---|---|",
        *[f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {t:.1f} | "
          f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |" for r, t, _ in per_kernel],
        "",
        f"Per call (every kernel above, timed steps): {timed_us:.1f} us, "
        f"{flops / (timed_us * 1e-6) / 1e12:.1f} TFLOP/s, {100 * flops / (timed_us * 1e-6) / 1e12 / peak:.1f} % of "
        f"{peak} TFLOP/s.",
        "",
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
        f"(roofline bound: {roofline_bound(w)}).",
        "",
        f"Kernel source sha256 {rec['source_sha256'][:16]}...; bench.py reports this traffic only while it matches.",
        "",
    ]
    with open(os.path.join(PROFILES, f"{w.name}.md"), "w") as f:
        f.write("\n".join(lines))
    log(f"wrote profiles/{w.name}.md and .traffic.json")


def find_workload(W, name):
    every = {x.name: x for x in (*W.CONFIGS.values(), *W.SHORT_KL, *W.HEAD_DIMS, *W.SPLIT_KV, *W.DROPOUT,
                                 *W.WINDOW, *W.RAGGED)}
    if name not in every:
        raise SystemExit(f"unknown workload {name!r}; known: {', '.join(sorted(every))}")
    return every[name]


def roofline_bound(w) -> str:
    """'mfma' when the algorithmic flop per byte is above the ridge of the
    dtype's matrix peak and the HBM peak, 'hbm' below it."""
    ridge = PEAK_TFLOPS[w.dtype] * 1e12 / (PEAK_HBM_GBS * 1e9)
    return "mfma" if w.flops() / algorithmic_bytes(w) >= ridge else "hbm"


def algorithmic_bytes(w) -> int:
    esz = 2 if w.dtype == "bf16" else 4
    qo = 2 * w.B * w.Hq * w.qL * w.D * esz
    kv = 2 * w.B * w.Hkv * w.kL * w.D * esz
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
    # the default warm-up (about 50 ms of work) lets the clocks settle after
    # the power dip that follows the first launches of a busy kernel, so the
    # timed steps measure the sustained rate
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="causal_bf16_d128_8k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (a known-size kernel that "
                         "scales the FETCH_SIZE / WRITE_SIZE counters), then exit")
    ap.add_argument("--summarize", metavar="PROF_DIR", default=None,
                    help="only write profiles/<workload>.md from rocprofv3 outputs under PROF_DIR, then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              f"(the attention path needs no cross-GPU exchange; see the sharding notes in the docs).",
              file=sys.stderr)
        sys.exit(2)

    import workloads as W

    if args.summarize:
        w = find_workload(W, args.workload)
        base = f"--workload {w.name}" if w.name != "causal_bf16_d128_8k" else ""
        cmds = {
            "copy_mib": 1024,
            "steps": args.steps,
            "trace": f"rocprofv3 --kernel-trace --stats --output-format csv -d {args.summarize}/trace -o trace -- "
                     f"python3 bench.py --steps {args.steps} --warmup {args.warmup} {base}".strip(),
            "fetch": f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {args.summarize}/fetch -o fetch -- "
                     f"python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline {base}".strip(),
            "write": f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {args.summarize}/write -o write -- "
                     f"python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline {base}".strip(),
            "copyf": f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {args.summarize}/copyf -o copyf -- "
                     "python3 bench.py --copy-calibration-mib 1024",
            "copyw": f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {args.summarize}/copyw -o copyw -- "
                     "python3 bench.py --copy-calibration-mib 1024",
        }
        summarize(args.summarize, w, cmds)
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
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    md = None if mask is None else mask.to(dev)
    out = None
    if w.token_major_out:
        out = torch.empty((w.B, w.qL, w.Hq, w.D), dtype=q.dtype, device=dev).transpose(1, 2)
    else:
        out = torch.empty((w.B, w.Hq, w.qL, w.D), dtype=q.dtype, device=dev)
    lse = torch.empty((w.B, w.Hq, w.qL), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        fa.fwd(qd, kd, vd, mask=md, causal=w.causal, scale=w.scale, out=out, lse=lse, stream=stream,
               dropout_p=w.dropout_p, seed=w.seed, window=w.window)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-launch kernel durations from HIP events on the launch stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    kern_avg_ms = sum(kern_ms) / len(kern_ms)
    ms_per_step = wall * 1e3 / args.steps

    flops = w.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kern_avg_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    log(f"kernel avg {kern_avg_ms * 1e3:.1f} us (min {min(kern_ms) * 1e3:.1f}, max {max(kern_ms) * 1e3:.1f}); "
        f"{achieved:.1f} TFLOP/s = {100 * achieved / peak:.1f}% of {peak} TFLOP/s")
    nbytes = algorithmic_bytes(w)
    log(f"algorithmic bytes {nbytes / 1e6:.1f} MB -> {nbytes / (kern_avg_ms * 1e-3) / 1e9:.0f} GB/s "
        f"({100 * nbytes / (kern_avg_ms * 1e-3) / 1e9 / PEAK_HBM_GBS:.1f}% of HBM)")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, q, k, v, mask, args.cpu_seconds)
        log(f"cpu baseline: {cpu}")

    bound = roofline_bound(w)
    gbs = nbytes / (kern_avg_ms * 1e-3) / 1e9
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
    roof.update({"traffic": recorded_traffic(w), "kernel_avg_us": round(kern_avg_ms * 1e3, 2)})
    metric = ("attention fwd TFLOP/s + % MFMA peak, bf16 D=128 causal qL=kL=8192" if w is W.HEADLINE
              else f"attention fwd TFLOP/s, {w.name}")
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
                   "o_layout": "token-major" if w.token_major_out else "head-major",
                   "flop_per_step": flops},
        "mfma_peak_frac": round(achieved / peak, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
