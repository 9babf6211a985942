"""Summaries of rocprofv3 output for the benchmark's profiles (no GPU needed).

    python -m block_diffusion_sparse_herald_amd.profiling --workload W \
        --stats DIR --fetch DIR --write DIR --copy-bytes N --out-dir profiles

reads the CSV output of three rocprofv3 runs of bench.py (kernel trace + stats; one
FETCH_SIZE pass; one WRITE_SIZE pass), and writes
  profiles/kernel_stats_<W>.md   per-kernel average duration (kernel trace),
  profiles/hbm_traffic_<W>.json  HBM bytes per launch of the profiled kernels.
The counters read in KiB per dispatch; each is scaled by what it reads for a copy of
known size (the benchmark's K/V replica copies, `--copy-bytes` each), so the figures
are bytes as the copy defines them. The JSON records a digest of the kernel sources
(with the header that fixes the launch geometry); bench.py reports the traffic only
while they are unchanged.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
from collections import defaultdict

MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_diffusion_sparse_herald_amd", "csrc")

# profiled kernel (as the benchmark names it) -> (kernel name prefixes, source files)
KERNELS = {
    "attn_kernel+attn_combine_kernel": (["herald::attn_kernel", "herald::attn_combine_kernel"], ["attn.hip", "common.hpp", "kernels.hpp"]),
    "attn_kernel": (["herald::attn_kernel"], ["attn.hip", "common.hpp", "kernels.hpp"]),
    "scan": (["herald::scan_"], ["select.hip", "common.hpp", "kernels.hpp"]),  # whichever scan kernel the workload uses
    "refine_stats": (["herald::refine_stats_kernel"], ["refine.hip", "common.hpp", "kernels.hpp"]),
    "refine_scores": (["herald::refine_scores_kernel"], ["refine.hip", "common.hpp", "kernels.hpp"]),
    "gather": (["herald::gather_kernel"], ["gather.hip", "common.hpp", "kernels.hpp"]),
    # the fp32 attention (VALU kernel); the fp32 refine runs the refine kernels above
    "attn_f32_kernel": (["herald::attn_f32_kernel"], ["attn.hip", "common.hpp", "kernels.hpp"]),
}


def sources_digest(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def short(name: str) -> str:
    n = name.split("(")[0]
    return n[5:] if n.startswith("void ") else n


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def kernel_stats(stats_dir: str):
    rows = []
    with open(_one(os.path.join(stats_dir, "**", "*kernel_stats.csv"))) as fh:
        for r in csv.DictReader(fh):
            rows.append((short(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return rows


def counter_means(pmc_dir: str, counter: str):
    """kernel short name -> list of per-dispatch values (KiB), and the copy kernels' values."""
    per = defaultdict(list)
    with open(_one(os.path.join(pmc_dir, "**", "*counter_collection.csv"))) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            per[(short(r["Kernel_Name"]), int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
    return per


def copy_factor(per, copy_bytes: int) -> tuple[float, float]:
    """KiB the counter should read per replica copy / KiB it reads (largest copy dispatches)."""
    copies = [(g, v) for (k, g), v in per.items() if "copyBuffer" in k]
    if not copies:
        raise RuntimeError("no copy kernel in the counter run")
    g, vals = max(copies, key=lambda x: x[0])
    measured = sum(vals) / len(vals)
    return (copy_bytes / 1024.0) / measured, measured


def per_launch_kib(per, prefixes) -> float:
    total = 0.0
    for pre in prefixes:
        vals = [v for (k, _), vs in per.items() if k.startswith(pre) for v in vs]
        if not vals:
            raise RuntimeError(f"no dispatch of {pre} in the counter run")
        total += sum(vals) / len(vals)
    return total


def mfma_summary(workload: str, pmc_dir: str, stats_dir: str, out_dir: str, cmd: str) -> str:
    """profiles/mfma_util_<workload>.md from a `rocprofv3 --pmc MfmaUtil MfmaFlopsBF16` run:
    per kernel the mean MFMA busy share of the dispatch (rocprof's MfmaUtil: MFMA busy
    cycles over active cycles of all SIMDs), the bf16 MFMA flops it issued, and those flops
    over the kernel's mean duration in the kernel-trace run of the same workload."""
    vals = defaultdict(lambda: defaultdict(list))
    with open(_one(os.path.join(pmc_dir, "**", "*counter_collection.csv"))) as fh:
        for r in csv.DictReader(fh):
            vals[short(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    dur = {n: avg for n, _, avg, _, _, _ in kernel_stats(stats_dir)}
    md = [f"# MFMA utilisation, workload {workload}", "",
          "rocprofv3 counters per dispatch (eager launches); duration from the kernel-trace run of the same",
          f"workload (`kernel_stats_{workload}.md`); bf16 dense MFMA peak {MFMA_PEAK_TFLOPS} TFLOP/s.", "",
          "Command:", "", "```", cmd, "```", "",
          "| kernel | dispatches | MfmaUtil % | bf16 MFMA GFLOP per dispatch | mean us | MFMA TFLOP/s | % of peak |",
          "|---|---|---|---|---|---|---|"]
    for name in sorted(vals, key=lambda n: -sum(vals[n].get("MfmaFlopsBF16", [0.0]))):
        fl = vals[name].get("MfmaFlopsBF16", [])
        ut = vals[name].get("MfmaUtil", [])
        if not fl or sum(fl) == 0.0:
            continue
        gf = sum(fl) / len(fl) / 1e9
        us = dur.get(name)
        tf = gf / us * 1e3 if us else float("nan")  # GFLOP per us -> TFLOP/s
        md.append(f"| `{name}` | {len(fl)} | {sum(ut) / len(ut):.1f} | {gf:.3f} | "
                  f"{us if us else float('nan'):.2f} | {tf:.1f} | {100.0 * tf / MFMA_PEAK_TFLOPS:.1f} |")
    path = os.path.join(out_dir, f"mfma_util_{workload}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(md) + "\n")
    return path


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", required=True)
    ap.add_argument("--stats", required=True)
    ap.add_argument("--fetch", default="")
    ap.add_argument("--write", default="")
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--calibration-from", default="",
                    help="take the copy factors from another workload's JSON (for runs without replica copies)")
    ap.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--stats-cmd", default="")
    ap.add_argument("--pmc-cmd", default="")
    ap.add_argument("--mfma", default="", help="directory of a `--pmc MfmaUtil MfmaFlopsBF16` run: write only "
                                                "profiles/mfma_util_<workload>.md")
    ap.add_argument("--mfma-cmd", default="")
    args = ap.parse_args(argv)
    if args.mfma:
        print(mfma_summary(args.workload, args.mfma, args.stats, args.out_dir, args.mfma_cmd))
        return 0
    os.makedirs(args.out_dir, exist_ok=True)

    stats = kernel_stats(args.stats)
    md = [f"# Kernel durations, workload {args.workload}", "",
          "rocprofv3 kernel trace of the benchmark (HIP graph replays, one block per sequence per step).", "",
          "Command:", "", "```", args.stats_cmd, "```", "",
          "| kernel | calls | average us | min us | max us | % of kernel time |", "|---|---|---|---|---|---|"]
    for n, c, avg, mn, mx, pct in sorted(stats, key=lambda x: -x[5]):
        md.append(f"| `{n}` | {c} | {avg:.2f} | {mn:.2f} | {mx:.2f} | {pct:.2f} |")
    with open(os.path.join(args.out_dir, f"kernel_stats_{args.workload}.md"), "w") as fh:
        fh.write("\n".join(md) + "\n")

    fetch = counter_means(args.fetch, "FETCH_SIZE")
    write = counter_means(args.write, "WRITE_SIZE")
    if args.calibration_from:
        with open(args.calibration_from) as fh:
            cal = json.load(fh)["calibration"]
        ff, fcopy, fw, wcopy = cal["fetch_factor"], cal["fetch_kib_per_copy"], cal["write_factor"], cal["write_kib_per_copy"]
    else:
        ff, fcopy = copy_factor(fetch, args.copy_bytes)
        fw, wcopy = copy_factor(write, args.copy_bytes)
    entries = []
    for kname, (prefixes, files) in KERNELS.items():
        try:
            fk, wk = per_launch_kib(fetch, prefixes), per_launch_kib(write, prefixes)
        except RuntimeError:
            continue
        entries.append({"kernel": kname, "workload": args.workload, "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                        "bytes_per_launch": round((fk * ff + wk * fw) * 1024.0),
                        "sources_sha256": sources_digest(files)})
    doc = {"calibration": {"copy_bytes": args.copy_bytes, "fetch_kib_per_copy": round(fcopy, 1),
                           "write_kib_per_copy": round(wcopy, 1), "fetch_factor": round(ff, 4),
                           "write_factor": round(fw, 4),
                           "from": os.path.basename(args.calibration_from) if args.calibration_from else "this run"},
           "command": args.pmc_cmd, "entries": entries}
    with open(os.path.join(args.out_dir, f"hbm_traffic_{args.workload}.json"), "w") as fh:
        json.dump(doc, fh, indent=1)
    print(json.dumps(doc["calibration"]), len(entries), "kernels")
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
