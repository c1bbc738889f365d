"""Turns rocprofv3 CSV output into the short text summaries kept under profiles/.

Three runs of the same bench command feed it:

  rocprofv3 --kernel-trace --stats --output-format csv -d <trace_dir> -o run -- python3 bench.py ...
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch_dir> -o run -- python3 bench.py ... --copy-calibration
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write_dir> -o run -- python3 bench.py ... --copy-calibration

The counter runs include one device copy of a known size (1 GiB read, 1 GiB
written, issued by ``bench.py --copy-calibration``). The ratio between that
size and what each counter reads for the copy is the scale factor applied to
every kernel's reading. The result is HBM-side traffic per launch.

Usage:
  python -m dsa_top_sparse_amd.profiling --trace T --fetch F --write W \
      --workload C3_chunk8k_off8192 --command "<the bench command>" --out profiles
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dsa_top_sparse_amd", "csrc")

# kernel symbol fragment -> (source file, short name)
KERNELS = {
    "mla_mfma_kernel": ("sparse_mla.hip", "mla_mfma_kernel"),
    "mla_combine_kernel": ("sparse_mla.hip", "mla_combine_kernel"),
    "mla_plain_kernel": ("sparse_mla.hip", "mla_plain_kernel"),
    "indexer_lds_kernel<true>": ("indexer.hip", "indexer_lds_kernel<true>"),
    "indexer_lds_kernel": ("indexer.hip", "indexer_lds_kernel"),
    "indexer_mfma_kernel": ("indexer.hip", "indexer_mfma_kernel"),
    "indexer_plain_kernel": ("indexer.hip", "indexer_plain_kernel"),
    "topk_filter_kernel": ("topk.hip", "topk_filter_kernel"),
    "topk_kernel": ("topk.hip", "topk_kernel"),
    "tau_kernel": ("fused.hip", "tau_kernel"),
    "cand_select_kernel": ("fused.hip", "cand_select_kernel"),
}
COPY_KERNEL = "copyBuffer"
COPY_BYTES = float(1 << 30)  # bench.py --copy-calibration: 2^28 fp32 read and written


def source_sha(name: str) -> str:
    return hashlib.sha256(open(os.path.join(CSRC, name), "rb").read()).hexdigest()[:16]


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def kernel_key(name: str):
    for frag, v in KERNELS.items():
        if frag in name:
            return v
    return None


def read_stats(trace_dir: str, skip: int = 0):
    """rocprofv3's per-kernel statistics, plus the mean over the dispatches
    after the first `skip` of each kernel (the bench's warm-up steps), taken
    from the kernel trace of the same run."""
    rows = list(csv.DictReader(open(_one(os.path.join(trace_dir, "**", "*kernel_stats.csv")))))
    out = {}
    for r in rows:
        k = kernel_key(r["Name"])
        if k:
            out[k[1]] = {"calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                         "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3,
                         "pct": float(r["Percentage"])}
    durs = {}
    for r in csv.DictReader(open(_one(os.path.join(trace_dir, "**", "*kernel_trace.csv")))):
        k = kernel_key(r["Kernel_Name"])
        if k:
            durs.setdefault(k[1], []).append(
                (int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    for short, st in out.items():
        d = [x[1] for x in sorted(durs.get(short, []))][skip:]
        st["timed_avg_us"] = statistics.mean(d) if d else float("nan")
    return out


def read_counter(pmc_dir: str, counter: str):
    """Mean counter value (KiB) per dispatch for each kernel, plus the copy kernel's."""
    rows = list(csv.DictReader(open(_one(os.path.join(pmc_dir, "**", "*counter_collection.csv")))))
    per, copy = {}, []
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        v = float(r["Counter_Value"])
        if COPY_KERNEL in r["Kernel_Name"]:
            copy.append(v)
            continue
        k = kernel_key(r["Kernel_Name"])
        if k:
            per.setdefault(k[1], []).append(v)
    if not copy:
        raise RuntimeError(f"no copy-kernel dispatch in {pmc_dir}: run bench.py with --copy-calibration")
    # the calibration copy is the largest one; other, small device copies of
    # the run (argument and workspace set-up) are not it
    return {k: statistics.mean(v) for k, v in per.items()}, max(copy)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--command", required=True, help="the bench command of the trace run")
    ap.add_argument("--pmc-command", default=None, help="the bench command of the counter runs (default: --command)")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--skip", type=int, default=0, help="warm-up dispatches per kernel left out of the timed mean")
    args = ap.parse_args()

    pmc_cmd = args.pmc_command or args.command
    stats = read_stats(args.trace, args.skip)
    fetch, fetch_copy = read_counter(args.fetch, "FETCH_SIZE")
    write, write_copy = read_counter(args.write, "WRITE_SIZE")
    f_fetch = COPY_BYTES / (fetch_copy * 1024.0)
    f_write = COPY_BYTES / (write_copy * 1024.0)

    os.makedirs(args.out, exist_ok=True)
    traffic_path = os.path.join(args.out, "traffic.json")
    try:
        traffic = json.load(open(traffic_path))
    except (OSError, ValueError):
        traffic = {}
    lines = [f"# rocprofv3 summary: {args.workload}", "",
             "Commands (each run separately, from the repository root):",
             f"  rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- {args.command}",
             f"  rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o run -- {pmc_cmd} --copy-calibration",
             f"  rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o run -- {pmc_cmd} --copy-calibration",
             "",
             "Counter scale (1 GiB device copy): FETCH_SIZE x %.4f, WRITE_SIZE x %.4f" % (f_fetch, f_write), "",
             f"avg us: rocprofv3's mean over all dispatches; timed avg us: mean after the first {args.skip} "
             "dispatches of each kernel (the bench's warm-up steps), the figure bench.py's HIP events measure.", "",
             "| kernel | calls | avg us | timed avg us | min us | max us | share | HBM read MB/launch | HBM write MB/launch | source sha |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for short, st in sorted(stats.items(), key=lambda kv: -kv[1]["avg_us"]):
        src = next(v[0] for v in KERNELS.values() if v[1] == short)
        rd = fetch.get(short, float("nan")) * 1024.0 * f_fetch
        wr = write.get(short, float("nan")) * 1024.0 * f_write
        sha = source_sha(src)
        lines.append(f"| {short} | {st['calls']} | {st['avg_us']:.1f} | {st['timed_avg_us']:.1f} | {st['min_us']:.1f} | {st['max_us']:.1f} | "
                     f"{st['pct']:.1f}% | {rd / 1e6:.1f} | {wr / 1e6:.1f} | {sha} |")
        traffic.setdefault(args.workload, {})[short] = {
            "source": src, "bytes_per_launch": rd + wr, "read_bytes": rd, "write_bytes": wr,
            "fetch_scale": f_fetch, "write_scale": f_write, "avg_launch_us": st["timed_avg_us"], "source_sha": sha}
    with open(os.path.join(args.out, f"kernels_{args.workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(traffic_path, "w") as f:
        json.dump(traffic, f, indent=1, sort_keys=True)
    print("\n".join(lines))


if __name__ == "__main__":
    main()
