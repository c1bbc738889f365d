"""Summarises two rocprofv3 hardware-counter runs of the bench command into
``profiles/counters_<workload>.md``: MFMA utilisation, L2 hit rate,
instruction mix and LDS bank conflicts per kernel.

The two runs (each in a process of its own, no trace domains):

  rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_MFMA \\
      SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE \\
      --output-format csv -d <dir_a> -o run -- python3 bench.py ...
  rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_SCA SQ_ACTIVE_INST_LDS \\
      SQ_ACTIVE_INST_VMEM SQ_WAIT_INST_ANY SQ_WAVE_CYCLES SQ_ACTIVE_INST_ANY GRBM_GUI_ACTIVE \\
      --output-format csv -d <dir_b> -o run -- python3 bench.py ...

Definitions (per dispatch, then averaged over the dispatches after the first
`--skip` of each kernel):
  * active cycles = GRBM_GUI_ACTIVE / 8 (the counter comes summed over the
    8 XCDs; divided by the dispatch's duration it gives the clock);
  * MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (active cycles x 1,024 SIMDs);
  * L2 hit rate = TCC_HIT / (TCC_HIT + TCC_MISS);
  * LDS bank conflicts = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE;
  * issue / wait shares = SQ_ACTIVE_INST_* and SQ_WAIT_INST_ANY over
    SQ_WAVE_CYCLES (wave-cycles).

Usage:
  python -m dsa_top_sparse_amd.counters --a A --b B --workload C3_chunk8k_off8192 \\
      --command "<the bench command>" --skip 3
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import os
import statistics

from .profiling import KERNELS, ROOT, kernel_key, source_sha

N_XCD = 8
N_SIMD = 1024  # 256 CUs x 4

PASS_A = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_MFMA SQ_INSTS_LDS "
          "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE")
PASS_B = ("TCC_HIT_sum TCC_MISS_sum SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_SCA SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VMEM "
          "SQ_WAIT_INST_ANY SQ_WAVE_CYCLES SQ_ACTIVE_INST_ANY GRBM_GUI_ACTIVE")


def load(pmc_dir: str, skip: int):
    """{kernel: {counter: mean over dispatches after `skip`}}, {kernel: mean duration us}."""
    path = sorted(glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True))[0]
    vals = collections.defaultdict(lambda: collections.defaultdict(dict))
    dur = collections.defaultdict(dict)
    for r in csv.DictReader(open(path)):
        key = kernel_key(r["Kernel_Name"])
        if key is None:
            continue
        short = key[1]
        d = int(r["Dispatch_Id"])
        vals[short][r["Counter_Name"]][d] = vals[short][r["Counter_Name"]].get(d, 0.0) + float(r["Counter_Value"])
        dur[short][d] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    out, dus = {}, {}
    for short, cs in vals.items():
        ds = sorted(dur[short])[skip:] or sorted(dur[short])
        out[short] = {c: statistics.mean(v[d] for d in ds if d in v) for c, v in cs.items()}
        dus[short] = statistics.mean(dur[short][d] for d in ds)
    return out, dus


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--a", required=True, help="output directory of the first counter run")
    ap.add_argument("--b", required=True, help="output directory of the second counter run")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--command", required=True, help="the bench command both runs profiled")
    ap.add_argument("--skip", type=int, default=0)
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    args = ap.parse_args()

    A, dur = load(args.a, args.skip)
    B, _ = load(args.b, args.skip)
    lines = [f"# rocprofv3 hardware counters: {args.workload}", "",
             "Commands (each run separately, from the repository root):",
             f"  rocprofv3 --pmc {PASS_A} --output-format csv -d <dir_a> -o run -- {args.command}",
             f"  rocprofv3 --pmc {PASS_B} --output-format csv -d <dir_b> -o run -- {args.command}",
             "",
             f"Means over the dispatches after the first {args.skip} of each kernel. Active cycles = "
             f"GRBM_GUI_ACTIVE / {N_XCD} (summed over the XCDs); MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
             f"(active cycles x {N_SIMD} SIMDs); L2 hit = TCC_HIT / (TCC_HIT + TCC_MISS); LDS conflicts = "
             "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; issue and wait shares are SQ_ACTIVE_INST_* and "
             "SQ_WAIT_INST_ANY over SQ_WAVE_CYCLES. Profiled runs are slower than the bench's own timing.",
             "",
             "| kernel | dispatch us | clock GHz | MFMA busy | L2 hit | VALU / SALU / MFMA / LDS instructions (M) | "
             "LDS conflicts | VALU / SALU / LDS issue share | waiting | source sha |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for short in sorted(A, key=lambda s: -dur[s]):
        a, b = A[short], B.get(short, {})
        act = a["GRBM_GUI_ACTIVE"] / N_XCD
        mfma = a["SQ_VALU_MFMA_BUSY_CYCLES"] / (act * N_SIMD)
        hit = b["TCC_HIT_sum"] / max(b["TCC_HIT_sum"] + b["TCC_MISS_sum"], 1.0) if b else float("nan")
        wc = b.get("SQ_WAVE_CYCLES", float("nan"))
        src = next(v[0] for v in KERNELS.values() if v[1] == short)
        lines.append(
            f"| {short} | {dur[short]:.1f} | {act / dur[short] / 1e3:.2f} | {100 * mfma:.1f} % | {100 * hit:.1f} % | "
            f"{a['SQ_INSTS_VALU'] / 1e6:.1f} / {a['SQ_INSTS_SALU'] / 1e6:.1f} / {a['SQ_INSTS_MFMA'] / 1e6:.1f} / "
            f"{a['SQ_INSTS_LDS'] / 1e6:.1f} | {100 * a['SQ_LDS_BANK_CONFLICT'] / max(a['SQ_LDS_IDX_ACTIVE'], 1.0):.0f} % | "
            f"{b.get('SQ_ACTIVE_INST_VALU', 0) / wc:.2f} / {b.get('SQ_ACTIVE_INST_SCA', 0) / wc:.2f} / "
            f"{b.get('SQ_ACTIVE_INST_LDS', 0) / wc:.2f} | {b.get('SQ_WAIT_INST_ANY', 0) / wc:.2f} | {source_sha(src)} |")
    os.makedirs(args.out, exist_ok=True)
    with open(os.path.join(args.out, f"counters_{args.workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
