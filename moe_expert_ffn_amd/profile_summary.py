"""Summaries of rocprofv3 CSV output for the expert-layer kernels.

  python -m moe_expert_ffn_amd.profile_summary stats  <kernel_stats.csv>
  python -m moe_expert_ffn_amd.profile_summary traffic <fetch.csv> <write.csv> \
        <copy_fetch.csv> <copy_write.csv> <copy_bytes> <kernel>

`stats` prints a markdown table of the library's kernels (calls, average and
total duration).  Kernel names are shortened to k_stream<SrcX> for the
persistent GEMM kernels (SrcX names the stage) and to the bare name otherwise;
`traffic` takes such a short name.  `traffic` prints, for one kernel, the average FETCH_SIZE and
WRITE_SIZE per dispatch (KiB), the calibration of both counters against a
plain elementwise copy of `copy_bytes` bytes read and written (the copy's own
dispatch is the one with the largest reading), and the calibrated HBM bytes
per dispatch.
"""
from __future__ import annotations

import collections
import csv
import re
import sys

STAGE_OF = {"k_stream<SrcFc1>": "fwd.fc1", "k_stream<SrcFc2>": "fwd.fc2",
            "k_stream<SrcFc1Fp8>": "fwd.fc1", "k_stream<SrcFc2Fp8>": "fwd.fc2",
            "k_stream<SrcDaFp8>": "bwd.dA", "k_stream<SrcDxFp8>": "bwd.dX",
            "k_quant_tok": "bwd.dA (D) + bwd.dW (dZ)",
            "k_stream<SrcDa>": "bwd.dA", "k_stream<SrcDx>": "bwd.dX", "k_stream<SrcDwT>": "bwd.dW",
            "k_fc1": "fwd.fc1", "k_fc2": "fwd.fc2", "k_bwd_da": "bwd.dA", "k_bwd_dx": "bwd.dX",
            "k_bwd_dw": "bwd.dW", "k_bwd_reduce": "bwd.reduce",
            "k_combine": "fwd.combine + bwd.combine", "k_sched": "fwd.sched + bwd.sched",
            "k_slot_gate": "fwd.sched + bwd.sched", "k_plan": "plan (fwd + bwd)",
            "k_route_count": "route", "k_route_scan": "route", "k_route_slot": "route"}


def short(name: str) -> str:
    """k_stream<SrcX> for the persistent GEMM kernels, the bare kernel name otherwise."""
    m = re.search(r"k_stream<moe::(\w+?)(T<(true|false)>)?[,<>]", name)
    if m:
        return f"k_stream<{m.group(1)}{'Fp8' if m.group(3) == 'true' else ''}>"
    m = re.search(r"moe::(\w+)", name)
    return m.group(1) if m else name[:60]


def stats(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["| kernel | stage | calls | avg us | total us |", "|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        if "moe::" not in r["Name"]:
            continue
        k = short(r["Name"])
        out.append(f"| {k} | {STAGE_OF.get(k, '')} | {r['Calls']} | "
                   f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['TotalDurationNs']) / 1e3:.1f} |")
    return "\n".join(out)


def per_kernel(path: str):
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        agg[short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return agg


def copy_reading(path: str) -> float:
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))]
    return max(vals)


def traffic(fetch: str, write: str, cfetch: str, cwrite: str, copy_bytes: int, kernel: str) -> str:
    f = per_kernel(fetch)
    w = per_kernel(write)
    key = next(k for k in f if k == kernel)
    fk = sum(f[key]) / len(f[key])
    wk = sum(w[key]) / len(w[key])
    sf = copy_bytes / (copy_reading(cfetch) * 1024.0)
    sw = copy_bytes / (copy_reading(cwrite) * 1024.0)
    total = fk * 1024.0 * sf + wk * 1024.0 * sw
    return (f"kernel {key}: dispatches {len(f[key])}; FETCH_SIZE {fk:.1f} KiB, WRITE_SIZE {wk:.1f} KiB "
            f"per dispatch\ncopy calibration: fetch x{sf:.4f}, write x{sw:.4f} "
            f"({copy_bytes} bytes read and written)\ncalibrated HBM traffic per dispatch: "
            f"{total:.0f} bytes (read {fk * 1024.0 * sf:.0f}, write {wk * 1024.0 * sw:.0f})")


def main(argv):
    if argv[1] == "stats":
        print(stats(argv[2]))
    elif argv[1] == "traffic":
        print(traffic(argv[2], argv[3], argv[4], argv[5], int(argv[6]), argv[7]))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv)
