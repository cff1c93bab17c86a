"""Summaries of rocprofv3 CSV output for the expert-layer kernels.

  python -m moe_expert_ffn_amd.profile_summary stats  <kernel_stats.csv>
  python -m moe_expert_ffn_amd.profile_summary traffic <fetch.csv> <write.csv> \
        <copy_fetch.csv> <copy_write.csv> <copy_bytes> <kernel>
  python -m moe_expert_ffn_amd.profile_summary mfma <counter_collection.csv>

`stats` prints a markdown table of the library's kernels (calls, average and
total duration).  Kernel names are shortened to k_stream<SrcX> for the
persistent GEMM kernels (SrcX names the stage) and to the bare name otherwise;
`traffic` takes such a short name.  `traffic` prints, for one kernel, the average FETCH_SIZE and
WRITE_SIZE per dispatch (KiB), the calibration of both counters against a
plain elementwise copy of `copy_bytes` bytes read and written (the copy's own
dispatch is the one with the largest reading), and the calibrated HBM bytes
per dispatch.  `mfma` takes a `--pmc MfmaUtil MfmaFlopsBF16` run and prints,
per GEMM kernel, the mean MfmaUtil, the executed MFMA work and the dispatch
duration (its own timestamps; counter runs serialise dispatches).  The work
is `MfmaFlopsBF16`, priced against the bf16 peak, or, for kernels that run
the fp8 MFMA, 512 · SQ_INSTS_VALU_MFMA_MOPS_F8 (the run then names that
counter in place of MfmaFlopsBF16), priced against the fp8 peak.
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
            "k_stream<SrcDwTFp8>": "bwd.dW",
            "k_stream2<Fc1+Fc2>": "fwd.fc1+fc2", "k_stream2<Fc1+Fc2Fp8>": "fwd.fc1+fc2",
            "k_stream2<Da+Dx>": "bwd.dA+dX", "k_stream2<Da+DxFp8>": "bwd.dA+dX",
            "k_fc1": "fwd.fc1", "k_fc2": "fwd.fc2", "k_bwd_da": "bwd.dA", "k_bwd_dx": "bwd.dX",
            "k_bwd_dw": "bwd.dW", "k_bwd_reduce": "bwd.reduce",
            "k_combine": "fwd.combine + bwd.combine", "k_sched": "fwd.sched + bwd.sched",
            "k_plan": "plan (fwd + bwd)",
            "k_stream<SrcFc1F8>": "fwd.fc1 (fp8 MFMA)", "k_stream<SrcFc2F8>": "fwd.fc2 (fp8 MFMA)",
            "k_stream<SrcDaF8>": "bwd.dA (fp8 MFMA)", "k_stream<SrcDxF8>": "bwd.dX (fp8 MFMA)",
            "k_quant_act": "fp8 MFMA: fwd.fc1 (x, A), bwd.dA (dy)",
            "k_swiglu_bwd_q": "bwd.dA (dZ, P, dZ's e4m3 rows; fp8 MFMA)",
            "k_route_count": "route", "k_route_scan": "route", "k_route_slot": "route"}


def short(name: str) -> str:
    """k_stream<SrcX> for the persistent GEMM kernels (SrcXFp8 with e4m3
    weights), k_stream2<X+Y> for a two-phase launch, the bare kernel name
    otherwise."""
    fp8 = lambda b: "Fp8" if b == "true" else ""
    m = re.search(r"k_stream2<moe::FlowProducer<moe::Src(\w+?)T<(true|false)\b.*?"
                  r"FlowConsumer<moe::Src(\w+?)T<", name)
    if m:
        return f"k_stream2<{m.group(1)}+{m.group(3)}{fp8(m.group(2))}>"
    m = re.search(r"k_stream<moe::SrcDwT<moe::GemmCfg<[^>]*>, (true|false)>", name)
    if m:
        return f"k_stream<SrcDwT{fp8(m.group(1))}>"
    m = re.search(r"k_stream<moe::Src(\w+?)T<(true|false)\b", name)
    if m:
        return f"k_stream<Src{m.group(1)}{fp8(m.group(2))}>"
    m = re.search(r"k_stream<moe::Src(\w+F8),", name)
    if m:
        return f"k_stream<Src{m.group(1)}>"
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


PEAK_BF16_TFLOPS = 2516.6
PEAK_FP8_TFLOPS = 5033.2


def mfma(path: str) -> str:
    util, flops, dur = (collections.defaultdict(list) for _ in range(3))
    kind = {}
    for r in csv.DictReader(open(path)):
        if "moe::" not in r["Kernel_Name"]:
            continue
        k = short(r["Kernel_Name"])
        if r["Counter_Name"] == "MfmaUtil":
            util[k].append(float(r["Counter_Value"]))
            dur[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        elif r["Counter_Name"] == "MfmaFlopsBF16":
            flops[k].append(float(r["Counter_Value"]))
            kind[k] = "bf16"
        elif r["Counter_Name"] == "SQ_INSTS_VALU_MFMA_MOPS_F8":
            flops[k].append(512.0 * float(r["Counter_Value"]))
            kind[k] = "fp8"
    peak = {"bf16": PEAK_BF16_TFLOPS, "fp8": PEAK_FP8_TFLOPS}
    out = ["| kernel | dispatches | MfmaUtil % | MFMA | executed GFLOP / launch | us / launch "
           "| TFLOP/s | % of that MFMA's peak |", "|---|---|---|---|---|---|---|---|"]
    for k in sorted(util, key=lambda k: -sum(dur[k]) / len(dur[k])):
        if not flops.get(k) or sum(flops[k]) == 0:
            continue
        u, f, t = (sum(v) / len(v) for v in (util[k], flops[k], dur[k]))
        tf = f / (t * 1e-6) / 1e12
        out.append(f"| {k} | {len(util[k])} | {u:.1f} | {kind[k]} | {f / 1e9:.1f} | {t:.1f} | "
                   f"{tf:.1f} | {100 * tf / peak[kind[k]]:.1f} of {peak[kind[k]]:,.1f} |")
    return "\n".join(out)


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
    elif argv[1] == "mfma":
        print(mfma(argv[2]))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv)
