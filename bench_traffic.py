"""Per-launch HBM traffic of the decode from two rocprofv3 counter runs of bench.py.

Reads the counter CSVs of a FETCH_SIZE run and a WRITE_SIZE run (both of
`bench.py --eager --no-compare --copy-calibration-mib N`), takes the decode
step's two kernels (the split kernel instantiated for the workload's group
size with the new token's work-groups, and the merge), scales each counter by what it
reads for the run's own device-to-device copies of N MiB (their true traffic
is N MiB read and N MiB written), and writes the summary that bench.py reports
as roofline.traffic when the decode sources still match. With --insts, a third
run's instruction counters (SQ_INSTS_VALU, SQ_INSTS_MFMA, SQ_INSTS_LDS,
SQ_INSTS_SALU, SQ_WAVES: wave-level instructions summed over the chip) go into
the same summary; bench.py reports the VALU count against the VALU issue roof.

    python bench_traffic.py --fetch DIR --write DIR --copy-mib N --workload W \\
        [--insts DIR] --command "..." --out profiles/decode_W_traffic.md
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def per_kernel(run_dir: str, counter: str):
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    vals = collections.defaultdict(list)
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return vals


def pick(vals, needle):
    hits = [v for k, vs in vals.items() if needle in k for v in vs]
    if not hits:
        raise SystemExit(f"no dispatch of a kernel named like {needle!r}")
    return hits


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--insts", default=None, help="run dir of the instruction-counter pass")
    ap.add_argument("--command", required=True, help="the two profiling commands, for the record")
    ap.add_argument("--out", required=True)
    a = ap.parse_args()

    from bench import decode_source_digest, ROW_BYTES
    import iqinputs

    fetch, write = per_kernel(a.fetch, "FETCH_SIZE"), per_kernel(a.write, "WRITE_SIZE")
    copy_kib = a.copy_mib * 1024.0
    # the calibration copies are the largest copy-kernel dispatches of each run
    f_copy = sorted(pick(fetch, "copyBuffer"))[-3:]
    w_copy = sorted(pick(write, "copyBuffer"))[-3:]
    f_scale = copy_kib / statistics.mean(f_copy)
    w_scale = copy_kib / statistics.mean(w_copy)
    w = iqinputs.WORKLOADS[a.workload]
    group = w.num_q_heads // w.num_kv_heads
    rows = []
    total = 0.0
    for label, needle in (("split", f"decode_split_kernel<{group}, 3, true>"), ("merge", "decode_merge_kernel<true>")):
        f = statistics.mean(pick(fetch, needle)) * f_scale * 1024
        wv = statistics.mean(pick(write, needle)) * w_scale * 1024
        rows.append((label, f, wv))
        total += f + wv
    alg = w.num_kv_heads * w.seq_len * 2 * ROW_BYTES
    inst_names = ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_WAVES")
    insts = {}
    if a.insts:
        runs = {c: per_kernel(a.insts, c) for c in inst_names}
        for label, needle in (("split", f"decode_split_kernel<{group}, 3, true>"),
                              ("merge", "decode_merge_kernel<true>")):
            insts[label] = {c: statistics.mean(pick(runs[c], needle)) for c in inst_names}
    lines = [
        f"# HBM traffic{' and instructions' if insts else ''} per decode launch: {a.workload}",
        "",
        f"Counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch){' and the instruction counters' if insts else ''}, "
        f"one rocprofv3 run each:",
        "",
        "```",
        a.command,
        "```",
        "",
        f"Calibration: the runs end with {a.copy_mib} MiB device-to-device copies; the counters read "
        f"{statistics.mean(f_copy):.1f} KiB fetched and {statistics.mean(w_copy):.1f} KiB written per copy, "
        f"so the scale factors are fetch x{f_scale:.4f}, write x{w_scale:.4f}.",
        "",
        "| kernel | fetched bytes | written bytes |",
        "|---|---|---|",
    ]
    for label, f, wv in rows:
        lines.append(f"| {label} | {f:,.0f} | {wv:,.0f} |")
    lines += [
        "",
        f"Algorithmic bytes per launch (packed K and V rows, 104 B per token and KV head): {alg:,}.",
        f"Measured / algorithmic: {total / alg:.3f}.",
        "",
        f"- hbm_bytes_per_launch: {total:.0f}",
        f"- fetch_scale: {f_scale:.6f}",
        f"- write_scale: {w_scale:.6f}",
    ]
    if insts:
        lines[-4:-4] = [
            "",
            "Instructions per dispatch (wave-level, summed over the chip):",
            "",
            "| kernel | " + " | ".join(inst_names) + " |",
            "|---|" + "---|" * len(inst_names),
        ] + [f"| {label} | " + " | ".join(f"{v[c]:,.0f}" for c in inst_names) + " |" for label, v in insts.items()]
        lines += [
            f"- valu_insts_per_launch: {sum(v['SQ_INSTS_VALU'] for v in insts.values()):.0f}",
            f"- mfma_insts_per_launch: {sum(v['SQ_INSTS_MFMA'] for v in insts.values()):.0f}",
        ]
    lines += [
        f"- decode_source_sha256: {decode_source_digest()}",
        "",
    ]
    with open(a.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


if __name__ == "__main__":
    main()
