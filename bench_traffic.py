"""Per-launch HBM traffic (and instructions) of a measured kernel from rocprofv3 counter runs of bench.py.

Reads the counter CSVs of a FETCH_SIZE run and a WRITE_SIZE run of bench.py
(with --copy-calibration-mib N), takes the kernels of one measured launch,
scales each counter by what it reads for the run's own device-to-device copies
of N MiB (their true traffic is N MiB read and N MiB written), and writes the
summary that bench.py reports when the kernel sources still match:
  --kind decode  the decode step's two kernels (the split kernel for the
                 workload's group size with the new token's work-groups, and
                 the merge); bench.py's roofline.traffic and valu_roof;
  --kind append  the bulk encode of the long-context workload
                 (bench.py --profile-append); bench.py's append_roofline;
  --kind decode_long  the 131072-token decode's split kernel and merge
                 (bench.py --profile-decode long_t131072);
  --kind decode_ragged  the 32-sequence ragged batch's split kernel and merge
                 (bench.py --profile-decode ragged32_gqa).
With --insts, a third run's instruction counters (SQ_INSTS_VALU, SQ_INSTS_MFMA,
SQ_INSTS_LDS, SQ_INSTS_SALU, SQ_WAVES: wave-level instructions summed over the
chip) go into the same summary; bench.py reports the VALU count against the
VALU issue roof. With --sq, more runs' shader counters (any SQ_* counters,
summed over the chip per dispatch) are tabulated per kernel as well, with the
instructions per 32-slot block of the decode kinds.

    python bench_traffic.py --kind decode|append|decode_long --fetch DIR --write DIR --copy-mib N \\
        --workload W [--insts DIR] [--sq DIR ...] --command "..." --out profiles/<kind>_W_traffic.md
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


def all_counters(run_dirs):
    """{kernel name: {counter: [values of its dispatches]}} over several run dirs."""
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for d in run_dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        for f in files:
            for r in csv.DictReader(open(f)):
                out[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return out


def pick(vals, needle):
    """Counter values of the dispatches of one kernel: `needle` is (demangled, mangled) names or a
    single name (the profiler writes either form, depending on its version and options)."""
    names = needle if isinstance(needle, tuple) else (needle,)
    hits = [v for k, vs in vals.items() if any(n in k for n in names) for v in vs]
    if not hits:
        raise SystemExit(f"no dispatch of a kernel named like {names!r}")
    return hits


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--kind", choices=("decode", "append", "decode_long", "decode_ragged"), default="decode")
    ap.add_argument("--insts", default=None, help="run dir of the instruction-counter pass")
    ap.add_argument("--sq", nargs="*", default=[], help="run dirs of further shader-counter passes")
    ap.add_argument("--command", required=True, help="the two profiling commands, for the record")
    ap.add_argument("--out", required=True)
    a = ap.parse_args()

    from bench import decode_source_digest, encode_source_digest, ROW_BYTES
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
    if a.kind == "decode":
        kernels = (("split", (f"decode_split_kernel<{group}, 3, true>", f"decode_split_kernelILi{group}ELi3ELb1E")),
                   ("merge", ("decode_merge_kernel<true, 32>", "decode_merge_kernelILb1ELi32E")))
        alg = w.num_kv_heads * w.seq_len * 2 * ROW_BYTES
        alg_text = "packed K and V rows, 104 B per token and KV head"
        digest = decode_source_digest()
    elif a.kind == "decode_ragged":
        import numpy as np
        lens = np.asarray(iqinputs.seq_lengths(w), np.int64)
        starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
        kernels = (("split", (f"decode_split_kernel<{group}, 3, false>", f"decode_split_kernelILi{group}ELi3ELb0E")),
                   ("merge", ("decode_merge_kernel<true, 8>", "decode_merge_kernelILb1ELi8E")))
        alg = int(w.num_kv_heads * lens.sum() * 2 * ROW_BYTES)
        alg_text = "packed K and V rows of the batch's tokens, 104 B per token and KV head"
        digest = decode_source_digest()
        # 32-slot blocks the launch streams: each sequence from its 32-aligned start
        ragged_blocks = int(w.num_kv_heads * sum(-(-(int(s) % 32 + int(n)) // 32) for s, n in zip(starts, lens)))
    elif a.kind == "decode_long":
        kernels = (("split", (f"decode_split_kernel<{group}, 3, false>", f"decode_split_kernelILi{group}ELi3ELb0E")),
                   ("merge", ("decode_merge_kernel<true, 32>", "decode_merge_kernelILb1ELi32E")))
        alg = w.num_kv_heads * w.seq_len * 2 * ROW_BYTES
        alg_text = "packed K and V rows, 104 B per token and KV head"
        digest = decode_source_digest()
    else:
        kernels = (("append", ("append_kernel<_Float16, false, false>", "append_kernelIDF16_Lb0ELb0E")),)
        alg = w.num_kv_heads * w.seq_len * 2 * (256 + ROW_BYTES)
        alg_text = "per token, KV head and K or V: 256 B of fp16 in, 48 B of codes and a 4 B norm out"
        digest = encode_source_digest()
    rows = []
    total = 0.0
    for label, needle in kernels:
        f = statistics.mean(pick(fetch, needle)) * f_scale * 1024
        wv = statistics.mean(pick(write, needle)) * w_scale * 1024
        rows.append((label, f, wv))
        total += f + wv
    inst_names = ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_WAVES")
    insts = {}
    if a.insts:
        runs = {c: per_kernel(a.insts, c) for c in inst_names}
        for label, needle in kernels:
            insts[label] = {c: statistics.mean(pick(runs[c], needle)) for c in inst_names}
    lines = [
        f"# HBM traffic{' and instructions' if insts else ''} per {a.kind} launch: {a.workload}",
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
        f"Algorithmic bytes per launch ({alg_text}): {alg:,}.",
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
    if a.sq:
        cs = all_counters(a.sq)
        blocks = (ragged_blocks if a.kind == "decode_ragged" else
                  w.num_kv_heads * w.seq_len // 32 if a.kind != "append" else None)
        for label, needle in kernels:
            names = needle if isinstance(needle, tuple) else (needle,)
            merged = collections.defaultdict(list)
            for k, d in cs.items():
                if any(n in k for n in names):
                    for c, v in d.items():
                        merged[c].extend(v)
            if not merged:
                continue
            lines += ["", f"Shader counters per dispatch, {label} kernel (mean over dispatches; per-block "
                          f"columns divide by the launch's {blocks:,} blocks of 32 slots)" if blocks else
                      f"Shader counters per dispatch, {label} kernel (mean over dispatches)", "",
                      "| counter | per dispatch |" + (" per block |" if blocks else ""),
                      "|---|---|" + ("---|" if blocks else "")]
            for c in sorted(merged):
                v = statistics.mean(merged[c])
                lines.append(f"| {c} | {v:,.0f} |" + (f" {v / blocks:,.1f} |" if blocks else ""))
            if "SQ_LDS_BANK_CONFLICT" in merged and "SQ_LDS_IDX_ACTIVE" in merged:
                bc, act = statistics.mean(merged["SQ_LDS_BANK_CONFLICT"]), statistics.mean(merged["SQ_LDS_IDX_ACTIVE"])
                lines.append(f"\nLDS cycles lost to bank conflicts: {bc / act:.2f} of its active cycles.")
    lines += [
        f"- source_sha256: {digest}",
        "",
    ]
    with open(a.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


if __name__ == "__main__":
    main()
