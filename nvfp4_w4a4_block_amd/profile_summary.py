"""Summaries of rocprofv3 runs of bench.py, as committed under profiles/.

    python -m nvfp4_w4a4_block_amd.profile_summary trace <kernel_stats.csv> <out.md> \
        --title TEXT --command TEXT [--bytes B | --flops F [--peak-tflops P]] [--kernel SUBSTR]
    python -m nvfp4_w4a4_block_amd.profile_summary traffic <fetch.csv> <write.csv> <out.json> \
        --kernel SUBSTR --sources FILE... --command TEXT --command TEXT [--copy-mib 128]
    python -m nvfp4_w4a4_block_amd.profile_summary counters <pass.csv>... <out.md> \
        --title TEXT --command TEXT... --kernel SUBSTR=LABEL... [--cus 256]

`trace` turns the per-kernel statistics of `rocprofv3 --kernel-trace --stats
--output-format csv` into a markdown table (and, with --bytes, the achieved
GB/s of the named kernel, or with --flops its TFLOP/s against a matrix-core
peak).  `traffic` reads two `rocprofv3 --pmc FETCH_SIZE`
/ `--pmc WRITE_SIZE` counter files of a bench run made with
--copy-reference-mib, scales each counter by what it reads for that plain copy
of known size (the last three copy dispatches), and writes the HBM bytes per
launch of the named kernel together with a SHA-256 of the kernel's sources;
bench.py reports the figure only while those sources are unchanged.
`counters` merges the `rocprofv3 --pmc` counter files of several passes over
the same command (one pass per counter set, since one pass holds at most
eight SQ counters), averages each counter over the dispatches of each named
kernel, and derives the matrix-core busy fraction, the instruction mix per
MFMA, the LDS bank-conflict share and the share of wave time spent waiting.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def sources_sha256(sources) -> str:
    h = hashlib.sha256()
    for src in sources:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def trace(args) -> None:
    rows = list(csv.DictReader(open(args.stats)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"# {args.title}", "", "Command (repository root, MI355X):", "", "```", args.command, "```", ""]
    if args.bench_json:
        # the benchmark's own line from the profiled process: its HIP-event timings of the
        # same launches the trace below records
        with open(args.bench_json) as f:
            rec = json.loads([ln for ln in f if ln.startswith("{")][-1])
        rl = rec.get("roofline", {})
        out += [f"Same process (bench.py's HIP events over the timed region, under the profiler): "
                f"{rec['ms_per_step'] * 1e3:,.2f} us per step, {rl.get('us_per_launch', float('nan')):,.2f} us "
                f"per launch of `{rl.get('kernel', '?')}`.", ""]
    if args.bytes and args.kernel:
        k = [r for r in rows if args.kernel in r["Name"]]
        if k:
            avg = float(k[0]["AverageNs"])
            out += [f"Algorithmic bytes per launch of `{args.kernel}`: {args.bytes:,}; "
                    f"average {avg:,.1f} ns -> {args.bytes / avg:,.1f} GB/s "
                    f"({100 * args.bytes / avg / 8000:.1f}% of 8 TB/s).", ""]
    if args.flops and args.kernel:
        k = [r for r in rows if args.kernel in r["Name"]]
        if k:
            avg = float(k[0]["AverageNs"])
            tf = args.flops / avg / 1e3
            out += [f"Algorithmic flops per launch of `{args.kernel}`: {args.flops:,}; "
                    f"average {avg:,.1f} ns -> {tf:,.1f} TFLOP/s "
                    f"({100 * tf / args.peak_tflops:.1f}% of {args.peak_tflops:,.0f} TFLOP/s).", ""]
    out += ["| Name | Calls | Total (ns) | Average (ns) | Percent | Min (ns) | Max (ns) |",
            "| :-- | --: | --: | --: | --: | --: | --: |"]
    for r in rows:
        out.append(f"| {r['Name'][:150]} | {r['Calls']} | {float(r['TotalDurationNs']):.0f} | "
                   f"{float(r['AverageNs']):.1f} | {float(r['Percentage']):.2f} | {float(r['MinNs']):.0f} | "
                   f"{float(r['MaxNs']):.0f} |")
    with open(args.out, "w") as f:
        f.write("\n".join(out) + "\n")


def _per_kernel(path: str, counter: str):
    """Counter values (KiB per dispatch) grouped as (kernel dispatches, copy dispatches)."""
    recs = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    recs.sort(key=lambda r: int(r["Dispatch_Id"]))
    return recs


def traffic(args) -> None:
    res = {}
    for counter, path in (("FETCH_SIZE", args.fetch), ("WRITE_SIZE", args.write)):
        recs = _per_kernel(path, counter)
        kern = [float(r["Counter_Value"]) for r in recs if args.kernel in r["Kernel_Name"]]
        copies = [float(r["Counter_Value"]) for r in recs if "copyBuffer" in r["Kernel_Name"]][-3:]
        if not kern or len(copies) < 3:
            sys.exit(f"{path}: {len(kern)} dispatches of {args.kernel!r}, {len(copies)} reference copies")
        res[counter] = (statistics.mean(kern), statistics.mean(copies), len(kern))
    ref_kib = args.copy_mib * 1024.0
    f_kib, f_ref, n = res["FETCH_SIZE"]
    w_kib, w_ref, _ = res["WRITE_SIZE"]
    f_scale, w_scale = ref_kib / f_ref, ref_kib / w_ref
    rec = {
        "kernel": args.kernel,
        "sources": args.sources,
        "sources_sha256": sources_sha256(args.sources),
        "dispatches": n,
        "fetch_size_kib_per_dispatch": round(f_kib, 1),
        "write_size_kib_per_dispatch": round(w_kib, 1),
        "copy_reference": f"device copy of {args.copy_mib} MiB: FETCH_SIZE {f_ref:.1f} KiB, "
                          f"WRITE_SIZE {w_ref:.1f} KiB",
        "fetch_scale": round(f_scale, 4),
        "write_scale": round(w_scale, 4),
        "traffic_bytes_per_launch": int(round((f_kib * f_scale + w_kib * w_scale) * 1024)),
        "commands": args.command,
    }
    with open(args.out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")


def _ratio(d, num, den, scale=1.0):
    if num in d and den in d and d[den]:
        return scale * d[num] / d[den]
    return None


def counters(args) -> None:
    labels = [kv.split("=", 1) for kv in args.kernel]
    per = {lab: {} for _, lab in labels}
    n_disp = {lab: {} for _, lab in labels}
    dur = {lab: [] for _, lab in labels}
    for path in args.passes:
        vals = {lab: {} for _, lab in labels}
        for r in csv.DictReader(open(path)):
            for sub, lab in labels:
                if sub in r["Kernel_Name"]:
                    vals[lab].setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                    if r["Counter_Name"] == next(iter(vals[lab])):
                        dur[lab].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        for lab, d in vals.items():
            for c, v in d.items():
                per[lab][c] = statistics.mean(v)
                n_disp[lab][c] = len(v)
    cus, simds = args.cus, 4 * args.cus
    out = [f"# {args.title}", "", "Commands (one pass per counter set; repository root, MI355X):", ""]
    out += ["```", *args.command, "```", ""]
    for sub, lab in labels:
        d = per[lab]
        if not d:
            sys.exit(f"no dispatches of {sub!r}")
        out += [f"## {lab}", "", f"Kernel: `{sub}`; mean over {min(n_disp[lab].values())} to "
                f"{max(n_disp[lab].values())} dispatches per counter; mean dispatch duration under the "
                f"counter passes {statistics.mean(dur[lab]) / 1e3:.1f} us.", ""]
        out += ["| Counter | Mean per dispatch |", "| :-- | --: |"]
        out += [f"| {c} | {v:,.0f} |" for c, v in sorted(d.items())]
        derived = []
        busy = None
        if "SQ_VALU_MFMA_BUSY_CYCLES" in d and d.get("SQ_BUSY_CU_CYCLES"):
            busy = (d["SQ_VALU_MFMA_BUSY_CYCLES"] / simds) / (d["SQ_BUSY_CU_CYCLES"] / cus)
            derived.append(("matrix-core busy: SQ_VALU_MFMA_BUSY_CYCLES per SIMD / SQ_BUSY_CU_CYCLES per CU",
                            f"{100 * busy:.1f}%"))
        if "SQ_INSTS_VALU" in d and d.get("SQ_INSTS_MFMA"):
            derived.append(("non-MFMA VALU instructions per MFMA: (SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA",
                            f"{(d['SQ_INSTS_VALU'] - d['SQ_INSTS_MFMA']) / d['SQ_INSTS_MFMA']:.2f}"))
        for name, num in (("SALU", "SQ_INSTS_SALU"), ("LDS", "SQ_INSTS_LDS"), ("vector-memory read", "SQ_INSTS_VMEM_RD")):
            v = _ratio(d, num, "SQ_INSTS_MFMA")
            if v is not None:
                derived.append((f"{name} instructions per MFMA: {num} / SQ_INSTS_MFMA", f"{v:.2f}"))
        v = _ratio(d, "SQ_LDS_BANK_CONFLICT", "SQ_BUSY_CU_CYCLES", 100)
        if v is not None:
            derived.append(("LDS bank-conflict cycles / CU busy cycles", f"{v:.1f}%"))
        for num in ("SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_WAIT_INST_LDS"):
            v = _ratio(d, num, "SQ_WAVE_CYCLES", 100)
            if v is not None:
                derived.append((f"{num} / SQ_WAVE_CYCLES", f"{v:.1f}%"))
        if "SQ_INSTS_VALU_MFMA_MOPS_F16" in d:
            derived.append(("f16 matrix flops per dispatch: 512 x SQ_INSTS_VALU_MFMA_MOPS_F16",
                            f"{512 * d['SQ_INSTS_VALU_MFMA_MOPS_F16']:.4g}"))
        if derived:
            out += ["", "| Derived | Value |", "| :-- | --: |"]
            out += [f"| {k} | {v} |" for k, v in derived]
        out.append("")
    with open(args.out, "w") as f:
        f.write("\n".join(out) + "\n")


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats")
    t.add_argument("out")
    t.add_argument("--title", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--bytes", type=int, default=0)
    t.add_argument("--flops", type=int, default=0)
    t.add_argument("--peak-tflops", type=float, default=2500.0)
    t.add_argument("--kernel", default="")
    t.add_argument("--bench-json", default="")
    r = sub.add_parser("traffic")
    r.add_argument("fetch")
    r.add_argument("write")
    r.add_argument("out")
    r.add_argument("--kernel", required=True)
    r.add_argument("--sources", nargs="+", required=True)
    r.add_argument("--command", action="append", required=True)
    r.add_argument("--copy-mib", type=int, default=128)
    c = sub.add_parser("counters")
    c.add_argument("passes", nargs="+")
    c.add_argument("out")
    c.add_argument("--title", required=True)
    c.add_argument("--command", action="append", required=True)
    c.add_argument("--kernel", action="append", required=True, help="SUBSTR=LABEL")
    c.add_argument("--cus", type=int, default=256)
    a = ap.parse_args()
    {"trace": trace, "traffic": traffic, "counters": counters}[a.cmd](a)


if __name__ == "__main__":
    main()
