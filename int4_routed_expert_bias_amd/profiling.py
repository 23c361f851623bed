"""Summaries of rocprofv3 output for the kernels of this library.

Used on the measurement side only (never by the compute path):

  python -m int4_routed_expert_bias_amd.profiling trace <run_kernel_trace.csv> --command "..."
      markdown table of per-kernel durations (avg / min / max, grid, registers)

  python -m int4_routed_expert_bias_amd.profiling counters <pmc dir> [<pmc dir> ...] \
      --match <kernel name substring> [--match ...]
      markdown table of the per-dispatch mean of every counter collected
      for the matching kernels, with the ratios derived from them

  python -m int4_routed_expert_bias_amd.profiling traffic \
      --fetch <pmc dir> --write <pmc dir> --copy-fetch <pmc dir> --copy-write <pmc dir> \
      --kernel <label> --match <trace name substring> [--match ...] --workload <name> \
      --out profiles/traffic.json
      HBM bytes per launch of one kernel from the FETCH_SIZE and WRITE_SIZE
      counters (KiB per dispatch), each scaled by the factor that maps the
      same counter on a plain device copy of known size to its true bytes.

The traffic record carries a hash of the kernel sources it was measured on;
bench.py reports it only while the sources are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30  # the calibration copy moves 1 GiB each way
COPY_KERNEL = "copyBuffer"  # the runtime blit kernel behind a device-to-device tensor copy


ALL_SOURCES = ("expert_f32.hip", "expert_i8.hip", "expert_i8v.hip", "stream.h", "common.h",
               "route.hip", "route_tokens.h", "union_wave.h", "union.hip", "combine.hip")


def kernel_sources(kernel: str):
    """The sources a kernel's traffic depends on (its translation unit and
    the headers it includes), so that a traffic record stays valid while
    only other kernels change."""
    if kernel.startswith("ggemm") or kernel.startswith("quant_rows"):
        return ("expert_i8.hip", "common.h")
    if "i8v" in kernel:
        return ("expert_i8v.hip", "stream.h", "route_tokens.h", "union_wave.h", "common.h")
    if kernel.startswith(("gateup_", "down_")):
        return ("expert_f32.hip", "stream.h", "route_tokens.h", "union_wave.h", "common.h")
    return ALL_SOURCES


def source_hash(files=ALL_SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(HERE, "csrc", f), "rb") as fp:
            h.update(fp.read())
    return h.hexdigest()[:16]


def _rows(path_or_dir: str, name: str):
    p = path_or_dir
    if os.path.isdir(p):
        hits = glob.glob(os.path.join(p, "**", name), recursive=True)
        if not hits:
            raise FileNotFoundError(f"{name} under {p}")
        p = hits[0]
    with open(p) as f:
        return list(csv.DictReader(f))


def trace_table(trace_csv: str, skip=("spin_kernel",)) -> str:
    rows = _rows(trace_csv, "*kernel_trace.csv")
    per = {}
    for r in rows:
        name = r["Kernel_Name"]
        if any(s in name for s in skip):
            continue
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        e = per.setdefault(name, {"d": [], "grid": f"{r['Grid_Size_X']}x{r['Grid_Size_Y']}",
                                  "block": r["Workgroup_Size_X"], "vgpr": r["VGPR_Count"],
                                  "agpr": r.get("Accum_VGPR_Count", "0"),
                                  "lds": r["LDS_Block_Size"]})
        e["d"].append(d)
    out = ["| kernel | calls | avg us | min us | max us | grid | block | VGPR | AGPR | LDS B |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    for name, e in sorted(per.items(), key=lambda kv: -statistics.mean(kv[1]["d"]) * len(kv[1]["d"])):
        d = e["d"]
        out.append(f"| `{name[:90]}` | {len(d)} | {statistics.mean(d):.2f} | {min(d):.2f} | "
                   f"{max(d):.2f} | {e['grid']} | {e['block']} | {e['vgpr']} | {e['agpr']} | "
                   f"{e['lds']} |")
    return "\n".join(out)


def pmc_avg(pmc_dir: str, counter: str, kernel_sub: str) -> float:
    rows = _rows(pmc_dir, "*counter_collection.csv")
    vals = [float(r["Counter_Value"]) for r in rows
            if r["Counter_Name"] == counter and kernel_sub in r["Kernel_Name"]]
    if not vals:
        raise ValueError(f"no {counter} rows for kernels matching {kernel_sub!r}")
    return statistics.mean(vals)


def counter_table(dirs, matches) -> str:
    """Per-dispatch means of every counter in the counter-collection CSVs
    under dirs, for the kernels whose names contain one of matches."""
    per = {}
    for d in dirs:
        for r in _rows(d, "*counter_collection.csv"):
            m = next((mm for mm in matches if mm in r["Kernel_Name"]), None)
            if m is None:
                continue
            per.setdefault(m, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    names = sorted({c for v in per.values() for c in v})
    out = ["| counter | " + " | ".join(f"`{m}`" for m in matches) + " |",
           "|---|" + "---|" * len(matches)]
    for c in names:
        cells = []
        for m in matches:
            v = per.get(m, {}).get(c)
            cells.append(f"{statistics.mean(v):,.0f} (n={len(v)})" if v else "-")
        out.append(f"| {c} | " + " | ".join(cells) + " |")

    def mean(m, c):
        v = per.get(m, {}).get(c)
        return statistics.mean(v) if v else None
    derived = []
    for m in matches:
        valu, mfma = mean(m, "SQ_INSTS_VALU"), mean(m, "SQ_INSTS_MFMA")
        busy, gui = mean(m, "SQ_VALU_MFMA_BUSY_CYCLES"), mean(m, "GRBM_GUI_ACTIVE")
        conf, lds = mean(m, "SQ_LDS_BANK_CONFLICT"), mean(m, "SQ_ACTIVE_INST_LDS")
        row = []
        if valu and mfma:
            row.append(f"VALU instructions per MFMA {valu / mfma:.2f}")
        if conf is not None and lds:
            row.append(f"LDS bank-conflict cycles per LDS-active cycle {conf / lds:.3f}")
        if busy and gui:
            row.append(f"SQ_VALU_MFMA_BUSY_CYCLES / GRBM_GUI_ACTIVE {busy / gui:.1f}")
        if row:
            derived.append(f"- `{m}`: " + "; ".join(row))
    return "\n".join(out) + ("\n\nDerived:\n\n" + "\n".join(derived) if derived else "")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("trace_csv")
    t.add_argument("--command", default="")
    cn = sub.add_parser("counters")
    cn.add_argument("dirs", nargs="+")
    cn.add_argument("--match", action="append", required=True)
    cn.add_argument("--command", action="append", default=[])
    tr = sub.add_parser("traffic")
    for a in ("fetch", "write", "copy_fetch", "copy_write", "kernel", "workload", "out"):
        tr.add_argument("--" + a.replace("_", "-"), required=True)
    tr.add_argument("--match", action="append", required=True)
    tr.add_argument("--bytes-per-launch", type=float, default=None,
                    help="algorithmic bytes of one launch (for the ratio in the record)")
    args = ap.parse_args(argv)
    if args.cmd == "trace":
        if args.command:
            print("Command:\n\n```\n" + args.command + "\n```\n")
        print(trace_table(args.trace_csv))
        return
    if args.cmd == "counters":
        if args.command:
            print("Commands:\n\n```\n" + "\n".join(args.command) + "\n```\n")
        print(counter_table(args.dirs, args.match))
        return
    # several --match: kernels launched together for one step (the grouped
    # GEMM's launches over its tile lists), their per-launch means added
    f_kib = sum(pmc_avg(args.fetch, "FETCH_SIZE", m) for m in args.match)
    w_kib = sum(pmc_avg(args.write, "WRITE_SIZE", m) for m in args.match)
    cf_kib = pmc_avg(args.copy_fetch, "FETCH_SIZE", COPY_KERNEL)
    cw_kib = pmc_avg(args.copy_write, "WRITE_SIZE", COPY_KERNEL)
    f_scale = COPY_BYTES / (cf_kib * 1024.0)
    w_scale = COPY_BYTES / (cw_kib * 1024.0)
    rec = {
        "kernel": args.kernel, "match": args.match, "workload": args.workload,
        "sources": list(kernel_sources(args.kernel)),
        "source_hash": source_hash(kernel_sources(args.kernel)),
        "fetch_kib_per_launch": round(f_kib, 1), "write_kib_per_launch": round(w_kib, 1),
        "copy_fetch_kib": round(cf_kib, 1), "copy_write_kib": round(cw_kib, 1),
        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
        "hbm_bytes_per_launch": round(f_kib * 1024.0 * f_scale + w_kib * 1024.0 * w_scale),
    }
    if args.bytes_per_launch:
        rec["algorithmic_bytes_per_launch"] = round(args.bytes_per_launch)
        rec["traffic_over_algorithmic"] = round(rec["hbm_bytes_per_launch"] / args.bytes_per_launch, 3)
    db = {}
    if os.path.exists(args.out):
        with open(args.out) as fp:
            db = json.load(fp)
    db[f"{args.workload}:{args.kernel}"] = rec
    with open(args.out, "w") as fp:
        json.dump(db, fp, indent=1, sort_keys=True)
        fp.write("\n")
    json.dump(rec, sys.stdout, indent=1)
    print()


if __name__ == "__main__":
    main()
