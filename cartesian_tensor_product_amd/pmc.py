"""Summaries of rocprofv3 counter runs (``rocprofv3 --pmc ... --output-format csv``).

    python -m cartesian_tensor_product_amd.pmc table DIR [DIR ...]
        per-kernel mean of every counter in the runs' *_counter_collection.csv

    python -m cartesian_tensor_product_amd.pmc stats DIR
        per-kernel durations from a ``--kernel-trace --stats`` run (its stats
        CSV, or its SQLite database) as markdown

    python -m cartesian_tensor_product_amd.pmc issue DIR [DIR ...]
        per-kernel instruction mix from runs holding SQ_WAVES, SQ_INSTS_VALU,
        SQ_INSTS_VALU_FMA_F32, SQ_INSTS_VALU_MUL_F32, SQ_INSTS_LDS,
        SQ_INSTS_SALU, SQ_INSTS_VMEM_RD, SQ_WAIT_INST_ANY (any subset; the
        runs are merged by kernel name)

    python -m cartesian_tensor_product_amd.pmc traffic --fetch DIR --write DIR \
        --copy-fetch DIR --copy-write DIR --copy-mib 512 --kernel NAME --out FILE
        HBM-side bytes per launch of one kernel: FETCH_SIZE and WRITE_SIZE
        (KiB per dispatch) each scaled by what the same counter reads for a
        device-to-device copy of known size, written as JSON together with the
        hash of the edge-kernel sources it was taken on.

Host-side tooling only: it reads CSV files and touches no GPU.
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Sources of the edge-convolution kernels; a traffic record is valid only for
# the sources it was measured on.
EDGE_KERNEL_SOURCES = ["cartesian_tensor_product_amd/csrc/fc_conv_kernels.h",
                       "cartesian_tensor_product_amd/csrc/fc_common.h",
                       "cartesian_tensor_product_amd/csrc/fc_conv.hip",
                       "cartesian_tensor_product_amd/csrc/generated/fc_tables.h"]


def edge_kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in EDGE_KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load(run_dir: str) -> dict:
    """{kernel name (without arguments): {counter: [value per dispatch]}}"""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *counter_collection.csv under {run_dir}")
    agg: dict = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in files:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                name = kernel_name(r["Kernel_Name"])
                agg[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return agg


def mean(v):
    return sum(v) / len(v)


def find(agg: dict, kernel: str):
    hits = [k for k in agg if kernel in k]
    if not hits:
        raise KeyError(f"kernel {kernel!r} not in run; kernels: {sorted(agg)}")
    return agg[sorted(hits, key=len)[0]]


def table(dirs):
    out = []
    for d in dirs:
        agg = load(d)
        out.append(f"### {os.path.basename(os.path.normpath(d))}\n")
        counters = sorted({c for cs in agg.values() for c in cs})
        out.append("| kernel | dispatches | " + " | ".join(counters) + " |")
        out.append("|---|---|" + "---|" * len(counters))
        for k, cs in sorted(agg.items()):
            n = max(len(v) for v in cs.values())
            vals = [f"{mean(cs[c]):.6g}" if c in cs else "" for c in counters]
            out.append(f"| `{k[:90]}` | {n} | " + " | ".join(vals) + " |")
        out.append("")
    return "\n".join(out)


def issue(dirs) -> str:
    merged: dict = collections.defaultdict(dict)
    for d in dirs:
        for k, cs in load(d).items():
            for c, v in cs.items():
                merged[k][c] = mean(v)
    cols = [("SQ_INSTS_VALU", "VALU"), ("SQ_INSTS_VALU_FMA_F32", "FMA_F32"), ("SQ_INSTS_VALU_MUL_F32", "MUL_F32"),
            ("SQ_INSTS_LDS", "LDS"), ("SQ_INSTS_SALU", "SALU"), ("SQ_INSTS_VMEM_RD", "VMEM_RD"),
            ("SQ_WAIT_INST_ANY", "WAIT_INST_ANY")]
    out = ["| kernel | waves | " + " | ".join(f"{n} / wave" for _, n in cols) + " | VALU total |",
           "|---|---|" + "---|" * (len(cols) + 1)]
    for k, cs in sorted(merged.items()):
        w = cs.get("SQ_WAVES")
        if not w or "SQ_INSTS_VALU" not in cs:
            continue
        vals = [f"{cs[c] / w:.0f}" if c in cs else "" for c, _ in cols]
        out.append(f"| `{k[:80]}` | {w:.0f} | " + " | ".join(vals) + f" | {cs['SQ_INSTS_VALU']:.4g} |")
    return "\n".join(out)


def kernel_name(raw: str) -> str:
    return raw.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")


def _stats_rows(run_dir: str):
    """(name, calls, avg ns, min ns, max ns, % time) per kernel, from the run's
    *kernel_stats.csv or, where rocprofv3 wrote its SQLite database
    (*_results.db), from the database's kernel dispatches."""
    files = glob.glob(os.path.join(run_dir, "**", "*kernel_stats.csv"), recursive=True)
    if files:
        with open(files[0]) as fh:
            return [(r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"]),
                     float(r["Percentage"])) for r in csv.DictReader(fh)]
    dbs = glob.glob(os.path.join(run_dir, "**", "*_results.db"), recursive=True)
    if not dbs:
        raise FileNotFoundError(f"no *kernel_stats.csv or *_results.db under {run_dir}")
    import sqlite3
    con = sqlite3.connect(dbs[0])
    rows = con.execute("select name, count(*), avg(duration), min(duration), max(duration), sum(duration) "
                       "from kernels group by name order by sum(duration) desc").fetchall()
    total = sum(r[5] for r in rows) or 1.0
    return [(n, c, a, lo, hi, 100.0 * t / total) for n, c, a, lo, hi, t in rows]


def stats(run_dir: str) -> str:
    out = ["| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for name, calls, avg, lo, hi, pct in _stats_rows(run_dir):
        out.append(f"| `{kernel_name(name)[:90]}` | {calls} | {avg / 1e3:.1f} | {lo / 1e3:.1f} | {hi / 1e3:.1f} | "
                   f"{pct:.2f} |")
    return "\n".join(out)


def traffic(a) -> dict:
    copy_kib = a.copy_mib * 1024.0
    cf = mean(find(load(a.copy_fetch), "copyBuffer")["FETCH_SIZE"])
    cw = mean(find(load(a.copy_write), "copyBuffer")["WRITE_SIZE"])
    kf = mean(find(load(a.fetch), a.kernel)["FETCH_SIZE"])
    kw = mean(find(load(a.write), a.kernel)["WRITE_SIZE"])
    ff, fw = copy_kib / cf, copy_kib / cw
    return {
        "kernel": a.kernel,
        "workload": a.workload,
        "kernel_source_sha": edge_kernel_source_sha(),
        "fetch_size_kib": kf,
        "write_size_kib": kw,
        f"copy_fetch_kib_for_{a.copy_mib}MiB": cf,
        f"copy_write_kib_for_{a.copy_mib}MiB": cw,
        "fetch_factor": ff,
        "write_factor": fw,
        "bytes_per_launch": (kf * ff + kw * fw) * 1024.0,
        "command": a.command,
    }


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("table")
    t.add_argument("dirs", nargs="+")
    sub.add_parser("stats").add_argument("dir")
    sub.add_parser("issue").add_argument("dirs", nargs="+")
    r = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        r.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    r.add_argument("--copy-mib", type=int, default=512)
    r.add_argument("--kernel", required=True)
    r.add_argument("--workload", default="")
    r.add_argument("--command", default="")
    r.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "table":
        print(table(a.dirs))
        return 0
    if a.cmd == "stats":
        print(stats(a.dir))
        return 0
    if a.cmd == "issue":
        print(issue(a.dirs))
        return 0
    rec = traffic(a)
    with open(a.out, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
