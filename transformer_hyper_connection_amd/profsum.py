"""Summaries of rocprofv3 output for the profiles/ folder.

    python -m transformer_hyper_connection_amd.profsum kernels DB --command CMD > profiles/NAME.md
    python -m transformer_hyper_connection_amd.profsum traffic --fetch DB --write DB --command CMD \
        --out profiles/NAME.json
    python -m transformer_hyper_connection_amd.profsum counters DB [DB ...] --command CMD \
        --kernels NAME [NAME ...] > profiles/NAME.md

``kernels`` tabulates a ``rocprofv3 --kernel-trace --stats`` database (count,
mean/min/max duration per kernel).  ``traffic`` reads two ``rocprofv3 --pmc``
databases, one with FETCH_SIZE and one with WRITE_SIZE (KiB per dispatch),
and scales each kernel's mean by what the same counter reads for a plain
streaming kernel of known size in the same run (bench.py's reference
stream: torch.mul over 1 GiB of bf16 into another 1 GiB, one dispatch that
reads 1 GiB and writes 1 GiB): factor = true bytes / counted bytes.  The
JSON records the SHA-256 of the kernel source, so a reader can tell whether
the counters still describe the current kernels.  ``counters`` tabulates the
mean per dispatch of every counter in one or more ``rocprofv3 --pmc``
databases for the kernels named, with a few ratios derived from them.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sqlite3
import sys

SOURCE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "hc.hip")
COPY_KERNEL = "MulFunctor"     # substring of the reference stream's kernel name
COPY_BYTES = 1 << 30          # read and written by each reference-stream dispatch


def source_sha256(path: str = SOURCE) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def short_name(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    return name.split("(")[0] if "(" in name else name


def kernel_rows(db_path: str):
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, count(*), avg(duration), min(duration), max(duration) "
                      "from kernels group by name order by sum(duration) desc").fetchall()
    return [(short_name(k), n, avg / 1e3, lo / 1e3, hi / 1e3) for k, n, avg, lo, hi in rows]


def cmd_kernels(args) -> None:
    print(f"# {args.title}\n")
    print(f"Command (from the repository root):\n\n    {args.command}\n")
    print("| kernel | calls | mean us | min us | max us |")
    print("|---|---:|---:|---:|---:|")
    for k, n, avg, lo, hi in kernel_rows(args.db):
        print(f"| `{k}` | {n} | {avg:.2f} | {lo:.2f} | {hi:.2f} |")
    print(f"\nKernel source SHA-256: `{source_sha256()}`")


def counter_means(db_path: str, counter: str):
    db = sqlite3.connect(db_path)
    rows = db.execute("select kernel_name, dispatch_id, sum(value) from counters_collection "
                      "where counter_name = ? group by kernel_name, dispatch_id", (counter,)).fetchall()
    per = {}
    for k, _, v in rows:
        per.setdefault(short_name(k), []).append(v)
    return per


def copy_factor(per: dict, counter: str) -> float:
    vals = [v for k, vs in per.items() if COPY_KERNEL in k for v in vs]
    if not vals:
        raise SystemExit(f"no {COPY_KERNEL} dispatch with {counter} in the database")
    top = max(vals)
    big = [v for v in vals if v > 0.9 * top]      # the 1 GiB dispatches
    counted = sum(big) / len(big) * 1024.0
    return COPY_BYTES / counted


def cmd_traffic(args) -> None:
    fetch = counter_means(args.fetch, "FETCH_SIZE")
    write = counter_means(args.write, "WRITE_SIZE")
    ff, fw = copy_factor(fetch, "FETCH_SIZE"), copy_factor(write, "WRITE_SIZE")
    kernels = {}
    for k in sorted(set(fetch) | set(write)):
        if COPY_KERNEL in k or k.startswith("void at::") or k.startswith("__amd"):
            continue
        f = fetch.get(k, [])
        w = write.get(k, [])
        if not f or not w:
            continue
        fk, wk = sum(f) / len(f), sum(w) / len(w)
        kernels[k] = {"dispatches": len(f), "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                      "fetch_bytes": round(fk * 1024 * ff), "write_bytes": round(wk * 1024 * fw)}
    out = {"command_fetch": args.command.replace("COUNTER", "FETCH_SIZE"),
           "command_write": args.command.replace("COUNTER", "WRITE_SIZE"),
           "calibration": {"kernel": COPY_KERNEL, "bytes_each_way": COPY_BYTES,
                           "fetch_factor": round(ff, 5), "write_factor": round(fw, 5)},
           "kernel_source_sha256": source_sha256(), "kernels": kernels}
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def dispatch_values(db_path: str):
    """{kernel: {counter: [per-dispatch value]}}; a dispatch's value is the sum
    over the instances rocprofv3 reports (GRBM_GUI_ACTIVE thus comes out as the
    busy clock summed over the XCDs)."""
    db = sqlite3.connect(db_path)
    rows = db.execute("select kernel_name, dispatch_id, counter_name, sum(value) "
                      "from counters_collection group by kernel_name, dispatch_id, counter_name").fetchall()
    out = {}
    for k, _, c, total in rows:
        out.setdefault(short_name(k), {}).setdefault(c, []).append(total)
    return out


def cmd_counters(args) -> None:
    merged = {}
    for db in args.db:
        for k, cs in dispatch_values(db).items():
            for c, vs in cs.items():
                merged.setdefault(k, {})[c] = vs
    print(f"# {args.title}\n")
    print(f"Commands (from the repository root):\n")
    for c in args.command:
        print(f"    {c}")
    print("\nMean per dispatch, summed over the chip.  GRBM_GUI_ACTIVE is the busy clock summed over\n"
          f"the {args.xcds} XCDs (divided by {args.xcds} and {args.mhz} MHz it matches the kernel's duration);\n"
          "the busy fractions below divide by that per-XCD clock times the SIMD count.  A wave64\n"
          "VALU instruction is counted as 4 cycles (16 lanes per cycle; transcendentals take longer).\n")
    for want in args.kernels:
        hits = [k for k in merged if want in k]
        for k in hits:
            cs = merged[k]
            mean = {c: sum(v) / len(v) for c, v in cs.items()}
            print(f"## `{k}` ({len(next(iter(cs.values())))} dispatches)\n")
            print("| counter | mean |")
            print("|---|---:|")
            for c in sorted(mean):
                print(f"| {c} | {mean[c]:,.0f} |")
            derived = []
            if mean.get("SQ_WAVES"):
                for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_VMEM"):
                    if c in mean:
                        derived.append((f"{c} per wave", mean[c] / mean["SQ_WAVES"]))
            if mean.get("SQ_LDS_IDX_ACTIVE") and "SQ_LDS_BANK_CONFLICT" in mean:
                derived.append(("LDS bank-conflict cycles / LDS active cycles",
                                mean["SQ_LDS_BANK_CONFLICT"] / mean["SQ_LDS_IDX_ACTIVE"]))
            if mean.get("GRBM_GUI_ACTIVE"):
                clk = mean["GRBM_GUI_ACTIVE"] / args.xcds
                derived.append((f"busy clock per XCD, us at {args.mhz} MHz", clk / args.mhz))
                if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
                    derived.append((f"MFMA busy, % of {args.simds} SIMDs x busy clock",
                                    100 * mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (clk * args.simds)))
                if "SQ_INSTS_VALU" in mean:
                    derived.append((f"VALU issue, % of {args.simds} SIMDs x busy clock (4 cycles each)",
                                    100 * 4 * mean["SQ_INSTS_VALU"] / (clk * args.simds)))
            if mean.get("TCC_HIT_sum") is not None and mean.get("TCC_MISS_sum") is not None:
                tot = mean["TCC_HIT_sum"] + mean["TCC_MISS_sum"]
                if tot:
                    derived.append(("L2 hit rate", mean["TCC_HIT_sum"] / tot))
            if derived:
                print("\n| derived | value |")
                print("|---|---:|")
                for name, v in derived:
                    print(f"| {name} | {v:,.4g} |")
            print()
    print(f"Kernel source SHA-256: `{source_sha256()}`")


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("db")
    k.add_argument("--command", required=True)
    k.add_argument("--title", default="rocprofv3 kernel trace")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--command", required=True, help="the rocprofv3 command, with COUNTER for the counter name")
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("db", nargs="+")
    c.add_argument("--command", required=True, action="append", help="one per database")
    c.add_argument("--kernels", required=True, nargs="+", help="substrings of the kernel names to report")
    c.add_argument("--title", default="rocprofv3 counters")
    c.add_argument("--simds", type=int, default=1024, help="SIMDs on the device (256 CUs x 4)")
    c.add_argument("--xcds", type=int, default=8, help="XCDs on the device")
    c.add_argument("--mhz", type=float, default=2400.0, help="shader clock")
    args = ap.parse_args(argv)
    {"kernels": cmd_kernels, "traffic": cmd_traffic, "counters": cmd_counters}[args.what](args)


if __name__ == "__main__":
    main(sys.argv[1:])
