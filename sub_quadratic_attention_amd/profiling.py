"""Summaries of rocprofv3 output for the committed profiles.

python -m sub_quadratic_attention_amd.profiling stats KERNEL_STATS_CSV "COMMAND"
    print a text table of a --kernel-trace --stats run (kernel, calls,
    average / total microseconds, share).

python -m sub_quadratic_attention_amd.profiling counters DIR [DIR ...] --command "COMMAND"
    per-kernel table of --pmc runs (each DIR a rocprofv3 --output-format csv
    output holding run_counter_collection.csv): instruction counts, MFMA
    operations by type, and the MFMA-busy fraction of the SIMD cycles
    (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE of one XCD times the 1024
    SIMDs, as rocprofv3's MfmaUtil metric defines it).

python -m sub_quadratic_attention_amd.profiling traffic --kernel LABEL --symbol NAME_FRAGMENT
        --source csrc/FILE.hip --workload NAME --fetch CSV --write CSV
        --copy-fetch CSV --copy-write CSV --copy-bytes N
    HBM traffic per launch of one kernel from two --pmc runs (FETCH_SIZE,
    then WRITE_SIZE, KiB per dispatch), each scaled by what the same counter
    reads for a plain copy of N bytes; writes profiles/traffic.json together
    with the SHA-256 of the kernel's source file, so that bench.py stops
    reporting the figure once the kernel changes.
"""

import argparse
import csv
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")

def source_hash(rel):
    with open(os.path.join(HERE, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def stats_table(path, command):
    rows = list(csv.DictReader(open(path)))
    key = lambda r, *names: next(r[n] for n in names if n in r)
    out = [f"command: {command}", "", f"{'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'total_us':>11s} {'share':>6s}"]
    for r in rows:
        name = key(r, "Name", "KernelName", "Kernel_Name")
        calls = int(float(key(r, "Calls", "TotalCalls")))
        tot = float(key(r, "TotalDurationNs", "Total_Duration_Ns")) / 1e3
        avg = float(key(r, "AverageNs", "Average_Ns")) / 1e3
        pct = float(key(r, "Percentage", "Percent"))
        short = name if len(name) <= 70 else name[:67] + "..."
        out.append(f"{short:70s} {calls:6d} {avg:10.2f} {tot:11.1f} {pct:5.1f}%")
    return "\n".join(out)


def counter_sum(path, symbol, counter):
    """Mean per dispatch of a counter over the dispatches of kernels whose name contains symbol."""
    per = {}
    for r in csv.DictReader(open(path)):
        if symbol in r["Kernel_Name"] and r["Counter_Name"] == counter:
            per.setdefault(r["Dispatch_Id"], 0.0)
            per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    return (sum(per.values()) / len(per), len(per)) if per else (0.0, 0)


def copy_counter(path, counter):
    """Largest per-dispatch value of a counter (the copy kernel of the calibration run)."""
    per = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            per.setdefault(r["Dispatch_Id"], 0.0)
            per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    return max(per.values())


def kernel_short_name(full):
    """pair_gram_kernel from 'void thin::(anonymous namespace)::pair_gram_kernel<1>(thin::GramLaunch, ...)'."""
    import re
    names = re.findall(r"::(\w+)(?:<[^>]*>)?\(", full)
    return names[-1] if names else full


def counters_table(dirs, command, xcds=8, simds=1024):
    """Sum every counter over the dispatches of each kernel, per --pmc run directory."""
    per = {}        # kernel -> counter -> total
    grbm = {}       # kernel -> sum over dispatches of GRBM_GUI_ACTIVE / xcds (one pass)
    dispatches = {}
    for n, d in enumerate(dirs):
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            k = kernel_short_name(r["Kernel_Name"])
            c, v = r["Counter_Name"], float(r["Counter_Value"])
            if c == "GRBM_GUI_ACTIVE":
                if n == 0:
                    grbm[k] = grbm.get(k, 0.0) + v / xcds
                    dispatches[k] = dispatches.get(k, 0) + 1
                continue
            per.setdefault(k, {})
            per[k][c] = per[k].get(c, 0.0) + v
    out = [f"command: {command}", ""]
    for k in sorted(per, key=lambda x: -grbm.get(x, 0.0)):
        c = per[k]
        g = grbm.get(k, 0.0)
        out.append(f"{k}: {dispatches.get(k, 0)} dispatches, {g:.4g} GPU cycles (GRBM_GUI_ACTIVE of one XCD)")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c and g:
            out.append(f"    MFMA busy: {100.0 * c['SQ_VALU_MFMA_BUSY_CYCLES'] / (g * simds):.1f}% of SIMD cycles")
        for name in sorted(c):
            if name == "SQ_VALU_MFMA_BUSY_CYCLES":
                continue
            out.append(f"    {name:34s} {c[name]:.6g}")
    return "\n".join(out)


def traffic_for(label, workload):
    """Bytes per launch recorded for this kernel and workload, or None if absent or stale."""
    try:
        rec = json.load(open(TRAFFIC_JSON))[label][workload]
    except (OSError, KeyError, ValueError):
        return None
    try:
        if rec.get("source_sha256") != source_hash(rec["source"]):
            return None
    except OSError:
        return None
    return rec["bytes_per_launch"]


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("command")
    cn = sub.add_parser("counters")
    cn.add_argument("dirs", nargs="+")
    cn.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    for name in ("kernel", "symbol", "source", "workload", "fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + name.replace("_", "-"), required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    args = p.parse_args(argv)
    if args.cmd == "stats":
        print(stats_table(args.csv, args.command))
        return 0
    if args.cmd == "counters":
        print(counters_table(args.dirs, args.command))
        return 0
    symbol, src = args.symbol, args.source
    f_kib, nf = counter_sum(args.fetch, symbol, "FETCH_SIZE")
    w_kib, nw = counter_sum(args.write, symbol, "WRITE_SIZE")
    cf = args.copy_bytes / (copy_counter(args.copy_fetch, "FETCH_SIZE") * 1024.0)
    cw = args.copy_bytes / (copy_counter(args.copy_write, "WRITE_SIZE") * 1024.0)
    rec = {
        "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib, "dispatches": [nf, nw],
        "copy_scale_fetch": cf, "copy_scale_write": cw,
        "bytes_per_launch": f_kib * 1024.0 * cf + w_kib * 1024.0 * cw,
        "source": src, "source_sha256": source_hash(src),
    }
    data = {}
    if os.path.exists(TRAFFIC_JSON):
        data = json.load(open(TRAFFIC_JSON))
    data.setdefault(args.kernel, {})[args.workload] = rec
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    json.dump(data, open(TRAFFIC_JSON, "w"), indent=1, sort_keys=True)
    print(json.dumps(rec, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
