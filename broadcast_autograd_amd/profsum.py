"""Text summaries of rocprofv3 output for the library's kernels.

    python -m broadcast_autograd_amd.profsum stats DIR [--title T] [--cmd C]
    python -m broadcast_autograd_amd.profsum counters --fetch DIR --write DIR
        --calib KERNEL:GRID:BYTES [--check KERNEL:GRID:BYTES[:FIRST_N] ...]
        [--traffic WORKLOAD:CLASS:GRID ...] [--cmd C ...]
    python -m broadcast_autograd_amd.profsum pmc DIR [--per-element GRID:ELEMENTS ...]

`stats` condenses a `--kernel-trace --stats` run (the *_kernel_stats.csv
rocprofv3 writes) into one line per kernel.  `counters` turns two `--pmc`
runs (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch) into HBM bytes per
dispatch, each counter scaled by what it reads for a copy of known size (the
calibration kernel and grid; another copy's factors are printed beside them
as a cross-check), and emits `traffic` lines for the benchmark
keyed to a hash of the kernel sources.  `pmc` averages any counters per
(kernel, grid) and, given the elements a grid processes, per element (an
SQ_INSTS_* count is of wave instructions, each serving 64 lanes, so per
element it is 64 times the count over the elements).
Only the CSV files rocprofv3 writes are read; nothing is executed.
"""
import argparse
import csv
import glob
import hashlib
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def source_hash():
    """sha256 of the device code, kernel argument blocks and planner (the
    sources that decide which kernels run and what they move)."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "broadcast_autograd_amd", "csrc", "*"))):
        if p.endswith((".hip", ".h")) or p.endswith("zk_plan.cpp"):
            with open(p, "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def short_name(name):
    """Kernel name without its parameter list ("void " and "(...)" dropped)."""
    n = name.strip().strip('"')
    if n.startswith("void "):
        n = n[5:]
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return n[:i]
    return n


def find_csv(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        sys.exit(f"no *{suffix} under {d}")
    return hits


def cmd_stats(a):
    rows = []
    for p in find_csv(a.dir, "kernel_stats.csv"):
        with open(p, newline="") as f:
            for r in csv.DictReader(f):
                rows.append(r)
    out = []
    if a.title:
        out.append(f"# {a.title}")
    for n in a.note or []:
        out.append(f"# {n}")
    for c in a.cmd or []:
        out.append(f"# command: {c}")
    out.append("# one line per kernel: calls, average / min / max duration (us), share of GPU time")
    out.append("")
    out.append(f"{'kernel':<64} {'calls':>7} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        n = short_name(r["Name"])
        if a.only and not re.search(a.only, n):
            continue
        out.append(f"{n[:64]:<64} {int(r['Calls']):>7} {float(r['AverageNs']) / 1e3:>10.2f} "
                   f"{float(r['MinNs']) / 1e3:>10.2f} {float(r['MaxNs']) / 1e3:>10.2f} "
                   f"{float(r['Percentage']):>6.2f}")
    print("\n".join(out))


def read_counters(d, first=None):
    """{(kernel, grid): {counter: [value per dispatch]}} from a --pmc run, in
    dispatch order; with first = {(kernel, grid): n}, only the first n
    dispatches of those groups."""
    rows = []
    for p in find_csv(d, "counter_collection.csv"):
        with open(p, newline="") as f:
            for r in csv.DictReader(f):
                rows.append((int(r["Dispatch_Id"]), (short_name(r["Kernel_Name"]), int(r["Grid_Size"])),
                             r["Counter_Name"], float(r["Counter_Value"])))
    rows.sort(key=lambda t: t[0])
    acc = defaultdict(lambda: defaultdict(list))
    for _, key, name, v in rows:
        if first and key in first and len(acc[key][name]) >= first[key]:
            continue
        acc[key][name].append(v)
    return acc


def mean(v):
    return sum(v) / len(v)


def cmd_counters(a):
    fetch, write = read_counters(a.fetch), read_counters(a.write)
    ck, cg, cb = a.calib.rsplit(":", 2)
    cg, cb = int(cg), int(cb)
    if not fetch.get((ck, cg), {}).get("FETCH_SIZE") or not write.get((ck, cg), {}).get("WRITE_SIZE"):
        sys.exit(f"calibration kernel {ck} with grid {cg} not found")
    f_cal = mean(fetch[(ck, cg)]["FETCH_SIZE"]) * 1024
    w_cal = mean(write[(ck, cg)]["WRITE_SIZE"]) * 1024
    # the copy reads cb / 2 bytes and writes cb / 2
    ff, fw = (cb / 2) / f_cal, (cb / 2) / w_cal
    out = ["# HBM traffic per dispatch from rocprofv3 hardware counters (MI355X)"]
    for c in a.cmd or []:
        out.append(f"#   {c}")
    out.append(f"# calibration: {ck} grid {cg}, a copy of {cb // 2} bytes read and {cb // 2} written,")
    out.append(f"#   reads FETCH_SIZE {f_cal / 1024:.1f} KiB and WRITE_SIZE {w_cal / 1024:.1f} KiB")
    out.append(f"#   -> scale factors fetch x{ff:.4f}, write x{fw:.4f} (applied below)")
    for chk in a.check or []:
        # NAME:GRID:BYTES[:N] -- the first N dispatches of that kernel and grid
        parts = chk.split(":")
        n2 = None
        if len(parts) >= 4 and parts[-1].isdigit() and parts[-2].isdigit() and parts[-3].isdigit():
            n2 = int(parts[-1])
            parts = parts[:-1]
        k2, g2, b2 = ":".join(parts[:-2]), int(parts[-2]), int(parts[-1])
        sel = {(k2, g2): n2} if n2 else None
        f2d, w2d = read_counters(a.fetch, sel), read_counters(a.write, sel)
        if not f2d.get((k2, g2), {}).get("FETCH_SIZE") or not w2d.get((k2, g2), {}).get("WRITE_SIZE"):
            sys.exit(f"cross-check kernel {k2} with grid {g2} not found")
        f2 = mean(f2d[(k2, g2)]["FETCH_SIZE"]) * 1024
        w2 = mean(w2d[(k2, g2)]["WRITE_SIZE"]) * 1024
        which = f"the first {n2} dispatches of " if n2 else ""
        out.append(f"# cross-check: {which}{k2} grid {g2}, a copy of {b2 // 2} bytes each way,")
        out.append(f"#   gives fetch x{(b2 / 2) / f2:.4f}, write x{(b2 / 2) / w2:.4f}")
    h = source_hash()
    out.append(f"# source_sha256 {h}")
    out.append("#")
    out.append(f"# {'kernel':<58} {'grid':>9} {'n':>5} {'fetch_KiB':>12} {'write_KiB':>12} {'scaled_MB':>10}")
    keys = sorted(set(fetch) & set(write),
                  key=lambda k: -(mean(fetch[k]["FETCH_SIZE"]) * ff + mean(write[k]["WRITE_SIZE"]) * fw))
    scaled = {}
    for k in keys:
        fk, wk = mean(fetch[k]["FETCH_SIZE"]), mean(write[k]["WRITE_SIZE"])
        b = (fk * ff + wk * fw) * 1024
        scaled[k] = b
        out.append(f"  {k[0][:58]:<58} {k[1]:>9} {len(fetch[k]['FETCH_SIZE']):>5} "
                   f"{fk:>12.1f} {wk:>12.1f} {b / 1e6:>10.3f}")
    out.append("#")
    out.append("# traffic <workload> <kernel class> <bytes per launch, scaled> <source sha256>")
    for t in a.traffic or []:
        wl, cls, grid = t.split(":")
        hit = [k for k in keys if k[1] == int(grid) and short_name(k[0]).split("<")[0].endswith("k_" + cls)]
        if len(hit) != 1:
            sys.exit(f"traffic {t}: {len(hit)} matching dispatch groups")
        out.append(f"traffic {wl} {cls} {int(round(scaled[hit[0]]))} {h}")
    print("\n".join(out))


def cmd_pmc(a):
    acc = read_counters(a.dir)
    per = {}
    for s in a.per_element or []:
        g, n = s.split(":")
        per[int(g)] = int(n)
    names = sorted({c for v in acc.values() for c in v})
    out = [f"# {n}" for n in a.note or []]
    for c in a.cmd or []:
        out.append(f"# command: {c}")
    out.append("# mean per dispatch (and per element where the grid's element count is given)")
    for k in sorted(acc, key=lambda k: (k[0], k[1])):
        if a.only and not re.search(a.only, k[0]):
            continue
        n = len(next(iter(acc[k].values())))
        out.append(f"{k[0]}  grid {k[1]}  dispatches {n}")
        for c in names:
            if c in acc[k]:
                v = mean(acc[k][c])
                extra = ""
                if k[1] in per:
                    # a wave instruction serves 64 lanes: per element it is
                    # 64 / elements of the count
                    f = 64.0 if c.startswith("SQ_INSTS") else 1.0
                    extra = f"   {v * f / per[k[1]]:.3f} per element"
                out.append(f"    {c:<28} {v:>16.1f}{extra}")
    print("\n".join(out))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--title")
    s.add_argument("--cmd", action="append")
    s.add_argument("--note", action="append")
    s.add_argument("--only")
    c = sub.add_parser("counters")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--calib", required=True)
    c.add_argument("--check", action="append")
    c.add_argument("--traffic", action="append")
    c.add_argument("--cmd", action="append")
    p = sub.add_parser("pmc")
    p.add_argument("dir")
    p.add_argument("--per-element", action="append")
    p.add_argument("--cmd", action="append")
    p.add_argument("--note", action="append")
    p.add_argument("--only")
    a = ap.parse_args(argv)
    {"stats": cmd_stats, "counters": cmd_counters, "pmc": cmd_pmc}[a.what](a)


if __name__ == "__main__":
    main()
