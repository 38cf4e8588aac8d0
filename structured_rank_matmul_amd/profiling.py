"""Summaries of rocprofv3 CSV output for the files under profiles/.

rocprofv3 writes, with ``--output-format csv``:

* ``<prefix>_kernel_stats.csv`` for ``--kernel-trace --stats``: one row per
  kernel name with call count and duration statistics (ns);
* ``<prefix>_counter_collection.csv`` for ``--pmc``: one row per dispatch and
  counter.

``stats`` turns the first into a short text table; ``counters`` lists every
counter of one ``--pmc`` run per kernel (means per dispatch) with the MFMA
busy fraction and bf16 MFMA FLOPs derived from them; ``traffic`` turns a
FETCH_SIZE run and a WRITE_SIZE run into HBM bytes per dispatch of one kernel,
each counter scaled by what it reads for a plain copy kernel whose bytes are
known (the copy reads and writes exactly ``--copy-bytes``).  The traffic file
also records a hash of the sources the kernel is built from (``--sources``), so
that a figure taken before a change to that kernel is recognised as stale.

    python -m structured_rank_matmul_amd.profiling stats DIR --command "..." --out profiles/x.txt
    python -m structured_rank_matmul_amd.profiling traffic FETCH_DIR WRITE_DIR --kernel REGEX \
        --copy-bytes N --command-fetch "..." --command-write "..." --out profiles/y.txt
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
# sources of the GEMM kernels (the output stage's kernel among them): a change
# to any of them invalidates a recorded traffic figure
GEMM_SOURCES = ("csrc/gemm.hip", "csrc/mfma_tile.h")


def sources_sha256(sources=GEMM_SOURCES, root: str = HERE) -> str:
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(root, rel), "rb") as f:
            h.update(rel.encode())
            h.update(f.read())
    return h.hexdigest()


def _find(directory: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    return hits[0]


def _col(fields, *names):
    low = {f.lower(): f for f in fields}
    for n in names:
        if n.lower() in low:
            return low[n.lower()]
    raise KeyError(f"none of {names} in {fields}")


def short_name(name: str, width: int = 110) -> str:
    return name if len(name) <= width else name[: width - 3] + "..."


def kernel_stats(directory: str):
    """[(name, calls, total_ns, avg_ns, min_ns, max_ns)] sorted by total time."""
    path = _find(directory, "kernel_stats.csv")
    rows = []
    with open(path, newline="") as f:
        r = csv.DictReader(f)
        cn = _col(r.fieldnames, "Name", "KernelName", "Kernel_Name")
        cc = _col(r.fieldnames, "Calls")
        ct = _col(r.fieldnames, "TotalDurationNs", "Total_Duration_Ns")
        ca = _col(r.fieldnames, "AverageNs", "Average_Ns")
        cmin = _col(r.fieldnames, "MinNs", "Min_Ns")
        cmax = _col(r.fieldnames, "MaxNs", "Max_Ns")
        for row in r:
            rows.append((row[cn], int(float(row[cc])), float(row[ct]), float(row[ca]), float(row[cmin]),
                         float(row[cmax])))
    rows.sort(key=lambda x: -x[2])
    return rows


def counter_means(directory: str, counter: str):
    """{kernel name: (dispatches, mean counter value per dispatch)}."""
    path = _find(directory, "counter_collection.csv")
    vals = {}
    with open(path, newline="") as f:
        r = csv.DictReader(f)
        cn = _col(r.fieldnames, "Kernel_Name", "KernelName", "Name")
        cc = _col(r.fieldnames, "Counter_Name", "CounterName")
        cv = _col(r.fieldnames, "Counter_Value", "CounterValue")
        cd = _col(r.fieldnames, "Dispatch_Id", "DispatchId", "Correlation_Id")
        per = {}
        for row in r:
            if row[cc] != counter:
                continue
            key = (row[cn], row[cd])
            per[key] = per.get(key, 0.0) + float(row[cv])  # sum over dimensions of one dispatch
        for (name, _), v in per.items():
            vals.setdefault(name, []).append(v)
    return {k: (len(v), statistics.fmean(v)) for k, v in vals.items()}


def cmd_stats(a):
    rows = kernel_stats(a.dir)
    total = sum(r[2] for r in rows) or 1.0
    out = [f"# rocprofv3 kernel trace summary: {a.title}", "", "command:", f"    {a.command}", "",
           f"{'calls':>6} {'avg us':>9} {'min us':>9} {'max us':>9} {'total %':>8}  kernel"]
    for name, calls, tot, avg, mn, mx in rows[: a.top]:
        out.append(f"{calls:>6} {avg / 1e3:>9.2f} {mn / 1e3:>9.2f} {mx / 1e3:>9.2f} {100 * tot / total:>8.2f}  "
                   f"{short_name(name)}")
    text = "\n".join(out) + "\n"
    _write(a.out, text)


def _pick(means, pattern):
    rx = re.compile(pattern)
    hits = {k: v for k, v in means.items() if rx.search(k)}
    if not hits:
        raise SystemExit(f"no kernel matches {pattern!r}")
    return hits


def cmd_traffic(a):
    fetch = counter_means(a.fetch_dir, "FETCH_SIZE")
    write = counter_means(a.write_dir, "WRITE_SIZE")
    copy_f = _pick(fetch, a.copy_kernel)
    copy_w = _pick(write, a.copy_kernel)
    # FETCH_SIZE / WRITE_SIZE are KiB per dispatch
    cf = max(copy_f.values(), key=lambda v: v[1])[1] * 1024.0
    cw = max(copy_w.values(), key=lambda v: v[1])[1] * 1024.0
    f_scale, w_scale = a.copy_bytes / cf, a.copy_bytes / cw
    kf = _pick(fetch, a.kernel)
    kw = _pick(write, a.kernel)
    nf = sum(v[0] for v in kf.values())
    nw = sum(v[0] for v in kw.values())
    fetch_b = sum(v[0] * v[1] for v in kf.values()) / nf * 1024.0 * f_scale
    write_b = sum(v[0] * v[1] for v in kw.values()) / nw * 1024.0 * w_scale
    out = [f"# HBM traffic per dispatch: {a.title}", "",
           "commands:", f"    {a.command_fetch}", f"    {a.command_write}", "",
           f"calibration: copy kernel of {a.copy_bytes} bytes read and written",
           f"    FETCH_SIZE {cf / 1024:.1f} KiB per dispatch -> scale {f_scale:.4f}",
           f"    WRITE_SIZE {cw / 1024:.1f} KiB per dispatch -> scale {w_scale:.4f}",
           f"kernel pattern: {a.kernel}"]
    for name, (cnt, v) in sorted(kf.items()):
        out.append(f"    FETCH_SIZE {v:12.1f} KiB mean over {cnt} dispatches  {short_name(name, 90)}")
    for name, (cnt, v) in sorted(kw.items()):
        out.append(f"    WRITE_SIZE {v:12.1f} KiB mean over {cnt} dispatches  {short_name(name, 90)}")
    out += ["", f"fetch_bytes_per_dispatch = {fetch_b:.6e}", f"write_bytes_per_dispatch = {write_b:.6e}",
            f"traffic_bytes_per_dispatch = {fetch_b + write_b:.6e}",
            f"kernel_sources = {','.join(a.sources)}",
            f"kernel_sources_sha256 = {sources_sha256(a.sources)}"]
    _write(a.out, "\n".join(out) + "\n")


def counter_table(directory: str):
    """{kernel name: {counter: (dispatches, mean value per dispatch)}} for every
    counter of one --pmc run."""
    path = _find(directory, "counter_collection.csv")
    names = set()
    with open(path, newline="") as f:
        r = csv.DictReader(f)
        cc = _col(r.fieldnames, "Counter_Name", "CounterName")
        for row in r:
            names.add(row[cc])
    table = {}
    for c in sorted(names):
        for k, v in counter_means(directory, c).items():
            table.setdefault(k, {})[c] = v
    return table


def cmd_counters(a):
    table = counter_table(a.dir)
    avg_ns = {}
    if a.stats_dir:
        avg_ns = {name: avg for name, _, _, avg, _, _ in kernel_stats(a.stats_dir)}
    rx = re.compile(a.kernel) if a.kernel else None
    counters = sorted({c for v in table.values() for c in v})
    out = [f"# rocprofv3 counters per dispatch: {a.title}", "", "commands:"]
    out += [f"    {c}" for c in a.command]
    out += ["", "derived (per dispatch, where the counters are present):",
            f"    mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {a.xcds} XCDs * {a.simds} SIMDs)",
            f"      (GRBM_GUI_ACTIVE sums the {a.xcds} XCDs' busy cycles, SQ_VALU_MFMA_BUSY_CYCLES the SIMDs'"
            " matrix-core cycles; gpu_clock_ghz below checks the first reading against the kernel trace)",
            "    mfma_bf16_flop = 512 * SQ_INSTS_VALU_MFMA_MOPS_BF16",
            "    mfma_bf16_tflops = mfma_bf16_flop / average kernel duration (kernel trace)",
            f"    mfma_bf16_frac = mfma_bf16_tflops / {a.peak_tflops:g} (the dense bf16 MFMA peak); the counter"
            " runs and the trace run are separate processes, so mfma_busy (one run's cycles) and this"
            " (both runs) can disagree; the implied clock shows by how much", ""]
    for name in sorted(table, key=lambda k: -max(v[1] for v in table[k].values())):
        if rx and not rx.search(name):
            continue
        vals = table[name]
        out.append(short_name(name, 120))
        for c in counters:
            if c in vals:
                out.append(f"    {c:32s} {vals[c][1]:16.1f}   ({vals[c][0]} dispatches)")
        busy, gui = vals.get("SQ_VALU_MFMA_BUSY_CYCLES"), vals.get("GRBM_GUI_ACTIVE")
        if busy and gui and gui[1] > 0:
            out.append(f"    {'mfma_busy':32s} {busy[1] / (gui[1] / a.xcds * a.simds):16.4f}")
            if name in avg_ns and avg_ns[name] > 0:
                out.append(f"    {'gpu_clock_ghz':32s} {gui[1] / a.xcds / avg_ns[name]:16.3f}")
        mops = vals.get("SQ_INSTS_VALU_MFMA_MOPS_BF16")
        if mops:
            flop = 512.0 * mops[1]
            out.append(f"    {'mfma_bf16_flop':32s} {flop:16.4e}")
            if name in avg_ns and avg_ns[name] > 0:
                out.append(f"    {'avg_duration_us':32s} {avg_ns[name] / 1e3:16.2f}")
                out.append(f"    {'mfma_bf16_tflops':32s} {flop / avg_ns[name] / 1e3:16.1f}")
                out.append(f"    {'mfma_bf16_frac':32s} {flop / avg_ns[name] / 1e3 / a.peak_tflops:16.4f}")
    _write(a.out, "\n".join(out) + "\n")


def read_traffic(path: str):
    """Traffic bytes per dispatch from a summary written by ``traffic``, or None
    if the file is missing or the kernel's sources changed since."""
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith(" "):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    sources = tuple(x for x in vals.get("kernel_sources", "").split(",") if x)
    if not sources or vals.get("kernel_sources_sha256") != sources_sha256(sources):
        return None
    try:
        return float(vals["traffic_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def _write(path, text):
    if path == "-":
        sys.stdout.write(text)
        return
    with open(path, "w") as f:
        f.write(text)
    sys.stdout.write(text)


def main(argv=None):
    ap = argparse.ArgumentParser(prog="python -m structured_rank_matmul_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="")
    s.add_argument("--top", type=int, default=25)
    s.add_argument("--out", default="-")
    s.set_defaults(fn=cmd_stats)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--kernel", required=True, help="regex on the kernel name")
    t.add_argument("--copy-kernel", default="neg_kernel",
                   help="regex on the calibration copy kernel's name (the probe copies with torch.neg)")
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    t.add_argument("--sources", type=lambda v: tuple(v.split(",")), default=GEMM_SOURCES,
                   help="comma-separated kernel sources, relative to the package")
    t.add_argument("--title", default="")
    t.add_argument("--out", default="-")
    t.set_defaults(fn=cmd_traffic)
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--command", action="append", required=True, help="the command(s) that made the runs")
    c.add_argument("--stats-dir", default=None, help="a --kernel-trace --stats run of the same command")
    c.add_argument("--kernel", default=None, help="regex on the kernel name")
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--simds", type=int, default=1024, help="SIMDs of the GPU (4 per CU)")
    c.add_argument("--peak-tflops", type=float, default=2500.0, help="dense bf16 MFMA peak (MI355X)")
    c.add_argument("--title", default="")
    c.add_argument("--out", default="-")
    c.set_defaults(fn=cmd_counters)
    a = ap.parse_args(argv)
    a.fn(a)


if __name__ == "__main__":
    main()
