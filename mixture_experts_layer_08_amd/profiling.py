"""Summaries of rocprofv3 counter runs for the roofline's `traffic` figure.

HBM traffic of a kernel is read from two `rocprofv3 --pmc` runs (FETCH_SIZE,
then WRITE_SIZE; both in KiB per dispatch).  Each counter is calibrated with
a plain device copy of known size profiled in the same run: the factor
(known bytes) / (counter bytes) scales the kernel's reading.

    python -m mixture_experts_layer_08_amd.profiling traffic \
        --fetch <fetch run>/p_counter_collection.csv \
        --write <write run>/p_counter_collection.csv \
        --copy-bytes 1073741824 --workload mixtral_bf16 \
        --out profiles/grouped_gemm_mixtral_bf16_traffic.json

``--kernel mx8`` summarises the MXFP8 grouped GEMM of the same run instead
(profiles/grouped_gemm_mx8_<workload>_traffic.json).
"""

from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
# Kernel families: the dispatches summarised and the sources their hash covers.
#   bf16: the forward's row-major (NN) instantiations, GEMM1 with GELU and GEMM2
#   mx8:  the MXFP8 grouped GEMM (both epilogues)
KERNELS = {
    "bf16": (re.compile(r"k_grouped_gemm_bf16<\s*0\s*,"), ("gemm.hip", "gemm_common.h")),
    "mx8": (re.compile(r"k_grouped_gemm_mx8<"), ("gemm_mx8.hip", "gemm_common.h", "mx.h")),
}
COPY_KERNEL = "copyBuffer"  # the HIP runtime's device-to-device copy kernel


def gemm_source_hash(kernel: str = "bf16") -> str:
    """Hash of a grouped GEMM's sources (the kernel and its shared helpers)."""
    h = hashlib.sha256()
    for name in KERNELS[kernel][1]:
        h.update(open(os.path.join(PKG, "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def per_dispatch(path: str, counter: str):
    """{dispatch_id: (kernel_name, grid, value summed over instances)}."""
    vals = collections.defaultdict(float)
    meta = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        vals[d] += float(r["Counter_Value"])
        meta[d] = (r["Kernel_Name"], int(r["Grid_Size"]))
    return {d: (meta[d][0], meta[d][1], v) for d, v in vals.items()}


def traffic(fetch_csv, write_csv, copy_bytes, workload, out, kernel="bf16"):
    pattern = KERNELS[kernel][0]
    res = {"workload": workload, "kernel": pattern.pattern,
           "gemm_source_sha256_16": gemm_source_hash(kernel), "copy_bytes": copy_bytes}
    totals = {}
    for name, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"),
                                ("write", write_csv, "WRITE_SIZE")):
        d = per_dispatch(path, counter)
        gemm_ids = [i for i, (k, g, v) in d.items() if pattern.search(k)]
        if not gemm_ids:
            raise SystemExit(f"{path}: no grouped-GEMM dispatch")
        gemms = [d[i][2] for i in gemm_ids]
        by_name = collections.defaultdict(list)
        for i in gemm_ids:
            by_name[re.sub(r"\(.*", "", d[i][0]).replace("void ", "")].append(d[i][2])
        # the calibration copy is launched after the timed steps: the largest
        # copy dispatch after the last GEMM
        copies = [v for i, (k, g, v) in d.items() if COPY_KERNEL in k and i > max(gemm_ids)]
        if not copies:
            raise SystemExit(f"{path}: no calibration copy after the GEMM dispatches")
        # a device copy of copy_bytes reads and writes copy_bytes each
        factor = copy_bytes / (max(copies) * 1024.0)
        res[f"{name}_calibration_factor"] = factor
        res[f"{name}_kib_per_launch_raw"] = sum(gemms) / len(gemms)
        totals[name] = sum(gemms) / len(gemms) * 1024.0 * factor
        res[f"{name}_bytes_per_launch"] = totals[name]
        res[f"{name}_launches"] = len(gemms)
        res[f"{name}_bytes_per_launch_by_kernel"] = {
            k: sum(v) / len(v) * 1024.0 * factor for k, v in sorted(by_name.items())}
    res["hbm_bytes_per_launch"] = totals["fetch"] + totals["write"]
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


def per_kernel(path: str, counter: str, patterns: dict):
    """{name: [values per dispatch]} for each kernel-name regex in patterns."""
    d = per_dispatch(path, counter)
    out = {n: [] for n in patterns}
    for i in sorted(d):
        k, _, v = d[i]
        for n, rx in patterns.items():
            if re.search(rx, k):
                out[n].append(v)
                break
    return out, d


# the bandwidth-bound kernels of the forward (bf16 and MXFP8 forms)
HBM_KERNELS = {
    "k_route_bf16": r"k_route_bf16<", "k_transpose_router": r"k_transpose_router",
    "k_scan_blocks": r"k_scan_blocks", "k_permute": r"k_permute<", "k_permute_mx8": r"k_permute_mx8<",
    "k_combine": r"k_combine<", "k_combine_mx8": r"k_combine_mx8<",
}


def hbm(fetch_csv, write_csv, copy_bytes, title, cmd, out):
    """Markdown table: calibrated HBM bytes read and written per dispatch of
    each bandwidth-bound kernel (mean over its dispatches)."""
    rows = {}
    for name, path, counter in (("read", fetch_csv, "FETCH_SIZE"), ("written", write_csv, "WRITE_SIZE")):
        vals, d = per_kernel(path, counter, HBM_KERNELS)
        copies = [v for i, (k, g, v) in d.items() if COPY_KERNEL in k]
        factor = copy_bytes / (max(copies) * 1024.0)
        for n, vs in vals.items():
            if vs:
                rows.setdefault(n, {})[name] = sum(vs) / len(vs) * 1024.0 * factor
                rows[n]["dispatches"] = len(vs)
        rows.setdefault("_factor", {})[name] = factor
    lines = [f"# {title}", "", "Command (run from the repository root on one MI355X):", "", "```",
             cmd, "```", "",
             "FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by the factor that maps the "
             f"same counter on a {copy_bytes} B device copy in the same run to its known bytes "
             f"(read {rows['_factor']['read']:.4f}, write {rows['_factor']['written']:.4f}).", "",
             "| kernel | dispatches | MB read | MB written | MB total |", "|---|---|---|---|---|"]
    for n in HBM_KERNELS:
        if n in rows:
            r = rows[n]
            lines.append(f"| `{n}` | {r['dispatches']} | {r.get('read', 0) / 1e6:.1f} | "
                         f"{r.get('written', 0) / 1e6:.1f} | "
                         f"{(r.get('read', 0) + r.get('written', 0)) / 1e6:.1f} |")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def mfma(csv_path, title, cmd, out, simds: int = 1024):
    """Markdown table: per grouped-GEMM dispatch, SQ_VALU_MFMA_BUSY_CYCLES over
    all SIMDs divided by (SIMDs x GRBM_GUI_ACTIVE per XCD): the fraction of
    the kernel's cycles the MFMA pipes were busy."""
    pats = {"k_grouped_gemm_bf16 (GEMM1, GELU)": r"k_grouped_gemm_bf16<\s*0\s*,\s*1>",
            "k_grouped_gemm_bf16 (GEMM2)": r"k_grouped_gemm_bf16<\s*0\s*,\s*0>",
            "k_grouped_gemm_mx8 (GEMM1, GELU)": r"k_grouped_gemm_mx8<1>",
            "k_grouped_gemm_mx8 (GEMM2)": r"k_grouped_gemm_mx8<0>"}
    busy, _ = per_kernel(csv_path, "SQ_VALU_MFMA_BUSY_CYCLES", pats)
    gui, _ = per_kernel(csv_path, "GRBM_GUI_ACTIVE", pats)
    lines = [f"# {title}", "", "Command (run from the repository root on one MI355X):", "", "```",
             cmd, "```", "",
             f"MFMA busy fraction = SQ_VALU_MFMA_BUSY_CYCLES (summed over the {simds} SIMDs) / "
             f"({simds} x GRBM_GUI_ACTIVE / 8), GRBM_GUI_ACTIVE being summed over the 8 XCDs.", "",
             "| kernel | dispatches | MFMA busy cycles | GUI active cycles (per XCD) | MFMA busy |",
             "|---|---|---|---|---|"]
    for n in pats:
        if busy[n]:
            b = sum(busy[n]) / len(busy[n])
            g = sum(gui[n]) / len(gui[n]) / 8.0
            lines.append(f"| `{n}` | {len(busy[n])} | {b:.4g} | {g:.4g} | {b / (simds * g):.1%} |")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def stats(stats_csv, trace_csv, bench_log, title, cmd, note, out, kernel="bf16", top=14,
          window=None):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run: the kernel
    table, then the grouped GEMM's mean launch duration from the trace beside
    bench.py's event-timed mean launch of the same run (from the JSON line it
    printed).  window = (start, count) restricts the trace mean to those
    matching dispatches in dispatch order (e.g. the timed forward's launches
    of a run that also has other legs); None takes every matching one."""
    rows = list(csv.DictReader(open(stats_csv)))
    short = lambda n: re.sub(r"\(.*", "", n).replace("void ", "")[:70]
    lines = [f"# {title}", "", "Command (run from the repository root on one MI355X):", "", "```",
             cmd, "```", "",
             "| kernel | calls | avg us | min us | max us | % of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in rows[:top]:
        lines.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.2f} |")
    pattern = KERNELS[kernel][0]
    disp = sorted((int(r["Dispatch_Id"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                  for r in csv.DictReader(open(trace_csv)) if pattern.search(r["Kernel_Name"]))
    durs = [d / 1e3 for _, d in disp]
    which = "every dispatch in the trace"
    if window is not None:
        start, count = window
        durs = durs[start:start + count]
        which = f"dispatches {start}..{start + len(durs) - 1} of the trace's {len(disp)} matching ones"
    bench = None
    for line in open(bench_log):
        if line.startswith("{") and '"metric"' in line:
            bench = json.loads(line)
    lines.append("")
    if durs:
        lines.append(f"Grouped GEMM (`{pattern.pattern}`), {which}: {len(durs)} launches, "
                     f"mean {sum(durs) / len(durs):.1f} us.")
    if bench is not None:
        g = bench["roofline"] if kernel == "bf16" else bench["mxfp8"]["grouped_gemm"]
        lines.append(f"bench.py's event-timed mean launch over its timed steps in the same run: "
                     f"{g['avg_launch_ms'] * 1e3:.1f} us ({g['achieved']:.1f} {g['unit']}, "
                     f"{g['achieved'] / g['peak']:.1%} of {g['peak']:.0f}).")
    if note:
        lines += ["", note]
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--kernel", choices=sorted(KERNELS), default="bf16")
    h = sub.add_parser("hbm")
    h.add_argument("--fetch", required=True)
    h.add_argument("--write", required=True)
    h.add_argument("--copy-bytes", type=int, required=True)
    h.add_argument("--title", required=True)
    h.add_argument("--command", required=True, help="the command that produced the runs")
    h.add_argument("--out", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--csv", required=True)
    m.add_argument("--title", required=True)
    m.add_argument("--command", required=True, help="the command that produced the run")
    m.add_argument("--out", required=True)
    st = sub.add_parser("stats")
    st.add_argument("--stats", required=True, help="kernel_stats.csv of the run")
    st.add_argument("--trace", required=True, help="kernel_trace.csv of the run")
    st.add_argument("--bench-log", required=True, help="stdout of the profiled bench.py")
    st.add_argument("--title", required=True)
    st.add_argument("--command", required=True, help="the command that produced the run")
    st.add_argument("--note", default="")
    st.add_argument("--kernel", choices=sorted(KERNELS), default="bf16")
    st.add_argument("--window", default=None, metavar="START:COUNT",
                    help="only these matching dispatches, in dispatch order")
    st.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.cmd == "traffic":
        traffic(a.fetch, a.write, a.copy_bytes, a.workload, a.out, a.kernel)
    elif a.cmd == "hbm":
        hbm(a.fetch, a.write, a.copy_bytes, a.title, a.command, a.out)
    elif a.cmd == "stats":
        win = tuple(int(v) for v in a.window.split(":")) if a.window else None
        stats(a.stats, a.trace, a.bench_log, a.title, a.command, a.note, a.out, a.kernel,
              window=win)
    else:
        mfma(a.csv, a.title, a.command, a.out)


if __name__ == "__main__":
    main()
