"""Summaries of rocprofv3 counter runs: the roofline's `traffic` figure, the
bandwidth-bound kernels' bytes, and the grouped GEMMs' clock and MFMA-busy
fractions.

Traffic of a kernel is read from two `rocprofv3 --pmc` runs (FETCH_SIZE,
then WRITE_SIZE; both in KiB per dispatch).  These count the requests that
miss the L2 (whether the Infinity Cache or HBM then serves them), so the
figure is L2-miss traffic, an upper bound on HBM bytes.  Each counter is
calibrated with a plain device copy of known size profiled in the same run:
the factor (known bytes) / (counter bytes) scales the kernel's reading.  On
this GPU FETCH_SIZE reports half of the copy's bytes read (factor 2.0) and
WRITE_SIZE all of its bytes written (1.0); the raw KiB are kept beside the
scaled bytes, since the copy's loads are plain vector loads and the GEMM's
are LDS-direct loads.

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
#   bf16: the forward's row-major (NN) instantiations of the four-wave kernel,
#         GEMM1 with GELU and GEMM2
#   mx8:  the MXFP8 grouped GEMM (both epilogues)
KERNELS = {
    "bf16": (re.compile(r"k_grouped_gemm_w4<\s*0\s*,"), ("gemm.hip", "gemm_common.h")),
    "mx8": (re.compile(r"k_grouped_gemm_mx8w4<"), ("gemm_mx8.hip", "gemm_common.h", "mx.h")),
}
COPY_KERNEL = "copyBuffer"  # the HIP runtime's device-to-device copy kernel


def code_of(text: str) -> str:
    """C/C++ source without its comments and with whitespace runs collapsed:
    an edit to a comment leaves it, and so a recorded profile, unchanged.
    (No string literal in these sources holds a comment marker.)"""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def gemm_source_hash(kernel: str = "bf16") -> str:
    """Hash of the code of a grouped GEMM's sources (the kernel and its shared
    helpers), comments left out."""
    h = hashlib.sha256()
    for name in KERNELS[kernel][1]:
        h.update(code_of(open(os.path.join(PKG, "csrc", name)).read()).encode())
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
    # FETCH_SIZE + WRITE_SIZE: requests that missed the L2, not HBM bytes
    res["l2_miss_bytes_per_launch"] = totals["fetch"] + totals["write"]
    res["l2_miss_bytes_per_launch_unscaled"] = (res["fetch_kib_per_launch_raw"] +
                                                res["write_kib_per_launch_raw"]) * 1024.0
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
    "k_route_bf16": r"k_route_bf16<", "k_aux": r"k_aux\b", "k_permute": r"k_permute<",
    "k_permute_mx8": r"k_permute_mx8<", "k_combine": r"k_combine<",
    "k_combine_mx8": r"k_combine_mx8<",
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


def clock(csv_path, title, cmd, out, xcds: int = 8, simds: int = 1024, peak_ghz: float = 2.4,
          copy_bytes: int = 1 << 30):
    """Markdown table of the grouped GEMMs' effective clock and MFMA use,
    from one `--pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE ...` run:
      - effective clock = GRBM_GUI_ACTIVE (shader-clock cycles, summed over
        the XCDs) / XCDs / the dispatch's duration; the run's calibration
        copy of copy_bytes, a memory-bound kernel, is listed as the check
        (it should read about the 2.4 GHz maximum);
      - MFMA busy per cycle = SQ_VALU_MFMA_BUSY_CYCLES / SIMDs / (effective
        clock x duration), and of the peak clock.  Their product is the
        fraction of dense MFMA peak."""
    pats = {"k_grouped_gemm_w4 (GEMM1, GELU)": r"k_grouped_gemm_w4<\s*0\s*,\s*1>",
            "k_grouped_gemm_w4 (GEMM2)": r"k_grouped_gemm_w4<\s*0\s*,\s*0>",
            "k_grouped_gemm_mx8w4 (GEMM1, GELU)": r"k_grouped_gemm_mx8w4<1>",
            "k_grouped_gemm_mx8w4 (GEMM2)": r"k_grouped_gemm_mx8w4<0>",
            "k_mfma_ceiling<0> (MFMA only, no memory)": r"k_mfma_ceiling<0>",
            "k_mfma_ceiling<1> (two alternating operand sets)": r"k_mfma_ceiling<1>",
            "k_mfma_ceiling<2> (one VALU instruction per MFMA)": r"k_mfma_ceiling<2>",
            "k_mfma_ceiling32 (32x32x16 MFMAs)": r"k_mfma_ceiling32",
            "k_permute (memory-bound)": r"k_permute<",
            "k_combine (memory-bound)": r"k_combine<"}
    per = collections.defaultdict(dict)
    for r in csv.DictReader(open(csv_path)):
        d = int(r["Dispatch_Id"])
        per[d]["name"] = r["Kernel_Name"]
        per[d]["dur"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        per[d][r["Counter_Name"]] = per[d].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    rows = {n: [] for n in pats}
    copies = []
    for d in sorted(per):
        v = per[d]
        if COPY_KERNEL in v["name"]:
            copies.append(v)
            continue
        for n, rx in pats.items():
            if re.search(rx, v["name"]):
                rows[n].append(v)
                break
    lines = [f"# {title}", "", "Command (run from the repository root on one MI355X):", "", "```",
             cmd, "```", "",
             f"Effective clock = GRBM_GUI_ACTIVE / {xcds} XCDs / dispatch duration (shader-clock "
             f"cycles); MFMA busy per cycle = SQ_VALU_MFMA_BUSY_CYCLES / {simds} SIMDs / "
             f"(clock x duration).  The first dispatch of each kernel is a warm-up and is left "
             f"out (counter runs serialise dispatches, so their durations run a little long).", "",
             "| kernel | dispatches | mean us | effective clock GHz | MFMA busy per cycle | "
             f"clock x busy / {peak_ghz} GHz |", "|---|---|---|---|---|---|"]
    big = [c for c in copies if c["dur"] > 100e-6]
    if big:
        c = max(big, key=lambda c: c["dur"])
        ghz = c["GRBM_GUI_ACTIVE"] / xcds / c["dur"] / 1e9
        lines.append(f"| device copy of {copy_bytes >> 20} MiB (check) | 1 | {c['dur'] * 1e6:.1f} | "
                     f"{ghz:.2f} | - | - |")
    for n, vs in rows.items():
        vs = vs[1:] if len(vs) > 1 else vs
        if not vs:
            continue
        dur = sum(v["dur"] for v in vs) / len(vs)
        ghz = sum(v["GRBM_GUI_ACTIVE"] / xcds / v["dur"] for v in vs) / len(vs) / 1e9
        mf = sum(v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for v in vs) / len(vs) / simds
        busy = mf / (ghz * 1e9 * dur) if mf else 0.0
        lines.append(f"| `{n}` | {len(vs)} | {dur * 1e6:.1f} | {ghz:.2f} | "
                     f"{busy:.1%} | {busy * ghz / peak_ghz:.1%} |")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


SQ_KERNELS = {"k_grouped_gemm_w4 (GEMM1, GELU)": r"k_grouped_gemm_w4<\s*0\s*,\s*1>",
              "k_grouped_gemm_w4 (GEMM2)": r"k_grouped_gemm_w4<\s*0\s*,\s*0>",
              "k_mfma_ceiling<0> (MFMA only)": r"k_mfma_ceiling<0>",
              "k_mfma_ceiling<1> (alternating operand sets)": r"k_mfma_ceiling<1>",
              "k_mfma_ceiling<2> (one VALU instruction per MFMA)": r"k_mfma_ceiling<2>",
              "k_mfma_ceiling32 (32x32x16 MFMAs)": r"k_mfma_ceiling32"}


def sq(csv_paths, title, cmd, out, xcds: int = 8, simds: int = 1024):
    """Markdown table of the grouped GEMM's instruction mix, waits and LDS
    conflicts beside the MFMA-only kernel's, from several `--pmc` passes of
    the same command (one csv per pass; counters summed over a dispatch's
    dimensions, averaged over a kernel's dispatches after the first):
      - clock = GRBM_GUI_ACTIVE / XCDs / duration; MFMA busy per cycle =
        SQ_VALU_MFMA_BUSY_CYCLES / SIMDs / (clock x duration);
      - instructions per MFMA: SQ_INSTS_VALU counts the MFMAs too, so the
        other VALU instructions are SQ_INSTS_VALU - SQ_INSTS_MFMA;
      - waits per wave-cycle: SQ_WAIT_ANY and SQ_WAIT_INST_ANY over
        SQ_WAVE_CYCLES (all three in quad-cycles);
      - LDS bank-conflict share: SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE."""
    acc = {n: collections.defaultdict(list) for n in SQ_KERNELS}
    for path in csv_paths:
        per = collections.defaultdict(dict)
        for r in csv.DictReader(open(path)):
            v = per[int(r["Dispatch_Id"])]
            v["name"] = r["Kernel_Name"]
            v["dur"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
            v[r["Counter_Name"]] = v.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        seen = collections.Counter()
        for d in sorted(per):
            v = per[d]
            for n, rx in SQ_KERNELS.items():
                if re.search(rx, v["name"]):
                    seen[n] += 1
                    if seen[n] > 1:  # the first dispatch of each kernel is a warm-up
                        for c, x in v.items():
                            if c != "name":
                                acc[n][c].append(x)
                    break
    mean = lambda xs: sum(xs) / len(xs) if xs else float("nan")
    lines = [f"# {title}", "", "Command (run from the repository root on one MI355X; one run per "
             "counter set):", "", "```", cmd, "```", "",
             "Counters summed over each dispatch's dimensions and averaged over a kernel's "
             "dispatches after the first.  Clock = GRBM_GUI_ACTIVE / 8 XCDs / duration; MFMA busy "
             "= SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (clock x duration); SQ_INSTS_VALU counts "
             "MFMAs too, so other VALU = SQ_INSTS_VALU - SQ_INSTS_MFMA; waits over SQ_WAVE_CYCLES "
             "(quad-cycles, as the waits); LDS conflict share = SQ_LDS_BANK_CONFLICT / "
             "SQ_LDS_IDX_ACTIVE.", "",
             "| kernel | clock GHz | MFMA busy | other VALU / MFMA | SALU / MFMA | LDS instr / MFMA "
             "| SQ_WAIT_ANY / wave-cycle | SQ_WAIT_INST_ANY / wave-cycle | LDS conflict share |",
             "|---|---|---|---|---|---|---|---|---|"]
    for n in SQ_KERNELS:
        m = {c: mean(xs) for c, xs in acc[n].items()}
        if not m:
            continue
        dur = m["dur"]
        ghz = m["GRBM_GUI_ACTIVE"] / xcds / dur / 1e9
        busy = m["SQ_VALU_MFMA_BUSY_CYCLES"] / simds / (ghz * 1e9 * dur)
        mf = m["SQ_INSTS_MFMA"]
        act = m["SQ_LDS_IDX_ACTIVE"]
        lines.append(
            f"| `{n}` | {ghz:.2f} | {busy:.1%} | {(m['SQ_INSTS_VALU'] - mf) / mf:.2f} | "
            f"{m['SQ_INSTS_SALU'] / mf:.2f} | {m['SQ_INSTS_LDS'] / mf:.2f} | "
            f"{m['SQ_WAIT_ANY'] / m['SQ_WAVE_CYCLES']:.1%} | "
            f"{m['SQ_WAIT_INST_ANY'] / m['SQ_WAVE_CYCLES']:.1%} | "
            + (f"{m['SQ_LDS_BANK_CONFLICT'] / act:.1%} |" if act else "- |"))
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
    short = lambda n: re.sub(r"\(.*", "", n.replace("(anonymous namespace)::", "")).replace("void ", "")[:70]
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
    m = sub.add_parser("clock")
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
    q = sub.add_parser("sq")
    q.add_argument("--csv", nargs="+", required=True, help="counter_collection.csv of each pass")
    q.add_argument("--title", required=True)
    q.add_argument("--command", required=True, help="the commands that produced the passes")
    q.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.cmd == "traffic":
        traffic(a.fetch, a.write, a.copy_bytes, a.workload, a.out, a.kernel)
    elif a.cmd == "hbm":
        hbm(a.fetch, a.write, a.copy_bytes, a.title, a.command, a.out)
    elif a.cmd == "stats":
        win = tuple(int(v) for v in a.window.split(":")) if a.window else None
        stats(a.stats, a.trace, a.bench_log, a.title, a.command, a.note, a.out, a.kernel,
              window=win)
    elif a.cmd == "sq":
        sq(a.csv, a.title, a.command, a.out)
    else:
        clock(a.csv, a.title, a.command, a.out)


if __name__ == "__main__":
    main()
