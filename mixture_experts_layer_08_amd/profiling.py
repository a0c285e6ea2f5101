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
    res["hbm_bytes_per_launch"] = totals["fetch"] + totals["write"]
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


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
    a = ap.parse_args()
    traffic(a.fetch, a.write, a.copy_bytes, a.workload, a.out, a.kernel)


if __name__ == "__main__":
    main()
