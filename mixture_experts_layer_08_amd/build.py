"""Build libmoe.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m mixture_experts_layer_08_amd.build   (always recompiles)

Objects go to _build/ at the repository root; the shared library is written
next to this file, where the binding loads it from.
"""

from __future__ import annotations

import concurrent.futures
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["route.hip", "permute.hip", "gemm.hip", "gemm_mx8.hip", "mxfp8.hip", "combine.hip",
           "backward.hip", "ceiling.hip", "api.hip"]
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
    # per-kernel register / scratch remarks, checked by check_resources()
    "-Rpass-analysis=kernel-resource-usage", "-fno-caret-diagnostics",
]

# Kernels whose LDS ring is kept in order by hand-counted `s_waitcnt vmcnt`
# waits: those counts assume the LDS-direct loads are the only vector-memory
# instructions in the K loop.  A register spill would add scratch loads and
# stores to the count and release a wait before its stage has landed, so the
# build refuses any scratch use or spill in them.
NO_SCRATCH_KERNELS = ("k_grouped_gemm_bf16", "k_grouped_gemm_w4", "k_grouped_gemm_mx8")


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libmoe.so")


_REMARK = re.compile(r"remark:\s+(Function Name|ScratchSize \[bytes/lane\]|VGPRs Spill|SGPRs Spill|"
                     r"VGPRs|AGPRs|Occupancy \[waves/SIMD\]):\s*(\S+)")


def resource_usage(remarks: str) -> dict:
    """{kernel symbol: {field: value}} from hipcc's kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in remarks.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key] = val
    return out


def check_resources(usage: dict) -> None:
    """Refuse scratch or spills in the kernels of NO_SCRATCH_KERNELS."""
    bad = []
    for sym, f in usage.items():
        if not any(k in sym for k in NO_SCRATCH_KERNELS):
            continue
        for key in ("ScratchSize [bytes/lane]", "VGPRs Spill", "SGPRs Spill"):
            if f.get(key, "0") != "0":
                bad.append(f"{sym}: {key} = {f[key]}")
    if bad:
        raise RuntimeError("kernels with hand-counted vmcnt waits must not use scratch:\n  "
                           + "\n  ".join(bad))


def _compile(src: str):
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    # surface warnings other than hipcc's note about the host-side feature
    # flag and the resource remarks
    noise = ("packed-fp32-ops", "not a recognized feature", "warning generated",
             "warnings generated", "kernel-resource-usage")
    msgs = [l for l in r.stderr.splitlines() if l.strip() and not any(n in l for n in noise)]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj, resource_usage(r.stderr)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    usage = {k: v for _, u in results for k, v in u.items()}
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        for sym in sorted(usage):
            f.write(sym + " " + " ".join(f"{k}={v}" for k, v in usage[sym].items()) + "\n")
    check_resources(usage)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    build_c_example(verbose)
    return LIB


C_EXAMPLE_SRC = os.path.join(ROOT, "tests", "c_abi", "forward.c")
C_EXAMPLE = os.path.join(ROOT, "tests", "c_abi", "forward")


def build_c_example(verbose: bool = True) -> str:
    """The plain-C forward of tests/c_abi (host code only: gcc, the HIP
    runtime API and libmoe.so, found next to it through an $ORIGIN rpath)."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no host C compiler for the C example")
    rel = os.path.relpath(PKG, os.path.dirname(C_EXAMPLE))
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           C_EXAMPLE_SRC, "-o", C_EXAMPLE, "-L", PKG, "-lmoe", "-L", os.path.join(rocm, "lib"),
           "-lamdhip64", f"-Wl,-rpath,$ORIGIN/{rel}", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C example build failed:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {C_EXAMPLE}")
    return C_EXAMPLE


if __name__ == "__main__":
    build()
