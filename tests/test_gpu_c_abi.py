"""The C ABI from plain C: one forward with no PyTorch in the process.

tests/c_abi/forward.c (built by build() with gcc against include/moe.h,
libmoe.so and the HIP runtime API) reads the inputs from a file, runs the five
calls on one stream and writes every output to a file.  This test draws the
inputs on the host, runs the program as a child process and checks its
outputs against the oracle like the other parity tests: routing bit-exact on
the program's own fp32 logits, logits within the fp32-sum bound, y within
the bf16 tolerance.
"""

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from mixture_experts_layer_08_amd import binding as B
from mixture_experts_layer_08_amd.build import C_EXAMPLE
from mixture_experts_layer_08_amd.inputs import Workload, make_inputs
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("kw", [
    dict(T=1000, H=256, E=8, K=2, h=192, cf=1.25),
    dict(T=333, H=128, E=6, K=3, h=136, cf=0.5),
])
def test_forward_from_plain_c(tmp_path, kw):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(C_EXAMPLE):
        pytest.fail(f"{C_EXAMPLE} is missing: run the package build")
    w = Workload("c_abi", **kw)
    say(f"[C ABI forward] {w}")
    p = make_inputs(w, seed=12, device="cpu")
    raw = lambda t: t.contiguous().view(torch.int16).numpy().tobytes()
    hdr = np.array([w.T, w.H, w.E, w.K, w.h, 0, B.MOE_BF16, 0], dtype=np.int32)
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(hdr.tobytes())
        f.write(np.float32(w.cf).tobytes())
        for k in ("x", "w_r", "w1", "w2"):
            f.write(raw(p[k]))
    r = subprocess.run([C_EXAMPLE, str(inp), str(outp)], capture_output=True, text=True,
                       timeout=120)
    say("  " + (r.stdout.strip() or r.stderr.strip()))
    assert r.returncode == 0, r.stderr

    T, E, K, H = w.T, w.E, w.K, w.H
    buf = open(outp, "rb").read()
    pos = 0

    def take(n, dt):
        nonlocal pos
        a = np.frombuffer(buf, dtype=dt, count=n, offset=pos)
        pos += a.nbytes
        return a

    logits = take(T * E, np.float32).reshape(T, E)
    ids = take(T * K, np.int32).reshape(T, K)
    tw = take(T * K, np.float32).reshape(T, K)
    counts = take(E, np.int32)
    kept = take(E, np.int32)
    offsets = take(E + 1, np.int32)
    row_of = take(T * K, np.int32).reshape(T, K)
    n_dropped = int(take(1, np.int32)[0])
    aux = float(take(1, np.float32)[0])
    y16 = take(T * H, np.int16).reshape(T, H)
    assert pos == len(buf)

    f64 = lambda t: t.to(torch.float64).numpy()
    x, wr = f64(p["x"]), f64(p["w_r"])
    ref_l = x @ wr
    bound = 8 * np.sqrt(H) * 2.0 ** -24 * (np.abs(x) @ np.abs(wr)).max()
    assert np.abs(logits - ref_l).max() <= bound

    r_ = O.route(logits.astype(np.float64), E, K, w.cf)
    assert np.array_equal(ids, r_["ids"])
    assert np.array_equal(counts, r_["counts"]) and np.array_equal(kept, r_["kept"])
    assert np.array_equal(offsets, r_["offsets"]) and np.array_equal(row_of, r_["row_of"])
    assert n_dropped == r_["n_dropped"]
    assert np.abs(tw - r_["w"]).max() <= 1e-6
    assert abs(aux - r_["aux"]) <= 1e-5 * abs(r_["aux"])

    y = torch.from_numpy(y16.copy()).view(torch.bfloat16).to(torch.float64).numpy()
    f32 = lambda t: t.to(torch.float32).numpy()
    ref = O.forward_tokens(f32(p["x"]), f32(p["w1"]), f32(p["w2"]), None, None, r_, np.arange(T))
    err = np.abs(y - ref).max() / np.abs(ref).max()
    say(f"  routing bit-exact, dropped {n_dropped}, aux {aux:.4f}, y max rel err {err:.2e}")
    assert err <= TOL_BF16
