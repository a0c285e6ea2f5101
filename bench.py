"""Benchmark of the MoE-layer forward on one MI355X.

A step is one whole forward (moe_route -> moe_aux_loss -> moe_permute ->
moe_expert_ffn -> moe_combine) over one batch of seeded synthetic tokens,
with inputs, weights and buffers resident in HBM before the timed region.
Default workload: T=32768 tokens (seq 4096 x micro-batch 8), H=4096, E=8,
top-2, h_exp=14336, bf16, capacity factor 1.25 (the worked example of the
cf-1.com page "Dissecting the MoE communication bottleneck", section 2.2).

Prints one JSON line: tokens/s of the whole forward, the roofline of the
dominant kernel (the grouped GEMM, timed with HIP events on its launch stream
over the timed region), permute / combine / router bandwidth, and the CPU
oracle (one warm-up, the median of three runs; the large workloads' FFN
extrapolated from a 2048-token sample).  Other objects on the same line: the
other workloads and one GPU's share under 8-way expert parallelism
(``configs``), the MXFP8 forward (``mxfp8``), the training step
(``backward``: a MOE_FLAG_TRAIN forward, then the four backward calls), the
noisy router and the pages' dense-FFN sanity ratio.  The headline value
stays the bf16 forward.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/s on 1 GPU + grouped-GEMM MFMA% and permute HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector / MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral_bf16")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample-tokens", type=int, default=2048)
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads and the EP-8 one-GPU share")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the training-step (forward + backward) leg")
    ap.add_argument("--backward-steps", type=int, default=10)
    ap.add_argument("--alpha", type=float, default=0.01,
                    help="aux-loss coefficient of the backward leg")
    ap.add_argument("--no-side-legs", action="store_true",
                    help="skip the noisy-router and dense-FFN comparisons (counter runs)")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the MXFP8-forward leg")
    ap.add_argument("--fp8-steps", type=int, default=20)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="after the timed region, run one device copy of BYTES bytes "
                         "(the known-size kernel that calibrates HBM counters)")
    return ap.parse_args()


def traffic_from_profile(workload: str, kernel: str = "bf16"):
    """L2-miss bytes per grouped-GEMM launch (FETCH_SIZE + WRITE_SIZE,
    calibrated on a device copy) from the committed rocprofv3 --pmc summary,
    if it was taken on the current kernel source; else None."""
    stem = "grouped_gemm" if kernel == "bf16" else f"grouped_gemm_{kernel}"
    p = os.path.join(ROOT, "profiles", f"{stem}_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    from mixture_experts_layer_08_amd.profiling import gemm_source_hash
    if d.get("gemm_source_sha256_16") != gemm_source_hash(kernel):
        return None
    return d.get("l2_miss_bytes_per_launch")


def _median_time(fn, runs: int = 3) -> float:
    """One untimed warm-up call, then the median wall time of `runs` calls."""
    fn()
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(sorted(ts)[len(ts) // 2])


def cpu_baseline(w, p, dev, n_sample: int = 2048, runs: int = 3):
    """The oracle, as it stands, timed on the host's cores: one warm-up, then
    the median of `runs` runs.

    The small workloads (tiny_fp32, small_bf16) run the whole float64 oracle
    forward.  The large ones (mixtral_bf16, finegrained_bf16, skewed_bf16)
    run the oracle's routing and row map over all T tokens, and the expert
    FFN plus combine on a seeded sample of `n_sample` tokens; their rate
    is extrapolated to T (labelled "extrapolated").  The headline value is
    the bench workload's."""
    import numpy as np
    import threadpoolctl
    import torch

    from mixture_experts_layer_08_amd.inputs import WORKLOADS, make_inputs, sample_tokens
    from oracle import moe_oracle as O

    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    f = lambda t: None if t is None else t.detach().cpu().to(torch.float32).numpy()
    per = {}
    for name in ("tiny_fp32", "small_bf16", "mixtral_bf16", "finegrained_bf16", "skewed_bf16"):
        wl = WORKLOADS[name]
        pp = p if name == w.name else make_inputs(wl, seed=0, device=dev)
        x, wr, br = f(pp["x"]), f(pp["w_r"]), f(pp["b_r"])
        w1, w2, ws1, ws2 = f(pp["w1"]), f(pp["w2"]), f(pp["ws1"]), f(pp["ws2"])
        if name in ("tiny_fp32", "small_bf16"):
            t = _median_time(lambda: O.forward(x, wr, br, w1, w2, ws1, ws2, K=wl.K, cf=wl.cf),
                             runs)
            per[name] = {"tokens_per_s": wl.T / t, "median_s": t, "runs": runs,
                         "how": "whole oracle forward"}
        else:
            def route_all():
                l = O.router_logits(x, wr, br).astype(np.float32).astype(np.float64)
                return O.route(l, wl.E, wl.K, wl.cf)

            t_route = _median_time(route_all, runs)
            r = route_all()
            toks = sample_tokens(wl.T, n_sample, seed=2).numpy()
            t_ffn = _median_time(lambda: O.forward_tokens(x, w1, w2, ws1, ws2, r, toks), runs)
            t_all = t_route + t_ffn * wl.T / len(toks)
            per[name] = {"tokens_per_s": wl.T / t_all, "extrapolated": True,
                         "route_median_s": t_route, "ffn_combine_sample_median_s": t_ffn,
                         "sample_tokens": int(len(toks)), "runs": runs,
                         "how": (f"router GEMM, routing and row map over all {wl.T} tokens, "
                                 f"plus expert FFN and combine of {len(toks)} sampled tokens "
                                 f"scaled to {wl.T}")}
        del x, w1, w2, ws1, ws2
        if name != w.name:
            del pp
            torch.cuda.empty_cache()
    head = per.get(w.name)
    return {
        "value": head["tokens_per_s"], "unit": "tokens/s", "cores": threads, "kind": "oracle",
        "sample": (f"{w.name}: " + head["how"] + f"; one warm-up then the median of {runs} runs; "
                   f"BLAS threads {threads}, host cpu_count {os.cpu_count()}"),
        "extrapolated": bool(head.get("extrapolated", False)),
        "configs": per,
    }


def mxfp8_leg(w, p, dev, steps: int, warmup: int) -> dict:
    """The MXFP8 forward (FP8 dispatch, expert GEMMs and combine; routing
    unchanged), each call bracketed by HIP events on the launch stream.  The
    expert weights are quantised once before the timed region, as a model
    would store them."""
    import torch

    from mixture_experts_layer_08_amd import counters, layer

    stream = torch.cuda.current_stream()
    mw = layer.MxWeights.quantize(w, p, stream)
    buf = layer.MxBuffers.allocate(w, device=dev)
    for _ in range(warmup):
        layer.forward_mxfp8(buf, p, mw, stream)
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    marks = [[ev() for _ in range(6)] for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        m = marks[s]
        m[0].record(stream)
        layer.route(buf, p, stream)
        m[1].record(stream)
        layer.aux_loss(buf, stream)
        m[2].record(stream)
        layer.permute_mxfp8(buf, p, stream)
        m[3].record(stream)
        layer.expert_ffn_mxfp8(buf, mw, stream)
        m[4].record(stream)
        layer.combine_mxfp8(buf, stream)
        m[5].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def stage_ms(i):
        return sum(marks[s][i].elapsed_time(marks[s][i + 1]) for s in range(steps)) / steps

    route_ms, aux_ms, perm_ms, ffn_ms, comb_ms = (stage_ms(i) for i in range(5))
    N = int(buf.offsets[-1].item())
    launches = 2 + (2 if w.hs else 0)
    flop = 2 * counters.grouped_gemm_flop_per_launch(N, w.H, w.h)
    if w.hs:
        flop += 2 * counters.grouped_gemm_flop_per_launch(w.T, w.H, w.hs)
    tflops = flop / (ffn_ms * 1e-3) / 1e12
    perm_bytes = counters.permute_mx8_bytes(w.T, N, w.H, w.K, bool(w.hs))
    comb_bytes = counters.combine_mx8_bytes(w.T, N, w.H, w.K, bool(w.hs))
    gbs = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9
    step_ms = wall * 1e3 / steps
    return {
        "tokens_per_s": w.T / (step_ms * 1e-3),
        "ms_per_step": step_ms,
        "steps": steps,
        "stages_ms": {"route": route_ms, "aux_loss": aux_ms, "permute_mxfp8": perm_ms,
                      "expert_ffn_mxfp8": ffn_ms, "combine_mxfp8": comb_ms},
        "grouped_gemm": {"kernel": "k_grouped_gemm_mx8w4", "bound": "mfma", "achieved": tflops,
                         "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                         "frac": tflops / PEAK_FP8_TFLOPS, "flop_per_launch": flop / launches,
                         "traffic": traffic_from_profile(w.name, "mx8"),
                         "avg_launch_ms": ffn_ms / launches},
        "hbm": {
            "permute_mxfp8": {"GB/s": gbs(perm_bytes, perm_ms),
                              "frac": gbs(perm_bytes, perm_ms) / PEAK_HBM_GBS,
                              "bytes": perm_bytes},
            "combine_mxfp8": {"GB/s": gbs(comb_bytes, comb_ms),
                              "frac": gbs(comb_bytes, comb_ms) / PEAK_HBM_GBS,
                              "bytes": comb_bytes},
        },
        "format": "MXFP8: E4M3 codes, one E8M0 scale per 32 values along the contraction",
    }


def router_noise_leg(w, p, dev, steps: int) -> dict:
    """The router stage with the noisy-router variant (Gumbel noise from the
    on-device Philox stream, temperature 1.2) against the plain router, on
    the same inputs; HIP events on the launch stream, the noise offset
    advancing every step as in training."""
    import torch

    from mixture_experts_layer_08_amd import layer

    stream = torch.cuda.current_stream()
    plain = layer.MoeBuffers.allocate(w, device=dev)
    noisy = layer.MoeBuffers.allocate(w, device=dev, router_tau=1.2, noise=(2024, 0))

    def time_route(buf, advance):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for i in range(3):
            layer.route(buf, p, stream)
        ev[0].record(stream)
        for i in range(steps):
            if advance:
                buf.shape.noise_offset = i
            layer.route(buf, p, stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / steps

    ms_plain = time_route(plain, False)
    ms_noisy = time_route(noisy, True)
    return {"route_ms_plain": ms_plain, "route_ms_gumbel_tau1.2": ms_noisy,
            "note": "moe_route (router GEMM, noise, softmax, top-k, block histograms)"}


def mfma_ceiling_leg(dev, gemm_tflops: float, peak: float, runs: int = 5) -> dict:
    """The MFMA-only rate of the grouped GEMM's inner loop (moe_mfma_ceiling):
    one workgroup of four waves per CU (one wave per SIMD, as the four-wave
    GEMM kernel), 64 v_mfma_f32_16x16x32_bf16 per round on random operands
    held in registers, no memory traffic.  Under this load the chip holds a
    clock below the 2.4 GHz the nominal peak assumes, so the rate is the
    practical ceiling the GEMM's rate is read against.  Also timed: two
    alternating operand sets (every sign and mantissa bit switching between
    rounds) and a zero-word XOR of every operand per round (one VALU
    instruction per MFMA).  Median of `runs` each."""
    import torch

    from mixture_experts_layer_08_amd import binding as B

    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    g = torch.Generator(device=dev).manual_seed(7)
    ops = torch.randn((16, 64, 8), generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty((cus * 256 * 4,), dtype=torch.float32, device=dev)
    iters = 20000
    flop = 2.0 * 16 * 16 * 32 * 64 * iters * 4 * cus
    stream = torch.cuda.current_stream()

    out32 = torch.empty((cus * 256 * 16,), dtype=torch.float32, device=dev)  # mode 3

    def median_ms(mode: int) -> float:
        o = out32 if mode == 3 else out
        B.moe_mfma_ceiling(ops, o, cus, iters // 10, mode, stream)  # warm-up
        times = []
        for _ in range(runs):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            B.moe_mfma_ceiling(ops, o, cus, iters, mode, stream)
            ev[1].record(stream)
            torch.cuda.synchronize()
            times.append(ev[0].elapsed_time(ev[1]))
        return sorted(times)[len(times) // 2]

    ms, ms_alt, ms_xor, ms_32 = median_ms(0), median_ms(1), median_ms(2), median_ms(3)
    tf, tf_alt, tf_xor, tf_32 = (flop / (t * 1e-3) / 1e12 for t in (ms, ms_alt, ms_xor, ms_32))
    return {"tflops": tf, "frac_of_peak": tf / peak, "ms": ms,
            "tflops_alternating_sets": tf_alt, "tflops_one_valu_per_mfma": tf_xor,
            "tflops_32x32x16": tf_32,
            "iters": iters, "workgroups": cus, "gemm_frac_of_ceiling": gemm_tflops / tf,
            "note": "MFMA-only loop of the four-wave GEMM's shape on random register operands "
                    "(moe_mfma_ceiling mode 0); tflops_alternating_sets: mode 1, every sign and "
                    "mantissa bit switching between rounds; tflops_one_valu_per_mfma: mode 2; "
                    "tflops_32x32x16: mode 3, the same work on 32x32x16 MFMAs; "
                    "gemm_frac_of_ceiling = roofline.achieved / tflops"}


def dense_ffn_ratio(w, p, dev, fwd_ms: float, steps: int) -> dict:
    """The pages' single-GPU sanity check: the MoE forward's time over that of
    one dense FFN of the same T, H, h (expert 0's weights) run through the
    same grouped-GEMM kernel as a single segment of all T tokens (E = K = 1,
    no capacity limit).  Top-2 does twice the dense FLOPs, so the ideal
    ratio is about 2."""
    import torch

    from mixture_experts_layer_08_amd import binding as B
    from mixture_experts_layer_08_amd.inputs import Workload

    d = Workload("dense", T=w.T, H=w.H, E=1, K=1, h=w.h, cf=0.0, dtype=w.dtype)
    s = B.make_shape(d.T, d.H, 1, 1, d.h, 0, 0.0, B.MOE_BF16 if w.dtype == "bf16" else B.MOE_F32)
    dt = w.torch_dtype()
    offsets = torch.tensor([0, w.T], dtype=torch.int32, device=dev)
    hbuf = torch.empty((w.T, w.h), dtype=dt, device=dev)
    out = torch.empty((w.T, w.H), dtype=dt, device=dev)
    ws = torch.empty((B.moe_workspace_size(s),), dtype=torch.uint8, device=dev)
    w1, w2 = p["w1"][:1], p["w2"][:1]
    stream = torch.cuda.current_stream()
    for _ in range(2):
        B.moe_expert_ffn(s, p["x"], offsets, w1, w2, hbuf, out, None, None, None, None, None, ws,
                         stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(steps):
        B.moe_expert_ffn(s, p["x"], offsets, w1, w2, hbuf, out, None, None, None, None, None, ws,
                         stream)
    ev[1].record(stream)
    torch.cuda.synchronize()
    dense_ms = ev[0].elapsed_time(ev[1]) / steps
    return {"dense_ffn_ms": dense_ms, "moe_forward_ms": fwd_ms, "ratio": fwd_ms / dense_ms,
            "top_k": w.K, "note": "MoE forward / dense FFN of the same T, H, h (one segment)"}


def backward_leg(w, p, dev, steps: int, warmup: int, alpha: float) -> dict:
    """Training step: forward with MOE_FLAG_TRAIN, then combine -> route ->
    expert FFN -> permute backward, each call bracketed by HIP events on the
    launch stream."""
    import torch

    from mixture_experts_layer_08_amd import counters, layer
    from mixture_experts_layer_08_amd.inputs import make_grad_output

    buf = layer.MoeBuffers.allocate(w, device=dev, train=True)
    g = layer.GradBuffers.allocate(w, device=dev)
    dy = make_grad_output(w, seed=0, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        layer.forward(buf, p, stream)
        layer.backward(buf, g, p, dy, alpha, stream)
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    marks = [[ev() for _ in range(6)] for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        m = marks[s]
        m[0].record(stream)
        layer.forward(buf, p, stream)
        m[1].record(stream)
        layer.combine_backward(buf, g, dy, stream)
        m[2].record(stream)
        layer.route_backward(buf, g, p, alpha, stream)
        m[3].record(stream)
        layer.expert_ffn_backward(buf, g, p, dy, stream)
        m[4].record(stream)
        layer.permute_backward(buf, g, p, stream)
        m[5].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def stage_ms(i):
        return sum(marks[s][i].elapsed_time(marks[s][i + 1]) for s in range(steps)) / steps

    fwd_ms, comb_ms, route_ms, ffn_ms, perm_ms = (stage_ms(i) for i in range(5))
    N = int(buf.offsets[-1].item())
    b = 2 if w.dtype == "bf16" else 4
    # four GEMMs per expert FFN backward (d u, d W2, d W1, d xp), 2*N*H*h each
    flop = 4 * counters.grouped_gemm_flop_per_launch(N, w.H, w.h)
    if w.hs:
        flop += 4 * counters.grouped_gemm_flop_per_launch(w.T, w.H, w.hs)
    comb_bytes = w.T * w.H * b + 2 * N * w.H * b
    perm_bytes = N * w.H * b + w.T * w.H * b * (3 if w.hs else 2)
    step_ms = wall * 1e3 / steps
    return {
        "training_tokens_per_s": w.T / (step_ms * 1e-3),
        "ms_per_training_step": step_ms,
        "steps": steps,
        "alpha": alpha,
        "stages_ms": {"forward_train": fwd_ms, "combine_backward": comb_ms,
                      "route_backward": route_ms, "expert_ffn_backward": ffn_ms,
                      "permute_backward": perm_ms},
        "expert_ffn_backward_tflops": flop / (ffn_ms * 1e-3) / 1e12,
        "expert_ffn_backward_frac_of_peak": flop / (ffn_ms * 1e-3) / 1e12 /
        (PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS),
        "combine_backward_GBs": comb_bytes / (comb_ms * 1e-3) / 1e9,
        "permute_backward_GBs": perm_bytes / (perm_ms * 1e-3) / 1e9,
        "note": "expert_ffn_backward: d u (NT + GELU'), d W2 and d W1 (TN, fp32 out), d xp (NT); "
                "permute_backward includes the d_logits W_r^T GEMM accumulated into dx",
    }


def time_forward(w, p, dev, steps: int, warmup: int, buf=None) -> dict:
    """The five calls of the forward, `warmup` untimed steps then `steps`
    timed ones; each call bracketed by HIP events on the launch stream.
    Returns per-stage mean times, the wall time per step, and the roofline
    figures of the grouped GEMM and the bandwidth-bound stages."""
    import torch

    from mixture_experts_layer_08_amd import counters, layer

    buf = buf or layer.MoeBuffers.allocate(w, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        layer.forward(buf, p, stream)
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    marks = [[ev() for _ in range(6)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        m = marks[s]
        m[0].record(stream)
        layer.route(buf, p, stream)
        m[1].record(stream)
        layer.aux_loss(buf, stream)
        m[2].record(stream)
        layer.permute(buf, p, stream)
        m[3].record(stream)
        layer.expert_ffn(buf, p, stream)
        m[4].record(stream)
        layer.combine(buf, stream)
        m[5].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def stage_ms(i):
        return sum(marks[s][i].elapsed_time(marks[s][i + 1]) for s in range(steps)) / steps

    route_ms, aux_ms, perm_ms, ffn_ms, comb_ms = (stage_ms(i) for i in range(5))
    ms_step = wall * 1e3 / steps
    N = int(buf.offsets[-1].item())
    b = 2 if w.dtype == "bf16" else 4
    launches = 2 + (2 if w.hs else 0)
    flop_step = 2 * counters.grouped_gemm_flop_per_launch(N, w.H, w.h)
    if w.hs:
        flop_step += 2 * counters.grouped_gemm_flop_per_launch(w.T, w.H, w.hs)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    achieved = flop_step / (ffn_ms * 1e-3) / 1e12
    kept = buf.kept.cpu().tolist()
    t_f, t_b, t_seg = counters.segment_roofline_s(kept, w.H, w.h, b, peak * 1e12,
                                                  PEAK_HBM_GBS * 1e9, w.T if w.hs else 0, w.hs)
    gbs = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9
    perm_bytes = counters.permute_bytes(w.T, N, w.H, b, w.K)
    comb_bytes = counters.combine_kernel_bytes(w.T, N, w.H, b, w.K, bool(w.hs))
    route_bytes = counters.router_bytes(w.T, w.H, w.E, w.K, b)
    return {
        "buf": buf, "N": N, "ms_step": ms_step, "tokens_per_s": w.T / (ms_step * 1e-3),
        "stages_ms": {"route": route_ms, "aux_loss": aux_ms, "permute": perm_ms,
                      "expert_ffn": ffn_ms, "combine": comb_ms},
        "gemm": {"achieved": achieved, "peak": peak, "frac": achieved / peak,
                 "flop_per_launch": flop_step / launches, "avg_launch_ms": ffn_ms / launches},
        "expert_ffn_roofline": {"flop_bound_ms": t_f * 1e3, "byte_bound_ms": t_b * 1e3,
                                "segment_bound_ms": t_seg * 1e3, "measured_ms": ffn_ms,
                                "frac_of_segment_bound": t_seg * 1e3 / ffn_ms},
        "hbm": {
            "permute": {"GB/s": gbs(perm_bytes, perm_ms),
                        "frac": gbs(perm_bytes, perm_ms) / PEAK_HBM_GBS, "bytes": perm_bytes},
            "combine": {"GB/s": gbs(comb_bytes, comb_ms),
                        "frac": gbs(comb_bytes, comb_ms) / PEAK_HBM_GBS, "bytes": comb_bytes},
            "route": {"GB/s": gbs(route_bytes, route_ms),
                      "frac": gbs(route_bytes, route_ms) / PEAK_HBM_GBS, "bytes": route_bytes},
        },
    }


def configs_leg(w_main, dev, steps: int, warmup: int) -> dict:
    """The other workloads, each timed as the headline one (fewer steps), and
    the expert FFN of one GPU's share under 8-way expert parallelism at the
    headline shape: one expert's segment of T*K rows (65536 at T=32768,
    top-2), H x h_exp, through the same grouped GEMM."""
    import torch

    from mixture_experts_layer_08_amd import binding as B
    from mixture_experts_layer_08_amd import counters
    from mixture_experts_layer_08_amd.inputs import WORKLOADS, make_inputs

    out = {}
    for name in ("tiny_fp32", "small_bf16", "mixtral_bf16", "finegrained_bf16", "skewed_bf16"):
        if name == w_main.name:
            continue
        wl = WORKLOADS[name]
        p = make_inputs(wl, seed=0, device=dev)
        r = time_forward(wl, p, dev, steps, warmup)
        out[name] = {
            "tokens_per_s": r["tokens_per_s"], "ms_per_step": r["ms_step"],
            "kept_rows": r["N"], "stages_ms": r["stages_ms"],
            "grouped_gemm_frac_of_peak": r["gemm"]["frac"],
            "grouped_gemm_tflops": r["gemm"]["achieved"],
            "frac_of_segment_bound": r["expert_ffn_roofline"]["frac_of_segment_bound"],
            "segment_bound_ms": r["expert_ffn_roofline"]["segment_bound_ms"],
            "hbm_frac": {k: v["frac"] for k, v in r["hbm"].items()},
        }
        del r, p
        torch.cuda.empty_cache()

    # EP-8 one-GPU share: a single segment of T*K rows through moe_expert_ffn
    wm = WORKLOADS["mixtral_bf16"]
    rows = wm.T * wm.K
    s = B.make_shape(rows, wm.H, 1, 1, wm.h, 0, 0.0, B.MOE_BF16)
    g = torch.Generator(device=dev).manual_seed(0)
    xp = (torch.randn((rows, wm.H), generator=g, device=dev)).to(torch.bfloat16)
    w1 = (torch.randn((1, wm.H, wm.h), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    w2 = (torch.randn((1, wm.h, wm.H), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    offsets = torch.tensor([0, rows], dtype=torch.int32, device=dev)
    hbuf = torch.empty((rows, wm.h), dtype=torch.bfloat16, device=dev)
    o = torch.empty((rows, wm.H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((B.moe_workspace_size(s),), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    call = lambda: B.moe_expert_ffn(s, xp, offsets, w1, w2, hbuf, o, None, None, None, None,
                                    None, ws, stream)
    for _ in range(2):
        call()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    n = 5
    ev[0].record(stream)
    for _ in range(n):
        call()
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / n
    flop = 2 * counters.grouped_gemm_flop_per_launch(rows, wm.H, wm.h)
    tf = flop / (ms * 1e-3) / 1e12
    out["ep8_share_mixtral"] = {
        "rows": rows, "H": wm.H, "h_exp": wm.h, "expert_ffn_ms": ms, "tflops": tf,
        "frac_of_peak": tf / PEAK_BF16_TFLOPS,
        "note": "one GPU's expert FFN under 8-way expert parallelism at T=32768, top-2: "
                "one expert, one segment of T*K rows (GEMM1 + GELU, GEMM2); no all-to-all"}
    del xp, w1, w2, hbuf, o, ws
    torch.cuda.empty_cache()
    return out


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only: the layer forward runs on one GPU's token "
              f"batch and has no multi-GPU path, so --gpus {a.gpus} is refused.", file=sys.stderr)
        sys.exit(2)

    import torch

    from mixture_experts_layer_08_amd import binding as B
    from mixture_experts_layer_08_amd import counters, layer
    from mixture_experts_layer_08_amd.inputs import WORKLOADS, make_inputs

    w = WORKLOADS[a.workload]
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    p = make_inputs(w, seed=a.seed, device=dev)
    r = time_forward(w, p, dev, a.steps, a.warmup)
    buf, N, ms_step = r["buf"], r["N"], r["ms_step"]
    dropped = int(buf.n_dropped.item())
    # dominant kernel: the grouped GEMM, launched twice per step (GEMM1 with
    # GELU, GEMM2) plus twice more for the shared expert when present
    gm = r["gemm"]
    traffic = traffic_from_profile(w.name)
    ffn_roofline = dict(r["expert_ffn_roofline"],
                        note="segment bound: sum over expert segments of max(FLOP / MFMA peak, "
                             "(weights + activations) bytes / HBM peak)")
    hbm = r["hbm"]
    hbm["permute"]["note"] = "moe_permute: one kernel (row map and copy)"
    hbm["route"]["note"] = "moe_route: one kernel (router GEMM, softmax, top-k, block partials)"
    hbm["aux_loss_ms"] = r["stages_ms"]["aux_loss"]

    res = {
        "metric": METRIC,
        "value": w.T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) tokens, N(0,0.02) weights, drawn on the GPU)",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "E": w.E, "top_k": w.K,
                   "h_exp": w.h, "h_shared": w.hs, "capacity_factor": w.cf,
                   "kept_rows": N, "dropped_assignments": dropped,
                   "aux_loss": float(buf.aux.item())},
        "roofline": {"kernel": "k_grouped_gemm_w4" if w.dtype == "bf16" else "k_grouped_gemm_f32",
                     "bound": "mfma", "achieved": gm["achieved"], "peak": gm["peak"],
                     "unit": "TFLOP/s", "frac": gm["frac"], "traffic": traffic,
                     "traffic_note": "L2-miss bytes per launch (FETCH_SIZE + WRITE_SIZE, "
                                     "calibrated on a device copy), from the committed profile "
                                     "when it matches the kernel source; else null",
                     "flop_per_launch": gm["flop_per_launch"],
                     "avg_launch_ms": gm["avg_launch_ms"]},
        "expert_ffn_roofline": ffn_roofline,
        "stages_ms": r["stages_ms"],
        "hbm": hbm,
        "cpu_baseline": None,
    }
    if w.dtype == "bf16":
        res["mfma_ceiling"] = mfma_ceiling_leg(dev, gm["achieved"], gm["peak"])
    if not a.no_side_legs:
        res["router_noise"] = router_noise_leg(w, p, dev, 20)
        res["dense_ffn_sanity"] = dense_ffn_ratio(w, p, dev, ms_step, 10)
    if not a.no_fp8 and w.dtype == "bf16":
        res["mxfp8"] = mxfp8_leg(w, p, dev, a.fp8_steps, min(a.warmup, 3))
        torch.cuda.empty_cache()
    if not a.no_backward:
        del buf
        r.pop("buf", None)
        torch.cuda.empty_cache()
        res["backward"] = backward_leg(w, p, dev, a.backward_steps, min(a.warmup, 3), a.alpha)
    if a.copy_calibration > 0:
        n = a.copy_calibration // 4
        src = torch.empty(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not a.no_configs:
        res["configs"] = configs_leg(w, dev, min(a.steps, 20), min(a.warmup, 3))
        torch.cuda.empty_cache()
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, p, dev, a.cpu_sample_tokens)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
