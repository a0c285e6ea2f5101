"""GPU parity of the MXFP8 forward against the MXFP8 oracle, through the C ABI.

Protocol:
  1. seeded inputs feed both sides; the GPU runs route -> aux_loss ->
     permute_mxfp8 -> expert_ffn_mxfp8 -> combine_mxfp8 with weights from
     moe_quantize_weights_mxfp8;
  2. routing is checked bit-exactly as in the bf16 tests (oracle routing from
     the GPU's fp32 logits);
  3. byte work is bit-exact: the quantised weights, the quantised dispatched
     rows (codes and scales) and the shared expert's quantised x;
  4. the FP8 results of the GEMMs (h, out, and the shared expert's) are
     quantised by both sides from float32 values that differ by accumulation
     order (and by the MFMA's internal precision), so a value near a rounding
     boundary may land on the neighbouring code.  Each is checked link by
     link of the chain, every value (tests/mx_checks.py):
       - h: every GPU code must be the round-to-nearest, at the GPU's own
         block scale, of some value within delta of the oracle's unquantised
         GELU output, and every block scale the shared exponent of a block
         maximum within delta of the oracle's; delta bounds the GPU's
         accumulation and GELU error (check_h_rounding).  A neighbouring code
         is therefore accepted only where the oracle's value lies within
         delta of the midpoint between the two codes.  On all rows with an
         upper bound of the per-step maxima from two matmuls, and on sampled
         rows with the exact maxima;
       - out: the same rule against the float64 product of the GPU's own
         dequantised h and the dequantised W2 (check_out_rounding), every row;
       - the shared expert's h and out likewise;
  5. y (bf16): every element equal to combine's definition on the GPU's own
     dequantised outputs (fp32 accumulation, one bf16 rounding); and against
     the oracle's whole FP8 layer, relative Frobenius error <= 1e-2.
"""

import sys

import numpy as np
import pytest
import torch

from mixture_experts_layer_08_amd import binding as B
from mixture_experts_layer_08_amd import layer
from mixture_experts_layer_08_amd.inputs import WORKLOADS, Workload, make_inputs, sample_tokens
from oracle import moe_oracle as O
from oracle import mxfp8_oracle as M
from tests.mx_checks import (accum_bounds, accum_bounds_fast, check_combine_definition,
                             check_h_rounding, check_mx_close, check_out_rounding)
from tests.test_gpu_parity import check_routing

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def np32(t):
    return None if t is None else t.detach().to("cpu").to(torch.float32).numpy()


def u8(t):
    return t.detach().cpu().numpy()


def unpanel(flat, G, K, N):
    """moe_quantize_weights_mxfp8's panel layout -> codes [G][N][K] (numpy):
    panels of 256 rows x 64 codes ordered (g, row block, K block)."""
    P = (N + 255) // 256
    a = u8(flat)[: G * P * 256 * K].reshape(G, P, K // 64, 256, 64)
    return a.transpose(0, 1, 3, 2, 4).reshape(G, P * 256, K)[:, :N, :]


def panel_rows(flat, G, K, N, cols):
    """Codes [G][len(cols)][K] of the given weight columns (rows of the
    transposed weights), gathered on the device by the panel formula."""
    P = (N + 255) // 256
    g = torch.arange(G, device=flat.device)[:, None, None]
    n = torch.as_tensor(cols, device=flat.device)[None, :, None]
    k = torch.arange(K, device=flat.device)[None, None, :]
    idx = ((g * P + n // 256) * (K // 64) + k // 64) * 16384 + (n % 256) * 64 + k % 64
    return u8(torch.take(flat, idx))


def op_rows(flat, R, Kd):
    """Operand-layout scales [ceil(Kd/128)][R][4] -> row layout [R][Kd/32]."""
    ns = (Kd + 127) // 128
    a = u8(flat)[: ns * R * 4].reshape(ns, R, 4).transpose(1, 0, 2).reshape(R, ns * 4)
    return a[:, : Kd // 32]


def run_mx(w: Workload, p: dict):
    mw = layer.MxWeights.quantize(w, p)
    buf = layer.MxBuffers.allocate(w)
    layer.forward_mxfp8(buf, p, mw)
    torch.cuda.synchronize()
    return buf, mw


def oracle_mx(w: Workload, p: dict, buf):
    l = buf.logits.cpu().numpy().astype(np.float64)
    return M.forward_mxfp8(np32(p["x"]), np32(p["w_r"]), None, np32(p["w1"]), np32(p["w2"]),
                           np32(p["ws1"]), np32(p["ws2"]), K=w.K, cf=w.cf, logits=l)


def check_h_sample(w, p, buf, ref, r, nmax, n_rows=256, seed=17):
    """check_h_rounding on up to n_rows packed rows (seeded, across segments)
    and, with a shared expert, on up to n_rows tokens of its h."""
    N = int(buf.offsets[-1].item())
    if N == 0:
        return
    rows = np.sort(np.random.default_rng(seed).choice(N, size=min(n_rows, N), replace=False))
    xd = M.mx_dequantize(ref["x_codes"], ref["x_scales"], axis=1)
    w1d = M.mx_dequantize(ref["w1_codes"], ref["w1_scales"], axis=1)
    off, tok = r["offsets"], r["token_of"]
    gc = u8(buf.h_q[:N])[rows]
    gs = op_rows(buf.h_s, nmax, w.h)[:N][rows]
    tmax = np.zeros((len(rows), w.h))
    tsum = np.zeros((len(rows), w.h))
    for e in range(w.E):
        m = (rows >= off[e]) & (rows < off[e + 1])
        if m.any():
            tmax[m], tsum[m] = accum_bounds(xd[tok[rows[m]]], w1d[e])
    check_h_rounding("h (sampled rows)", gc, gs, ref["h"][rows], tmax, tsum, w.H)
    if w.hs:
        ts = np.sort(np.random.default_rng(seed + 1).choice(w.T, size=min(n_rows, w.T),
                                                            replace=False))
        ws1d = M.mx_roundtrip(np32(p["ws1"]), axis=0)
        tmax, tsum = accum_bounds(xd[ts], ws1d)
        check_h_rounding("shared h (sampled tokens)", u8(buf.hsh_q)[ts],
                         op_rows(buf.hsh_s, w.T, w.hs)[ts], ref["sh_h"][ts], tmax, tsum, w.H)


def check_out_all(name, gc, gs, hd, w2d, off, E):
    """check_out_rounding on every packed row: the reference of segment e is
    the float64 product of the GPU's own dequantised h rows hd and expert
    e's dequantised W2 (w2d [E][h][H]); step maxima bounded by
    accum_bounds_fast."""
    R, n = gc.shape
    v = np.zeros((R, n))
    tmax = np.zeros((R, n))
    tsum = np.zeros((R, n))
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            v[a:b] = hd[a:b] @ w2d[e]
            tmax[a:b], tsum[a:b] = accum_bounds_fast(hd[a:b], w2d[e])
    check_out_rounding(name, gc, gs, v, tmax, tsum, hd.shape[1])
    return v


def check_forward(w: Workload, p: dict, buf, mw, ref=None):
    r = check_routing(w, buf)
    ref = ref if ref is not None else oracle_mx(w, p, buf)
    N = int(buf.offsets[-1].item())
    nmax = buf.xp_q.shape[0]
    tok = r["token_of"]
    off = r["offsets"]
    # byte work: bit-exact
    assert np.array_equal(u8(buf.xp_q[:N]), ref["x_codes"][tok]), "dispatched codes differ"
    assert np.array_equal(op_rows(buf.xp_s, nmax, w.H)[:N], ref["x_scales"][tok]), \
        "dispatched scales differ"
    if w.hs:
        assert np.array_equal(u8(buf.x_q), ref["x_codes"]), "shared-expert x codes differ"
        assert np.array_equal(op_rows(buf.x_s, w.T, w.H), ref["x_scales"])
    xd = M.mx_dequantize(ref["x_codes"], ref["x_scales"], axis=1)
    w1d = M.mx_dequantize(ref["w1_codes"], ref["w1_scales"], axis=1)
    w2d = M.mx_dequantize(ref["w2_codes"], ref["w2_scales"], axis=1)
    # h against the oracle's unquantised GELU output, every row (bounds of
    # the step maxima from accum_bounds_fast), then sampled rows with the
    # exact step maxima; the share of equal codes is reported too
    h_c, h_s = u8(buf.h_q[:N]), op_rows(buf.h_s, nmax, w.h)[:N]
    check_mx_close("h", h_c, h_s, ref["h_codes"], ref["h_scales"])
    if N:
        tmax = np.zeros((N, w.h))
        tsum = np.zeros((N, w.h))
        for e in range(w.E):
            a, b = int(off[e]), int(off[e + 1])
            if b > a:
                tmax[a:b], tsum[a:b] = accum_bounds_fast(xd[tok[a:b]], w1d[e])
        check_h_rounding("h (all rows)", h_c, h_s, ref["h"], tmax, tsum, w.H)
        del tmax, tsum
    check_h_sample(w, p, buf, ref, r, nmax)
    # out against the float64 product of the GPU's own h and W2, every row
    o_c, o_s = u8(buf.out_q[:N]), u8(buf.out_s[:N])
    hd = M.mx_dequantize(h_c, h_s, axis=1)
    if N:
        check_out_all("out (all rows)", o_c, o_s, hd, w2d, off, w.E)
    out_d = M.mx_dequantize(o_c, o_s, axis=1) if N else np.zeros((0, w.H))
    sh_d = None
    if w.hs:
        sh_hc, sh_hs = u8(buf.hsh_q), op_rows(buf.hsh_s, w.T, w.hs)
        check_mx_close("shared h", sh_hc, sh_hs, ref["sh_h_codes"], ref["sh_h_scales"])
        ws1d = M.mx_roundtrip(np32(p["ws1"]), axis=0)
        ws2d = M.mx_roundtrip(np32(p["ws2"]), axis=0)
        tmax, tsum = accum_bounds_fast(xd, ws1d)
        check_h_rounding("shared h (all tokens)", sh_hc, sh_hs, ref["sh_h"], tmax, tsum, w.H)
        check_out_all("shared out (all tokens)", u8(buf.sh_q), u8(buf.sh_s),
                      M.mx_dequantize(sh_hc, sh_hs, axis=1), ws2d[None], [0, w.T], 1)
        sh_d = M.mx_dequantize(u8(buf.sh_q), u8(buf.sh_s), axis=1)
    # y: combine's definition on the GPU's own outputs (every element), and
    # the whole layer against the oracle's float64 y
    got = buf.y.cpu().to(torch.float64).numpy()
    check_combine_definition("y", got, out_d, r["row_of"],
                             buf.topk_w.cpu().numpy().astype(np.float64), sh_d)
    want = ref["y"]
    err = float(np.abs(got - want).max()) / max(float(np.abs(want).max()), 1e-30)
    fro = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    say(f"  y vs the oracle's FP8 layer: max rel err {err:.3e}, relative Frobenius error "
        f"{fro:.3e} (tol 1e-2)")
    assert fro <= 1e-2
    return r, ref


# ---------------------------------------------------------------- byte work

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("G,K,N", [(3, 192, 96), (1, 64, 32), (2, 4096, 64)])
def test_quantize_weights_bit_exact(dtype, G, K, N):
    """Per-column magnitudes from 2^-30 to 2^30, a zero column, exact E4M3
    values at the top of the range, and ties: codes and scales bit-exact."""
    say(f"[quantize weights {dtype}] G={G} K={K} N={N}")
    g = torch.Generator().manual_seed(G * 1000 + K + N)
    w = torch.randn((G, K, N), generator=g) * torch.exp2(torch.randint(-30, 31, (G, 1, N),
                                                                       generator=g).float())
    w[:, :, 0] = 0.0
    w[0, :32, 1] = 448.0 * 2.0 ** -5
    w[0, 32:64, 1] = torch.tensor([1.0, 1.0625, 1.125, 1.1875] * 8)  # 1.0625: a tie
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    w = w.to(tdt)
    dev = w.to("cuda")
    nbytes = B.moe_mx_weight_code_bytes(G, K, N)
    assert nbytes == G * ((N + 255) // 256) * 256 * K
    q = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.empty((G * B.moe_mx_operand_scale_bytes(N, K),), dtype=torch.uint8, device="cuda")
    B.moe_quantize_weights_mxfp8(dev, B.MOE_BF16 if dtype == "bf16" else B.MOE_F32, G, K, N, q, s)
    torch.cuda.synchronize()
    rc, rs = M.quantize_weights(w.to(torch.float32).numpy())
    assert np.array_equal(unpanel(q, G, K, N), rc.transpose(0, 2, 1))
    # the padding rows of each slice's last panel are left as they were
    P = (N + 255) // 256
    full = u8(q).reshape(G, P, K // 64, 256, 64).transpose(0, 1, 3, 2, 4).reshape(G, P * 256, K)
    assert np.all(full[:, N:, :] == 0xA5)
    per = B.moe_mx_operand_scale_bytes(N, K)
    for e in range(G):
        assert np.array_equal(op_rows(s[e * per:(e + 1) * per], N, K), rs[e].T), f"scales {e}"


def test_dispatch_codes_bit_exact_and_extreme_rows():
    """Rows of zeros, rows scaled by 2^-40 .. 2^40, values that saturate: the
    dispatched codes and scales equal the oracle's quantisation of x."""
    w = Workload("extreme", T=300, H=192, E=5, K=2, h=64, hs=64, cf=1.0)
    say(f"[dispatch] {w}")
    p = make_inputs(w, seed=21, device="cuda")
    x = p["x"].float()
    g = torch.Generator(device="cuda").manual_seed(3)
    x *= torch.exp2(torch.randint(-40, 41, (w.T, 1), generator=g, device="cuda").float())
    x[7] = 0.0
    x[8, :32] = torch.tensor([480.0] + [1.0] * 31, device="cuda")  # 480 / 2^0 saturates
    p["x"] = x.to(torch.bfloat16)
    buf, mw = run_mx(w, p)
    check_forward(w, p, buf, mw)


# ---------------------------------------------------------------- whole forward

CASES = [
    ("tiny", dict(T=256, H=64, E=4, K=2, h=128, cf=0.0)),
    ("ragged_odd_ksteps", dict(T=333, H=192, E=6, K=3, h=320, hs=128, cf=0.9, bias="normal")),
    ("one_expert", dict(T=1000, H=128, E=1, K=1, h=64, cf=0.0)),
    ("wide_h_tail", dict(T=130, H=256, E=2, K=1, h=576, cf=0.0)),
    ("T1", dict(T=1, H=64, E=4, K=2, h=64, cf=1.25)),
    ("E256_K8", dict(T=130, H=64, E=256, K=8, h=64, cf=1.25)),
    ("C1_drops", dict(T=257, H=64, E=8, K=2, h=64, cf=0.01)),
    # one segment whose last 256-row tile holds 33, 161 and 224 rows: the two
    # row-waves of the GEMM own 1/1, 3/3 and 4/3 of its 32-row groups
    ("tail_33", dict(T=289, H=128, E=1, K=1, h=128, cf=0.0)),
    ("tail_161", dict(T=417, H=128, E=1, K=1, h=128, cf=0.0)),
    ("tail_224", dict(T=480, H=128, E=1, K=1, h=128, cf=0.0)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_forward_parity(name, kw):
    w = Workload(name, **kw)
    say(f"[mxfp8 {name}] {w}")
    p = make_inputs(w, seed=13, device="cuda")
    buf, mw = run_mx(w, p)
    check_forward(w, p, buf, mw)


def test_small_bf16_full_tensors():
    w = WORKLOADS["small_bf16"]
    say(f"[mxfp8 small_bf16] {w}")
    p = make_inputs(w, seed=0, device="cuda")
    buf, mw = run_mx(w, p)
    _, ref = check_forward(w, p, buf, mw)
    # distance from the bf16 layer (information: the cost of FP8)
    f = O.forward_tokens(np32(p["x"]), np32(p["w1"]), np32(p["w2"]), None, None,
                         O.route(buf.logits.cpu().numpy().astype(np.float64), w.E, w.K, w.cf),
                         np.arange(0, w.T, 16))
    d = np.linalg.norm(ref["y"][::16] - f) / np.linalg.norm(f)
    say(f"  FP8 layer vs float layer: relative Frobenius difference {d:.4f}")


def test_empty_experts_and_all_dropped_tokens():
    w = Workload("empty", T=400, H=64, E=8, K=2, h=64, cf=0.5)
    p = make_inputs(w, seed=3, device="cuda")
    p["b_r"] = torch.zeros(8, device="cuda")
    p["b_r"][:2] = 100.0
    buf, mw = run_mx(w, p)
    r, _ = check_forward(w, p, buf, mw)
    assert (r["kept"][2:] == 0).all() and (r["row_of"] < 0).all(1).sum() > 0


def test_determinism_bitwise():
    w = WORKLOADS["small_bf16"].replace(T=1000, cf=0.9)
    p = make_inputs(w, seed=5, device="cuda")
    a, _ = run_mx(w, p)
    b, _ = run_mx(w, p)
    for name in ("xp_q", "xp_s", "h_q", "h_s", "out_q", "out_s"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    assert torch.equal(a.y.view(torch.int16), b.y.view(torch.int16))


def _offset_copy(t, off):
    """A copy of byte tensor t that starts `off` bytes past a 16-byte boundary."""
    big = torch.zeros(t.numel() + 32, dtype=torch.uint8, device=t.device)
    base = (-big.data_ptr()) % 16
    v = big[base + off:base + off + t.numel()]
    v.copy_(t.reshape(-1))
    return v.view(t.shape)


@pytest.mark.parametrize("off", [4, 8, 12])
def test_misaligned_scale_pointers_bitwise(off):
    """Scale pointers need only 4-byte alignment: the GEMM loads the scale
    words of a tile from the pointer rounded down to 16 bytes and shifts its
    reads.  Every scale tensor of moe_expert_ffn_mxfp8 (inputs, weights and
    the h / shared-expert h it writes and reads back) moved `off` bytes off
    16-byte alignment gives bitwise the same codes and scales."""
    import dataclasses
    w = Workload("mis", T=600, H=256, E=8, K=2, h=192, hs=128, cf=1.25)
    p = make_inputs(w, seed=23, device="cuda")
    buf, mw = run_mx(w, p)
    print(f"[misaligned scales off={off}] {w}", flush=True)
    outs = ("h_q", "h_s", "out_q", "out_s", "hsh_q", "hsh_s", "sh_q", "sh_s")
    # reference: the aligned call again, into zeroed outputs (bytes the GEMMs
    # never write then compare equal)
    ref = dataclasses.replace(buf, **{n: torch.zeros_like(getattr(buf, n)) for n in outs})
    layer.expert_ffn_mxfp8(ref, mw)
    mb = dataclasses.replace(
        buf, **{n: _offset_copy(getattr(buf, n), off) for n in ("xp_s", "x_s")},
        **{n: torch.zeros_like(getattr(buf, n)) for n in ("h_q", "out_q", "hsh_q", "sh_q")},
        **{n: _offset_copy(torch.zeros_like(getattr(buf, n)), off)
           for n in ("h_s", "out_s", "hsh_s", "sh_s")})
    mm = dataclasses.replace(
        mw, **{n: _offset_copy(getattr(mw, n), off) for n in ("w1_s", "w2_s", "ws1_s", "ws2_s")})
    for t in (mb.xp_s, mb.h_s, mm.w1_s, mm.w2_s):
        assert t.data_ptr() % 16 == off
    layer.expert_ffn_mxfp8(mb, mm)
    torch.cuda.synchronize()
    for name in outs:
        assert torch.equal(getattr(ref, name), getattr(mb, name)), name


# ---------------------------------------------------------------- full size

def test_mixtral_full_size_sampled():
    """T=32768, H=4096, E=8, top-2, h=14336 in the bench's launch
    configuration.  Routing complete and bit-exact; dispatched codes of a
    token sample bit-exact; weight codes of sampled columns bit-exact; 16
    packed rows of each of two experts against the oracle's FP8 expert FFN
    (all h columns; four 32-column blocks of out against the product of the
    GPU's own h rows and W2); y of sampled tokens
    against combine's definition on the GPU's out rows (a property that holds
    at any size)."""
    w = WORKLOADS["mixtral_bf16"]
    say(f"[mxfp8 mixtral full size] {w}")
    p = make_inputs(w, seed=0, device="cuda")
    buf, mw = run_mx(w, p)
    r = check_routing(w, buf)
    N = int(buf.offsets[-1].item())
    nmax = buf.xp_q.shape[0]
    toks = sample_tokens(w.T, 256, seed=9).numpy()
    xs = np32(p["x"][torch.as_tensor(toks, device="cuda")])
    xc, xsc = M.mx_quantize(xs, axis=1)
    ro = r["row_of"]
    xps = op_rows(buf.xp_s, nmax, w.H)
    for i, t in enumerate(toks):
        for k in range(w.K):
            if ro[t, k] >= 0:
                assert np.array_equal(u8(buf.xp_q[int(ro[t, k])]), xc[i]), (t, k)
                assert np.array_equal(xps[int(ro[t, k])], xsc[i]), (t, k)
    say("  dispatched codes of 256 tokens bit-exact")
    cols = np.array([0, 1, 5000, 14335])
    w1c = np32(p["w1"][:, :, torch.as_tensor(cols, device="cuda")])
    rc, rs = M.quantize_weights(w1c)
    gq = panel_rows(mw.w1_q, w.E, w.H, w.h, cols)
    assert np.array_equal(gq, rc.transpose(0, 2, 1))
    say("  W1 codes of sampled columns bit-exact")
    off = r["offsets"]
    blocks = np.array([0, 37, 64, 127])  # 32-column blocks of out
    ocols = (blocks[:, None] * 32 + np.arange(32)[None, :]).ravel()
    for e in (0, 5):
        if off[e + 1] <= off[e]:
            continue
        rows = np.linspace(off[e], off[e + 1] - 1, 16).astype(np.int64)
        xd = M.mx_roundtrip(np32(p["x"][torch.as_tensor(r["token_of"][rows], device="cuda")]),
                            axis=1)
        u = np.zeros((len(rows), w.h))
        for c0 in range(0, w.h, 2048):  # W1[e] in column slices (blocks run down columns)
            sl = np32(p["w1"][e, :, c0:c0 + 2048])
            u[:, c0:c0 + 2048] = xd @ M.mx_roundtrip(sl, axis=0)
        hv = O.gelu_tanh(u)
        hc, hs = M.mx_quantize(hv, axis=1)
        tmax = np.zeros_like(u)
        tsum = np.zeros_like(u)
        for c0 in range(0, w.h, 2048):
            sl = M.mx_roundtrip(np32(p["w1"][e, :, c0:c0 + 2048]), axis=0)
            tmax[:, c0:c0 + 2048], tsum[:, c0:c0 + 2048] = accum_bounds(xd, sl)
        check_h_rounding(f"h rows of expert {e} (strict)",
                         u8(buf.h_q[torch.as_tensor(rows, device="cuda")]),
                         op_rows(buf.h_s, nmax, w.h)[rows], hv, tmax, tsum, w.H)
        # out columns against the float64 product of the GPU's own h rows
        # and the dequantised W2 columns (exact step maxima)
        rt = torch.as_tensor(rows, device="cuda")
        gh_c, gh_s = u8(buf.h_q[rt]), op_rows(buf.h_s, nmax, w.h)[rows]
        check_mx_close(f"h rows of expert {e}", gh_c, gh_s, hc, hs)
        hd = M.mx_dequantize(gh_c, gh_s, axis=1)
        w2d = M.mx_roundtrip(np32(p["w2"][e][:, torch.as_tensor(ocols, device="cuda")]), axis=0)
        tmax, tsum = accum_bounds(hd, w2d)
        check_out_rounding(f"out rows of expert {e} (strict)", u8(buf.out_q[rt])[:, ocols],
                           u8(buf.out_s[rt])[:, blocks], hd @ w2d, tmax, tsum, w.h)
    # y against combine's definition on the GPU's own FP8 outputs
    y = buf.y.cpu().to(torch.float64).numpy()
    for t in toks[:64]:
        acc = np.zeros(w.H)
        for k in range(w.K):
            rr = int(ro[t, k])
            if rr >= 0:
                d = M.mx_dequantize(u8(buf.out_q[rr])[None], u8(buf.out_s[rr])[None], axis=1)[0]
                acc += float(buf.topk_w[t, k].item()) * d
        mag = np.zeros(w.H)
        for k in range(w.K):
            rr = int(ro[t, k])
            if rr >= 0:
                d = M.mx_dequantize(u8(buf.out_q[rr])[None], u8(buf.out_s[rr])[None], axis=1)[0]
                mag += abs(float(buf.topk_w[t, k].item())) * np.abs(d)
        # bf16 rounding of the sum, plus fp32 rounding of the terms
        err = np.abs(y[t] - acc) / (2.0 ** -8 * np.abs(acc) + 2.0 ** -20 * mag + 1e-30)
        assert err.max() <= 1.0, (t, err.max())
    say(f"  y of 64 tokens = bf16(sum_k w deq(out)); N = {N}")
