"""moe_mfma_ceiling, the MFMA-only measurement kernel behind bench.py's
mfma_ceiling figure: its arithmetic checked on a few workgroups against
float64 numpy, so that the rate it reports is the rate of the stated work.

Each lane of each wave must hold rows 4 (l / 16) + r, column l % 16 of
sum_t sum_{i,j} B_j(t) A_i(t)^T, with fragment f's lane l supplying row
l % 16, k = 8 (l / 16) .. +7 of a 16 x 32 matrix (the layout include/moe.h
states; mode 3, the 32x32x16 shape, has its own test below); round t's operands are the given ones (modes 0 and 2) or, in mode 1,
those with every sign and mantissa bit flipped in odd rounds, re-derived here
from the bf16 bit layout.
"""

import numpy as np
import pytest
import torch

from mixture_experts_layer_08_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def fragments_as_matrices(ops: np.ndarray) -> np.ndarray:
    """[16][64][8] lane data -> [16][16 rows][32 k] matrices."""
    m = np.zeros((16, 16, 32))
    for l in range(64):
        m[:, l % 16, 8 * (l // 16):8 * (l // 16) + 8] = ops[:, l, :]
    return m


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("workgroups,iters", [(1, 1), (3, 7), (5, 64)])
def test_mfma_ceiling_arithmetic(workgroups, iters, mode):
    g = torch.Generator(device="cuda").manual_seed(workgroups * 100 + iters)
    ops = torch.randn((16, 64, 8), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.full((workgroups * 256 * 4,), float("nan"), device="cuda")
    print(f"[mfma ceiling] workgroups={workgroups} iters={iters} mode={mode}", flush=True)
    B.moe_mfma_ceiling(ops, out, workgroups, iters, mode=mode)
    torch.cuda.synchronize()
    bits = ops.view(torch.int16).cpu().numpy().view(np.uint16)  # [16][64][8]
    total = np.zeros((16, 16))
    bound = np.zeros((16, 16))
    for t in range(iters):
        # mode 1, odd rounds: sign (bit 15) and mantissa (bits 0-6) flipped
        m = np.uint16(0x807F if mode == 1 and t % 2 else 0)
        mats = fragments_as_matrices(bf16_bits_to_f64(bits ^ m))
        total += mats[8:].sum(0) @ mats[:8].sum(0).T  # sum_j B_j times (sum_i A_i)^T
        bound += np.abs(mats[8:]).sum(0) @ np.abs(mats[:8]).sum(0).T
    got = out.cpu().numpy().reshape(workgroups, 4, 64, 4)
    lanes = np.arange(64)
    want = np.stack([total[4 * (lanes // 16) + r, lanes % 16] for r in range(4)], axis=1)
    err = np.abs(got - want[None, None]).max() / bound.max()
    print(f"  max err / max sum of |terms| {err:.2e}", flush=True)
    assert err <= 1e-5


def fragments_as_matrices32(ops: np.ndarray) -> np.ndarray:
    """[16][64][8] lane data -> [16][32 rows][16 k] matrices (32x32x16 layout)."""
    m = np.zeros((16, 32, 16))
    for l in range(64):
        m[:, l % 32, 8 * (l // 32):8 * (l // 32) + 8] = ops[:, l, :]
    return m


@pytest.mark.parametrize("workgroups,iters", [(1, 1), (3, 5)])
def test_mfma_ceiling_32x32_arithmetic(workgroups, iters):
    """Mode 3: 4 x 4 tiles of v_mfma_f32_32x32x16_bf16 on fragments 0-3 (A)
    and 8-11 (B), 2 * iters passes; lane l holds rows 8 (r / 4) + 4 (l / 32)
    + r % 4, column l % 32 of the result."""
    g = torch.Generator(device="cuda").manual_seed(workgroups * 10 + iters)
    ops = torch.randn((16, 64, 8), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.full((workgroups * 256 * 16,), float("nan"), device="cuda")
    print(f"[mfma ceiling 32x32] workgroups={workgroups} iters={iters}", flush=True)
    B.moe_mfma_ceiling(ops, out, workgroups, iters, mode=3)
    torch.cuda.synchronize()
    bits = ops.view(torch.int16).cpu().numpy().view(np.uint16)
    mats = fragments_as_matrices32(bf16_bits_to_f64(bits))
    total = 2 * iters * (mats[8:12].sum(0) @ mats[0:4].sum(0).T)  # sum_j B_j (sum_i A_i)^T
    bound = 2 * iters * (np.abs(mats[8:12]).sum(0) @ np.abs(mats[0:4]).sum(0).T)
    got = out.cpu().numpy().reshape(workgroups, 4, 64, 16)
    lanes = np.arange(64)
    want = np.stack([total[8 * (r // 4) + 4 * (lanes // 32) + r % 4, lanes % 32]
                     for r in range(16)], axis=1)
    err = np.abs(got - want[None, None]).max() / bound.max()
    print(f"  max err / max sum of |terms| {err:.2e}", flush=True)
    assert err <= 1e-5


def test_mfma_ceiling_rejects_bad_arguments():
    ops = torch.zeros((16, 64, 8), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros(1024, device="cuda")
    for wg, it in [(0, 1), (1, 0), (1 << 17, 1)]:
        with pytest.raises(B.MoeError):
            B.moe_mfma_ceiling(ops, out, wg, it)
