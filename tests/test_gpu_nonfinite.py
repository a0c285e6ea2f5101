"""moe_count_nonfinite: the count of NaN / inf router logits (the precondition
of routing), exact on the GPU against a host count."""

import numpy as np
import pytest
import torch

from mixture_experts_layer_08_amd import binding as B
from mixture_experts_layer_08_amd import layer
from mixture_experts_layer_08_amd.inputs import Workload, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def count(buf):
    c = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    B.moe_count_nonfinite(buf.shape, buf.logits, c)
    torch.cuda.synchronize()
    return int(c.item())


def test_count_nonfinite_logits():
    w = Workload("nonfinite", T=3001, H=128, E=24, K=4, h=64, cf=1.0)
    p = make_inputs(w, seed=41, device="cuda")
    buf = layer.MoeBuffers.allocate(w)
    layer.route(buf, p)
    torch.cuda.synchronize()
    assert count(buf) == 0
    r = np.random.default_rng(42)
    idx = r.choice(w.T * w.E, 997, replace=False)
    vals = np.array([np.nan, np.inf, -np.inf], dtype=np.float32)[r.integers(0, 3, idx.size)]
    flat = buf.logits.view(-1)
    flat[torch.from_numpy(idx).cuda()] = torch.from_numpy(vals).cuda()
    assert count(buf) == idx.size
    # NaN token rows make every logit of those tokens NaN through the router
    p["x"][[5, 77, 3000]] = float("nan")
    layer.route(buf, p)
    torch.cuda.synchronize()
    assert count(buf) == 3 * w.E
    assert int((~torch.isfinite(buf.logits)).sum().item()) == 3 * w.E
