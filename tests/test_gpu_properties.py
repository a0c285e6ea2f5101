"""GPU parity over random small shapes (hypothesis), through the C ABI.

Each example draws T <= 200, E <= 24, K <= min(E, 8), H and h multiples of 8
up to 128, a capacity factor from {0 (no limit), 0.3, 0.5, 1, 1.25}, a dtype,
an optional shared expert and a logits mode:
  * "given": integer-valued logits with many exact ties and signed zeros,
    passed with MOE_FLAG_LOGITS_IN (the tie rule and the drop order under
    pressure);
  * "router": the GPU's own router GEMM on seeded inputs.
Routing is then bit-exact against the oracle on the GPU's logits, the GPU's
own logits (router mode) within the fp32-sum bound of the oracle's float64
router GEMM, and y within the tolerance of its dtype and its per-element
bound, as in the fixed-shape parity tests.
Derandomised: every run draws the same examples.
"""

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from mixture_experts_layer_08_amd import binding as B
from mixture_experts_layer_08_amd import layer
from mixture_experts_layer_08_amd.inputs import Workload, make_inputs
from tests.test_gpu_parity import check_logits, check_routing, check_y

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


@st.composite
def case(draw):
    E = draw(st.integers(1, 24))
    return dict(
        T=draw(st.integers(1, 200)), E=E, K=draw(st.integers(1, min(E, 8))),
        H=8 * draw(st.integers(1, 16)), h=8 * draw(st.integers(1, 16)),
        hs=8 * draw(st.integers(1, 8)) if draw(st.booleans()) else 0,
        cf=draw(st.sampled_from([0.0, 0.3, 0.5, 1.0, 1.25])),
        dtype=draw(st.sampled_from(["bf16", "f32"])),
        mode=draw(st.sampled_from(["given", "router"])),
        seed=draw(st.integers(0, 2 ** 31 - 1)))


@settings(max_examples=60, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])
@given(case())
def test_random_shapes(c):
    w = Workload("prop", T=c["T"], H=c["H"], E=c["E"], K=c["K"], h=c["h"], hs=c["hs"],
                 cf=c["cf"], dtype=c["dtype"])
    print(f"[property] {c}", flush=True)
    p = make_inputs(w, seed=c["seed"] % 100000, device="cuda")
    given_logits = c["mode"] == "given"
    buf = layer.MoeBuffers.allocate(w, logits_in=given_logits)
    if given_logits:
        r = np.random.default_rng(c["seed"])
        lg = r.integers(-2, 3, size=(w.T, w.E)).astype(np.float32)
        lg[r.random((w.T, w.E)) < 0.2] = -0.0
        buf.logits.copy_(torch.from_numpy(lg))
    layer.forward(buf, p)
    torch.cuda.synchronize()
    routing = check_routing(w, buf)
    if not given_logits:
        check_logits(w, p, buf)
    check_y(w, p, buf, routing)
