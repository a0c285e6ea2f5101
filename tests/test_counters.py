"""Host checks of the bench's roofline arithmetic (counters.segment_roofline_s)."""

import pytest

from mixture_experts_layer_08_amd import counters


def test_large_segment_is_flop_bound():
    H, h, b, P, BW = 4096, 14336, 2, 2.5e15, 8e12
    f, m, seg = counters.segment_roofline_s([8192], H, h, b, P, BW)
    assert f == pytest.approx(4 * 8192 * H * h / P)
    assert m == pytest.approx((2 * H * h + 2 * 8192 * (H + h)) * b / BW)
    assert seg == pytest.approx(f) and f > m


def test_small_segment_is_weight_bound_and_segments_add():
    H, h, b, P, BW = 4096, 1408, 2, 2.5e15, 8e12
    f1, m1, s1 = counters.segment_roofline_s([140], H, h, b, P, BW)
    assert s1 == pytest.approx(m1) and m1 > f1  # 140 rows cannot amortise the weights
    f2, m2, s2 = counters.segment_roofline_s([140, 0, 20000], H, h, b, P, BW)
    fb, mb, sb = counters.segment_roofline_s([20000], H, h, b, P, BW)
    assert s2 == pytest.approx(s1 + sb)  # empty segments cost nothing
    assert f2 == pytest.approx(f1 + fb) and m2 == pytest.approx(m1 + mb)


def test_shared_expert_is_one_more_segment():
    H, h, hs, b, P, BW = 256, 64, 96, 4, 1e14, 1e12
    base = counters.segment_roofline_s([10, 20], H, h, b, P, BW)
    with_sh = counters.segment_roofline_s([10, 20], H, h, b, P, BW, shared_rows=30, hs=hs)
    sh = counters.segment_roofline_s([30], H, hs, b, P, BW)
    assert all(x == pytest.approx(y + z) for x, y, z in zip(with_sh, base, sh))


def test_profile_hash_ignores_comments_not_code():
    """A recorded profile stays valid across comment edits of the GEMM
    sources and is dropped for any change to their code."""
    from mixture_experts_layer_08_amd.profiling import code_of

    base = "int f(int a) {\n  // step\n  return a + 1; /* one */\n}\n"
    assert code_of(base) == code_of("int f(int a) {\n  return a + 1;   // other words\n}\n")
    assert code_of(base) == code_of("/* header\n   lines */ int  f(int a) {\n return a + 1; }")
    assert code_of(base) != code_of(base.replace("a + 1", "a + 2"))
    assert code_of('asm("s_nop 0\\n\\ts_nop 0");') == 'asm("s_nop 0\\n\\ts_nop 0");'
