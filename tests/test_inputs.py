"""The seeded generator: reproducible, laid out as the pages' MoE pack, and
producing the workload's routing regimes."""
import numpy as np
import pytest

import moe_inputs as mi
import oracle as o


def test_bf16_rounding_ties_to_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e-39], np.float32)
    bits = mi.f32_to_bf16_bits(vals)
    back = mi.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even (1.0)
    assert back[1] == 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to even (1 + 2^-6)
    assert back[2] == 1.0 + 2 ** -6
    assert back[3] == 1.0
    assert back[4] == -2.5
    assert bits[0] == 0x3F80


def test_seeds_reproduce_and_differ():
    sp = mi.custom_spec(T=8, H=16, E=4, k=2, Im=4, micro=2, dtype=mi.BF16, seed=3)
    a, b = mi.make_layer(sp), mi.make_layer(sp)
    for f in ("x", "wg", "w1", "w2"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = mi.make_layer(mi.custom_spec(T=8, H=16, E=4, k=2, Im=4, micro=2, dtype=mi.BF16, seed=4))
    assert not np.array_equal(a.x, c.x)


def test_two_micro_pack_is_relayout_of_expert_major():
    """The 2-micro layer holds exactly the 1-micro layer's weights, stored
    micro-major with the [gate_m0, up_m0] / [gate_m1, up_m1] order."""
    s1, s2 = mi.spec("denoise_1micro"), mi.spec("denoise_2micro")
    for e in (0, 37):
        a1, b1 = mi.expert_pack(s1, e)
        a2, b2 = mi.expert_pack(s2, e)
        w13, down = a1[0], b1[0]
        I, Im = 1536, 768
        for m in range(2):
            assert np.array_equal(a2[m][:Im], w13[m * Im:(m + 1) * Im])
            assert np.array_equal(a2[m][Im:], w13[I + m * Im:I + (m + 1) * Im])
            assert np.array_equal(b2[m], down[:, m * Im:(m + 1) * Im])


def test_layer_table():
    assert [s.name for s in mi.LAYERS] == ["tiny_fp32", "denoise_1micro", "denoise_2micro",
                                           "decode", "skewed_cfg"]
    s = mi.spec("denoise_1micro")
    assert (s.T, s.H, s.E, s.k, s.I) == (4096, 4096, 64, 8, 1536)
    assert mi.spec("denoise_2micro").I == 1536 and mi.spec("denoise_2micro").micro == 2
    assert mi.spec("decode").T == 8 and mi.spec("decode").I == 768
    assert mi.spec("skewed_cfg").T == 8192


def test_skewed_layer_leaves_experts_empty():
    """Route the skewed layer with the oracle: the bias must produce a heavy
    head and some empty experts."""
    sp = mi.spec("skewed_cfg")
    x32 = o.widen(mi.make_x(sp), sp.dtype)
    wg, bias = mi.make_router(sp)
    ids = o.select_topk(o.router_logits(x32, wg, bias), sp.k)
    counts = o.expert_counts(ids, sp.E)
    assert counts.sum() == sp.T * sp.k
    assert (counts == 0).sum() >= 1
    assert counts.max() > 4 * counts.mean()


def test_near_uniform_denoise_routing():
    sp = mi.spec("denoise_1micro")
    x32 = o.widen(mi.make_x(sp), sp.dtype)
    wg, bias = mi.make_router(sp)
    assert bias is None
    ids = o.select_topk(o.router_logits(x32, wg, bias), sp.k)
    counts = o.expert_counts(ids, sp.E)
    assert counts.min() > 350 and counts.max() < 700
