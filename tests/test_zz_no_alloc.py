"""moe_forward_noalloc: the whole layer on the library's static per-GPU
scratch, for callers that cannot allocate.  Its output must be the same
bits as moe_forward's (same kernels, same launch sequence, only the
workspace differs) and within the bar against the oracle, on two calls in a
row, the second with fewer tokens (the scratch then holds the first call's
intermediates)."""
import ctypes

import numpy as np
import pytest

import moe_inputs as mi
import oracle as o
from helpers import assert_close, device_inputs, shape_of, to_host_f32

torch = pytest.importorskip("torch")


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """A shape whose workspace exceeds the static scratch is rejected on the
    host before anything is enqueued (no GPU needed)."""
    import mixture_experts_ffn_moe_amd as m
    lib = m._lib.lib
    P = ctypes.c_void_p(4096)
    big = m.make_shape(4096, 4096, 64, 8, 1536, 1, "bf16")
    assert m.moe_workspace_size(big) > m.NOALLOC_SCRATCH_BYTES
    assert lib.moe_forward_noalloc(ctypes.byref(big), P, P, None, P, P, P, None) == m.MOE_ERR_WORKSPACE
    # the decode layer fits with room to spare
    dec = m.make_shape(8, 4096, 64, 8, 768, 1, "bf16")
    assert m.moe_workspace_size(dec) < m.NOALLOC_SCRATCH_BYTES // 8
    # invalid arguments are reported before the size check, an empty batch is a no-op
    bad = m.make_shape(8, 4096, 65, 8, 768, 1, "bf16")
    assert lib.moe_forward_noalloc(ctypes.byref(bad), P, P, None, P, P, P, None) == m.MOE_ERR_UNSUPPORTED
    zero = m.make_shape(0, 4096, 64, 8, 768, 1, "bf16")
    assert lib.moe_forward_noalloc(ctypes.byref(zero), P, P, None, P, P, P, None) == m.MOE_OK
    assert lib.moe_forward_noalloc(ctypes.byref(dec), None, P, None, P, P, P, None) == m.MOE_ERR_INVALID_ARG


CASES = [
    # small-token (decode) path: 16 tokens, then 5
    dict(name="decode_path", T=(16, 5), H=2048, E=32, k=4, Im=256, micro=1, dtype=mi.BF16, seed=71,
         sigma_g=0.02, sigma_w=0.02),
    # token path, bf16, two micros: 200 tokens, then 60
    dict(name="token_path_bf16", T=(200, 60), H=512, E=16, k=4, Im=256, micro=2, dtype=mi.BF16, seed=72,
         sigma_g=0.02, sigma_w=0.02),
    # token path, fp32: 64 tokens, then 20
    dict(name="token_path_f32", T=(64, 20), H=256, E=8, k=2, Im=128, micro=1, dtype=mi.F32, seed=73,
         sigma_g=0.1, sigma_w=0.02),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_noalloc_matches_forward(case):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dataclasses
    import mixture_experts_ffn_moe_amd as m
    c = dict(case)
    name, Ts = c.pop("name"), c.pop("T")
    sp_full = mi.custom_spec(T=Ts[0], name=name, **c)
    inp_full = mi.make_layer(sp_full)
    for T in Ts:
        sp = dataclasses.replace(sp_full, T=T)
        inp = mi.LayerInputs(sp, np.ascontiguousarray(inp_full.x[:T]), inp_full.wg, inp_full.bias,
                             inp_full.w1, inp_full.w2)
        print(f"[no-alloc] {name}: T={T} H={sp.H} E={sp.E} k={sp.k} Im={sp.Im} mu={sp.micro}", flush=True)
        d = device_inputs(inp)
        s = shape_of(sp)
        out = torch.full((T, sp.H), float("nan"), dtype=d["x"].dtype, device="cuda")
        m.moe_forward_noalloc(s, d["x"], d["wg"], d["bias"], d["w1"], d["w2"], out)
        ref = m.MoELayerBuffers(s).forward(d["x"], d["wg"], d["bias"], d["w1"], d["w2"])
        torch.cuda.synchronize()
        view = (lambda t: t.view(torch.int16)) if sp.dtype == mi.BF16 else (lambda t: t.view(torch.int32))
        assert torch.equal(view(out), view(ref)), f"{name} T={T}: differs from moe_forward"
        ma, rl = assert_close(to_host_f32(out), o.forward(inp)["out"], sp.dtype, f"{name} T={T}")
        print(f"[no-alloc] {name} T={T}: same bits as moe_forward; vs oracle max-abs {ma:.2e} rel-L2 {rl:.2e}",
              flush=True)
