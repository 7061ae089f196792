"""The C ABI without a GPU: the library loads, exports every declared entry
point, and its host-side validation rejects bad calls before any launch.

Every call below fails validation (or has T == 0) on the host, so no kernel is
ever launched with the placeholder pointers used here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]


@pytest.fixture(scope="module")
def m():
    import mixture_experts_ffn_moe_amd as m
    return m


def declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_0-9]+)\s*\(", src, flags=re.M))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("moe_route", "moe_permute", "moe_grouped_gemm_w13_swiglu", "moe_grouped_gemm_down",
              "moe_finalize", "moe_forward", "moe_workspace_size", "moe_status_string",
              "moe_get_workspace_layout"):
        assert n in names


def test_library_exports_every_declared_symbol(m):
    lib = ctypes.CDLL(m.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(m.EXPORTED)


def test_probe_validation(m):
    lib = m._lib.lib
    P = ctypes.c_void_p(4096)
    assert lib.moe_probe_mfma_bf16(0, P, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_probe_mfma_bf16(10, P, None) == m.MOE_ERR_INVALID_ARG  # not a multiple of 4
    assert lib.moe_probe_mfma_bf16(12, None, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_probe_read(P, 0, P, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_probe_read(ctypes.c_void_p(4096 + 4), 1024, P, None) == m.MOE_ERR_UNSUPPORTED
    assert lib.moe_probe_read(P, 1000, P, None) == m.MOE_ERR_UNSUPPORTED
    assert lib.moe_probe_mfma_flops(3) == 256 * 8 * 8 * 32768 * 3


def test_status_strings(m):
    for c in range(5):
        assert m.status_string(c).startswith("MOE_")
    assert "unknown" in m.status_string(99)


def test_workspace_size_and_layout(m):
    s = m.make_shape(4096, 4096, 64, 8, 1536, 1, "bf16")
    L = m.moe_get_workspace_layout(s)
    R = 4096 * 8
    assert L["total"] == m.moe_workspace_size(s)
    assert L["h"] - L["inv"] >= R * 4 and L["y"] - L["h"] >= R * 1536 * 2
    assert L["total"] - L["y"] >= R * 4096 * 2 + R * 16  # y: fp16 values + one exponent per 256 columns
    for v in L.values():
        assert v % 256 == 0
    # micro split does not change the size
    assert m.moe_workspace_size(m.make_shape(4096, 4096, 64, 8, 768, 2, "bf16")) == L["total"]
    # fp32 intermediates are twice as wide
    assert m.moe_workspace_size(m.make_shape(64, 256, 8, 2, 128, 1, "f32")) > \
        m.moe_workspace_size(m.make_shape(64, 256, 8, 2, 128, 1, "bf16"))


@pytest.mark.parametrize("args,code", [
    ((64, 256, 65, 2, 128, 1), "MOE_ERR_UNSUPPORTED"),    # E > 64
    ((64, 256, 8, 9, 128, 1), "MOE_ERR_INVALID_ARG"),     # k > E
    ((64, 256, 8, 0, 128, 1), "MOE_ERR_INVALID_ARG"),     # k < 1
    ((-1, 256, 8, 2, 128, 1), "MOE_ERR_INVALID_ARG"),     # T < 0
    ((64, 256, 8, 2, 128, 0), "MOE_ERR_INVALID_ARG"),     # no micro-shard
    ((64, 200, 8, 2, 128, 1), "MOE_ERR_UNSUPPORTED"),     # H not a multiple of 64
    ((64, 288, 8, 2, 128, 1), "MOE_ERR_UNSUPPORTED"),     # H a multiple of 32, not of 64
    ((64, 256, 8, 2, 48, 1), "MOE_ERR_UNSUPPORTED"),      # Im not a multiple of 32
    ((64, 256, 8, 2, 80, 2), "MOE_ERR_UNSUPPORTED"),      # Im a multiple of 16, not of 32
    ((1 << 28, 4096, 64, 8, 128, 1), "MOE_ERR_UNSUPPORTED"),  # T*k*H beyond 2^31
])
def test_shape_validation(m, args, code):
    s = m.make_shape(*args, dtype="bf16")
    assert m.moe_workspace_size(s) == 0
    want = getattr(m, code)
    lib = m._lib.lib
    P = ctypes.c_void_p(4096)  # placeholder, never dereferenced: validation fails first
    assert lib.moe_forward(ctypes.byref(s), P, P, None, P, P, P, P, ctypes.c_size_t(1 << 40), None) == want
    assert lib.moe_route(ctypes.byref(s), P, P, None, P, P, P, None) == want
    assert lib.moe_finalize(ctypes.byref(s), P, P, P, P, None) == want


def test_bad_dtype_and_null_shape(m):
    s = m.MoeShape(64, 256, 8, 2, 128, 1, 7)
    lib = m._lib.lib
    P = ctypes.c_void_p(4096)
    assert lib.moe_grouped_gemm_down(ctypes.byref(s), P, P, P, P, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_forward(None, P, P, None, P, P, P, P, ctypes.c_size_t(1 << 40), None) == m.MOE_ERR_INVALID_ARG


def test_pointer_and_workspace_validation(m):
    lib = m._lib.lib
    s = m.make_shape(64, 256, 8, 2, 128, 1, "bf16")
    need = m.moe_workspace_size(s)
    P = ctypes.c_void_p(4096)
    mis = ctypes.c_void_p(4096 + 8)
    ws = ctypes.c_void_p(1 << 20)
    # null input
    assert lib.moe_forward(ctypes.byref(s), None, P, None, P, P, P, ws, need, None) == m.MOE_ERR_INVALID_ARG
    # misaligned weight
    assert lib.moe_forward(ctypes.byref(s), P, P, None, mis, P, P, ws, need, None) == m.MOE_ERR_UNSUPPORTED
    # workspace too small / missing / misaligned
    assert lib.moe_forward(ctypes.byref(s), P, P, None, P, P, P, ws, need - 1, None) == m.MOE_ERR_WORKSPACE
    assert lib.moe_forward(ctypes.byref(s), P, P, None, P, P, P, None, need, None) == m.MOE_ERR_WORKSPACE
    assert lib.moe_forward(ctypes.byref(s), P, P, None, P, P, P, ctypes.c_void_p((1 << 20) + 16), need, None) \
        == m.MOE_ERR_UNSUPPORTED
    # permute: x and permuted_x must come together
    assert lib.moe_permute(ctypes.byref(s), P, P, P, P, P, P, None, None) == m.MOE_ERR_INVALID_ARG


def test_expert_block_over_4gib_is_unsupported(m):
    # 4 * Im * H bytes = 4 * 32768 * 32768 = 2^32: one expert's w1 block does
    # not fit the GEMMs' 32-bit offsets
    s = m.make_shape(1, 32768, 1, 1, 32768, 1, "bf16")
    assert m._lib.lib.moe_workspace_size(ctypes.byref(s)) == 0
    s2 = m.make_shape(1, 32768, 1, 1, 16384, 1, "bf16")
    assert m._lib.lib.moe_workspace_size(ctypes.byref(s2)) > 0


def test_zero_tokens_is_a_no_op(m):
    lib = m._lib.lib
    s = m.make_shape(0, 256, 8, 2, 128, 1, "bf16")
    P = ctypes.c_void_p(4096)
    assert lib.moe_forward(ctypes.byref(s), P, P, None, P, P, P, P, ctypes.c_size_t(0), None) == m.MOE_OK
    assert lib.moe_route(ctypes.byref(s), P, P, None, P, P, P, None) == m.MOE_OK
    assert lib.moe_grouped_gemm_w13_swiglu(ctypes.byref(s), P, P, P, P, P, None) == m.MOE_OK


def test_renormalize_flag(m):
    """renormalize is 0 or 1; anything else is an invalid argument."""
    lib = m._lib.lib
    P = ctypes.c_void_p(4096)
    for v, want in ((0, m.MOE_OK), (1, m.MOE_OK), (2, m.MOE_ERR_INVALID_ARG), (-1, m.MOE_ERR_INVALID_ARG)):
        s = m.make_shape(64, 256, 8, 2, 128, 1, "bf16")
        s.renormalize = v
        assert (lib.moe_workspace_size(ctypes.byref(s)) > 0) == (want == m.MOE_OK)
        if want != m.MOE_OK:
            assert lib.moe_route(ctypes.byref(s), P, P, None, P, P, P, None) == want
    assert m.make_shape(64, 256, 8, 2, 128, 1, "bf16").renormalize == 1
    assert m.make_shape(64, 256, 8, 2, 128, 1, "bf16", renormalize=False).renormalize == 0


def test_shape_struct_matches_header(m):
    """The ctypes mirror of moe_shape has the header's fields, in order."""
    import re
    hdr = open(os.path.join(ROOT, "include", "moe_mi355x.h")).read()
    body = re.search(r"typedef struct \{(.*?)\} moe_shape;", hdr, flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"int32_t\s+(\w+);", body)
    assert fields == [f[0] for f in m.MoeShape._fields_]


def test_binding_raises_on_error(m):
    s = m.make_shape(64, 256, 65, 2, 128, 1, "bf16")
    with pytest.raises(m.MoeError) as ei:
        m._lib._check(m._lib.lib.moe_route(ctypes.byref(s), None, None, None, None, None, None, None), "moe_route")
    assert ei.value.code == m.MOE_ERR_UNSUPPORTED


def test_binding_checks_tensors_before_the_call(m):
    """The C entry points take raw pointers and cannot check sizes, so the
    binding checks each tensor's device, dtype and element count against the
    shape before calling (a wrong-size tensor would otherwise be written out
    of bounds on the GPU)."""
    torch = pytest.importorskip("torch")
    s = m.make_shape(4, 256, 8, 2, 128, 1, "bf16")
    f = m._lib._arg
    assert f("bias", None, torch.float32, 8, nullable=True) is None
    with pytest.raises(ValueError, match="required"):
        f("x", None, torch.bfloat16, 4 * 256)
    with pytest.raises(TypeError):
        f("x", [0.0] * 1024, torch.bfloat16, 4 * 256)
    with pytest.raises(ValueError, match="GPU tensor"):
        f("x", torch.zeros(4, 256, dtype=torch.bfloat16), torch.bfloat16, 4 * 256)
    # every wrapper checks before it calls the library: host tensors are refused
    x = torch.zeros(4, 256, dtype=torch.bfloat16)
    wg = torch.zeros(8, 256)
    with pytest.raises(ValueError, match="GPU tensor"):
        m.moe_route(s, x, wg, None, torch.zeros(4, 8), torch.zeros(4, 2, dtype=torch.int32), torch.zeros(4, 2))
    with pytest.raises(ValueError, match="workspace"):
        m.moe_forward(s, x, wg, None, x, x, x, None)


# ---------------------------------------------------------------- shared expert (moe_shared.h)


@pytest.mark.parametrize("H,Im,mu", [(320, 96, 1), (64, 32, 3), (448, 160, 2), (4096, 1536, 1)])
def test_envelope_accepts_multiples_of_64_and_32(m, H, Im, mu):
    """H % 64 == 0 and Im % 32 == 0 are inside the envelope (the bf16 kernels
    then take the narrow tile shapes or a partial last output tile)."""
    for dt in ("bf16", "f32"):
        s = m.make_shape(16, H, 8, 2, Im, mu, dt)
        assert m.moe_workspace_size(s) > 0


@pytest.mark.parametrize("H", [64, 192, 256, 320, 4096])
def test_y_layout_size(m, H):
    """Block-scaled half y: fp16 values then one int8 exponent per started
    block of 256 columns (MOE_Y_BYTES); fp32 y in the fp32 layer."""
    rows = 7
    nb = (H + 255) // 256
    assert m.y_nbytes(m.make_shape(4, H, 8, 2, 64, 1, "bf16"), rows) == rows * H * 2 + rows * nb
    assert m.y_nbytes(m.make_shape(4, H, 8, 2, 64, 1, "f32"), rows) == rows * H * 4
    L = m.moe_get_workspace_layout(m.make_shape(4, H, 8, 2, 64, 1, "bf16"))
    assert L["total"] - L["y"] >= 4 * 2 * (H * 2 + nb)


def test_shared_workspace_layout(m):
    s = m.make_shape(4096, 4096, 64, 8, 1536, 1, "bf16")
    base = m.moe_workspace_size(s)
    Ls = m.moe_get_shared_workspace_layout(s, 1536)
    assert Ls["total"] == m.moe_shared_workspace_size(s, 1536)
    # the routed workspace comes first, unchanged; then hs [T, Is] and ys [T, H]
    assert Ls["hs"] == base
    assert Ls["ys"] - Ls["hs"] >= 4096 * 1536 * 2
    assert Ls["total"] - Ls["ys"] >= 4096 * 4096 * 2 + 4096 * 16  # ys: block-scaled half
    assert all(v % 256 == 0 for v in Ls.values())


@pytest.mark.parametrize("Is,code", [
    (0, "MOE_ERR_INVALID_ARG"), (-128, "MOE_ERR_INVALID_ARG"),
    (48, "MOE_ERR_UNSUPPORTED"), (1 << 20, "MOE_ERR_UNSUPPORTED"),
])
def test_shared_width_validation(m, Is, code):
    s = m.make_shape(64, 4096, 8, 2, 128, 1, "bf16")
    want = getattr(m, code)
    assert m.moe_shared_workspace_size(s, Is) == 0
    lib = m._lib.lib
    P = ctypes.c_void_p(4096)
    assert lib.moe_shared_ffn(ctypes.byref(s), Is, P, P, P, P, P, None) == want
    assert lib.moe_forward_shared(ctypes.byref(s), Is, P, P, None, P, P, P, P, P, P,
                                  ctypes.c_size_t(1 << 40), None) == want


def test_shared_pointer_and_workspace_validation(m):
    lib = m._lib.lib
    s = m.make_shape(64, 256, 8, 2, 128, 1, "bf16")
    Is = 128
    need = m.moe_shared_workspace_size(s, Is)
    assert need > m.moe_workspace_size(s)
    P = ctypes.c_void_p(4096)
    ws = ctypes.c_void_p(1 << 20)
    call = lambda w1s, w2s, ws_, n: lib.moe_forward_shared(  # noqa: E731
        ctypes.byref(s), Is, P, P, None, P, P, w1s, w2s, P, ws_, ctypes.c_size_t(n), None)
    assert call(None, P, ws, need) == m.MOE_ERR_INVALID_ARG
    assert call(P, ctypes.c_void_p(4096 + 4), ws, need) == m.MOE_ERR_UNSUPPORTED
    # the routed layer's workspace is not enough
    assert call(P, P, ws, m.moe_workspace_size(s)) == m.MOE_ERR_WORKSPACE
    assert call(P, P, None, need) == m.MOE_ERR_WORKSPACE
    assert lib.moe_finalize_shared(ctypes.byref(s), P, P, P, None, P, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_shared_ffn(ctypes.byref(s), Is, P, P, P, None, P, None) == m.MOE_ERR_INVALID_ARG
    # T == 0 enqueues nothing
    s0 = m.make_shape(0, 256, 8, 2, 128, 1, "bf16")
    assert lib.moe_forward_shared(ctypes.byref(s0), Is, P, P, None, P, P, P, P, P, P,
                                  ctypes.c_size_t(0), None) == m.MOE_OK
    assert lib.moe_shared_ffn(ctypes.byref(s0), Is, P, P, P, P, P, None) == m.MOE_OK
