"""Seeded synthetic inputs for the routed MoE FFN layer.

This module is shared by the CPU oracle and the GPU path, and by nothing else
of either: it holds no step of the layer's arithmetic (no routing, no
permutation, no GEMM, no activation).  It only draws numbers and lays them out.

Shapes follow the resident MoE pack of "Hunyuan Image 3.0 hybrid parallelism"
(LightX2V blog, section 5): hidden 4096, 64 experts, a TP2 shard with 1536
intermediate columns per expert, split into two micro-shards of 768 that are
stored micro-major (all experts of micro 0 first, then micro 1), and the fused
gate/up order [gate_micro0, up_micro0, gate_micro1, up_micro1] of section 4.4.

Every tensor comes from its own counter-like seed stream
``SeedSequence([seed, tag, index])`` over numpy's PCG64, so one expert's
weights can be regenerated alone (the oracle checks sampled tokens at full
size that way) and the experts of a layer can be drawn on several threads.

Floating-point values are drawn in fp32 as ``sigma * N(0, 1)``; bf16 tensors
are the round-to-nearest-even truncation of those fp32 values and are kept as
their raw 16-bit patterns in ``np.uint16`` arrays (numpy has no bf16 type).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# Stream tags: one per tensor kind.
TAG_X = 1
TAG_WG = 2
TAG_W13 = 3
TAG_DOWN = 4
TAG_BIAS = 5
TAG_SHARED = 6

F32 = "f32"
BF16 = "bf16"


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, tag: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, index])))


def normal_f32(seed: int, tag: int, index: int, shape, sigma: float) -> np.ndarray:
    a = _rng(seed, tag, index).standard_normal(shape, dtype=np.float32)
    a *= np.float32(sigma)
    return a


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


@dataclass
class LayerSpec:
    """One MoE FFN layer call: shapes, precision, distributions, seeds."""
    name: str
    T: int                 # tokens
    H: int                 # hidden size
    E: int                 # experts
    k: int                 # routes per token (top-k)
    Im: int                # intermediate columns per micro-shard
    micro: int             # micro-shards stored micro-major
    dtype: str             # F32 or BF16 for x, expert weights, h, y, out
    x_seed: int            # stream seed of the activations
    layer_seed: int        # stream seed of router and expert weights
    sigma_x: float = 1.0
    sigma_g: float = 0.02
    sigma_w: float = 0.02
    zipf_bias: Optional[dict] = None   # {"s": 1.2, "scale": 2.0, "seed": 4}
    note: str = ""
    renormalize: bool = True  # routing weights renormalised over the k selected experts

    @property
    def I(self) -> int:
        """Intermediate columns per expert over all micro-shards."""
        return self.Im * self.micro


@dataclass
class LayerInputs:
    spec: LayerSpec
    x: np.ndarray                 # [T, H]  fp32, or bf16 bits (uint16)
    wg: np.ndarray                # [E, H]  fp32
    bias: Optional[np.ndarray]    # [E]     fp32, or None
    w1: np.ndarray                # [micro, E, 2*Im, H]   rows: gate then up
    w2: np.ndarray                # [micro, E, H, Im]
    meta: dict = field(default_factory=dict)


# The five layers of the workload, by name.
LAYERS = [
    LayerSpec("tiny_fp32", T=64, H=256, E=8, k=2, Im=128, micro=1, dtype=F32,
              x_seed=0, layer_seed=0, sigma_g=0.1,
              note="tiny fp32 correctness layer"),
    LayerSpec("denoise_1micro", T=4096, H=4096, E=64, k=8, Im=1536, micro=1, dtype=BF16,
              x_seed=1, layer_seed=1,
              note="denoise image tokens, one TP2 shard stored expert-major"),
    LayerSpec("denoise_2micro", T=4096, H=4096, E=64, k=8, Im=768, micro=2, dtype=BF16,
              x_seed=1, layer_seed=1,
              note="the same layer and tokens, shard stored micro-major as 2 micros"),
    LayerSpec("decode", T=8, H=4096, E=64, k=8, Im=768, micro=1, dtype=BF16,
              x_seed=3, layer_seed=3,
              note="AR decode on one TP4 micro view"),
    LayerSpec("skewed_cfg", T=8192, H=4096, E=64, k=8, Im=768, micro=2, dtype=BF16,
              x_seed=4, layer_seed=1, zipf_bias={"s": 1.2, "scale": 2.0, "seed": 4},
              note="cond+uncond batch, Zipf-skewed expert loads"),
]


def spec(name: str) -> LayerSpec:
    for s in LAYERS:
        if s.name == name:
            return s
    raise KeyError(name)


def zipf_bias(E: int, s: float, scale: float, seed: int) -> np.ndarray:
    """Router bias that skews expert popularity toward a Zipf(s) profile.

    A random expert gets popularity rank r in 1..E, and its bias is
    ``scale * ln p(r)`` with ``p(r) = r^-s / sum_r' r'^-s``.
    """
    rank = 1 + _rng(seed, TAG_BIAS, 0).permutation(E)
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-s)
    p /= p.sum()
    return (scale * np.log(p[rank - 1])).astype(np.float32)


def expert_weights_unsharded(sp: LayerSpec, e: int):
    """Full (all micros) fp32 weights of expert e: w13 [2I, H] (gate rows
    then up rows) and down [H, I]."""
    I = sp.I
    w13 = normal_f32(sp.layer_seed, TAG_W13, e, (2 * I, sp.H), sp.sigma_w)
    down = normal_f32(sp.layer_seed, TAG_DOWN, e, (sp.H, I), sp.sigma_w)
    return w13, down


def _cast(sp: LayerSpec, a: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(a) if sp.dtype == BF16 else np.ascontiguousarray(a, np.float32)


def micro_pack_expert(sp: LayerSpec, w13: np.ndarray, down: np.ndarray):
    """Split one expert's unsharded weights into its micro slices.

    Micro m owns gate rows [m*Im, (m+1)*Im) and the matching up rows
    [I + m*Im, I + (m+1)*Im) of w13 (paired column split), and columns
    [m*Im, (m+1)*Im) of down (row split)."""
    I, Im = sp.I, sp.Im
    w1s, w2s = [], []
    for m in range(sp.micro):
        g = w13[m * Im:(m + 1) * Im]
        u = w13[I + m * Im:I + (m + 1) * Im]
        w1s.append(np.concatenate([g, u], axis=0))
        w2s.append(np.ascontiguousarray(down[:, m * Im:(m + 1) * Im]))
    return w1s, w2s


def expert_pack(sp: LayerSpec, e: int):
    """Return (w1[m] [2Im,H], w2[m] [H,Im]) for expert e in the layer's dtype."""
    w13, down = expert_weights_unsharded(sp, e)
    w1s, w2s = micro_pack_expert(sp, w13, down)
    return [_cast(sp, a) for a in w1s], [_cast(sp, a) for a in w2s]


def make_x(sp: LayerSpec) -> np.ndarray:
    return _cast(sp, normal_f32(sp.x_seed, TAG_X, 0, (sp.T, sp.H), sp.sigma_x))


def make_router(sp: LayerSpec):
    wg = normal_f32(sp.layer_seed, TAG_WG, 0, (sp.E, sp.H), sp.sigma_g)
    bias = None
    if sp.zipf_bias is not None:
        z = sp.zipf_bias
        bias = zipf_bias(sp.E, z["s"], z["scale"], z["seed"])
    return wg, bias


def shared_width(sp: LayerSpec) -> int:
    """Intermediate width of the layer's shared expert on this rank: the
    pages give no shape for it, so it takes one routed expert's width on the
    rank (the whole TP shard I, not split into micros)."""
    return sp.I


def make_shared(sp: LayerSpec, Is: Optional[int] = None):
    """The shared expert's weights, in the layer's dtype: w1s [2*Is, H] (gate
    rows, then the matching up rows) and w2s [H, Is], both sigma_w * N(0, 1)
    from the layer's stream under their own tag."""
    Is = shared_width(sp) if Is is None else Is
    w1s = normal_f32(sp.layer_seed, TAG_SHARED, 0, (2 * Is, sp.H), sp.sigma_w)
    w2s = normal_f32(sp.layer_seed, TAG_SHARED, 1, (sp.H, Is), sp.sigma_w)
    return _cast(sp, w1s), _cast(sp, w2s)


def make_layer(sp, weights: bool = True) -> LayerInputs:
    """Draw every input of one layer call.  With weights=False, w1/w2 are
    empty placeholders (for callers that fetch experts one at a time)."""
    if not isinstance(sp, LayerSpec):
        sp = spec(sp)
    x = make_x(sp)
    wg, bias = make_router(sp)
    wdt = np.uint16 if sp.dtype == BF16 else np.float32
    if weights:
        w1 = np.empty((sp.micro, sp.E, 2 * sp.Im, sp.H), dtype=wdt)
        w2 = np.empty((sp.micro, sp.E, sp.H, sp.Im), dtype=wdt)

        def fill(e):
            a, b = expert_pack(sp, e)
            for m in range(sp.micro):
                w1[m, e] = a[m]
                w2[m, e] = b[m]

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(sp.E)))
    else:
        w1 = np.empty((sp.micro, sp.E, 0, sp.H), dtype=wdt)
        w2 = np.empty((sp.micro, sp.E, sp.H, 0), dtype=wdt)
    return LayerInputs(sp, x, wg, bias, w1, w2)


def custom_spec(T, H, E, k, Im, micro=1, dtype=F32, seed=100, sigma_g=0.1, sigma_w=0.05,
                zipf=None, name="custom", renormalize=True) -> LayerSpec:
    """A layer of arbitrary (small) shape for tests."""
    return LayerSpec(name, T=T, H=H, E=E, k=k, Im=Im, micro=micro, dtype=dtype,
                     x_seed=seed, layer_seed=seed + 1, sigma_g=sigma_g, sigma_w=sigma_w,
                     zipf_bias=zipf, renormalize=renormalize)
