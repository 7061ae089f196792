"""Shared test helpers: move seeded inputs to the device, read results back,
and the parity bars."""
from __future__ import annotations

import numpy as np

import moe_inputs as mi

# Output tolerances of the workload: bf16 layers max-abs 2e-2 and relative
# L2 1e-2; the fp32 layer 1e-5 for both.
TOL = {mi.BF16: (2e-2, 1e-2), mi.F32: (1e-5, 1e-5)}


def to_dev(a: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == mi.BF16 and a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host_f32(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return mi.bf16_bits_to_f32(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.detach().cpu().numpy()


def device_inputs(inp: mi.LayerInputs, device="cuda") -> dict:
    import torch
    sp = inp.spec
    d = {
        "x": to_dev(inp.x, sp.dtype, device),
        "wg": torch.from_numpy(inp.wg).to(device),
        "bias": None if inp.bias is None else torch.from_numpy(inp.bias).to(device),
        "w1": to_dev(inp.w1, sp.dtype, device),
        "w2": to_dev(inp.w2, sp.dtype, device),
    }
    return d


def shape_of(sp: mi.LayerSpec):
    from mixture_experts_ffn_moe_amd import make_shape
    return make_shape(sp.T, sp.H, sp.E, sp.k, sp.Im, sp.micro, sp.dtype, sp.renormalize)


def y_buffer(sp, rows, device="cuda"):
    """A y buffer (raw bytes) of `rows` rows for layer sp."""
    import torch
    from mixture_experts_ffn_moe_amd import y_nbytes
    return torch.empty(y_nbytes(shape_of(sp), rows), dtype=torch.uint8, device=device)


def decode_y(sp, buf, rows) -> np.ndarray:
    """y values [rows, H] as float64 from a y buffer: fp32 for the fp32 layer;
    for the bf16 layers block-scaled half, fp16 values [rows, H] then int8
    exponents [rows, ceil(H / 256)], y = value * 2^exponent (exact in float64)."""
    raw = buf.cpu().numpy().view(np.uint8)
    H = sp.H
    if sp.dtype == mi.F32:
        return raw.view(np.float32).reshape(rows, H).astype(np.float64)
    nb = -(-H // 256)
    vals = raw[:rows * H * 2].view(np.float16).reshape(rows, H).astype(np.float64)
    exps = raw[rows * H * 2:rows * H * 2 + rows * nb].view(np.int8).reshape(rows, nb)
    return vals * np.exp2(np.repeat(exps.astype(np.float64), 256, axis=1)[:, :H])


def check_y_blocks(sp, buf, rows):
    """Block-scaled half y: every block's largest |value| lies in [2^14, 2^15]
    (scaled by the block's exponent into [2^14, 2^15), then rounded to fp16,
    which can carry the largest up to 2^15), or the block is all zero with
    exponent 0."""
    raw = buf.cpu().numpy().view(np.uint8)
    H = sp.H
    nb = -(-H // 256)
    vals = raw[:rows * H * 2].view(np.float16).reshape(rows, H).astype(np.float64)
    exps = raw[rows * H * 2:rows * H * 2 + rows * nb].view(np.int8).reshape(rows, nb)
    m = np.stack([np.abs(vals[:, 256 * b:256 * (b + 1)]).max(axis=1) for b in range(nb)], axis=1)
    zero = m == 0
    assert (exps[zero] == 0).all()
    assert ((m[~zero] >= 2.0 ** 14) & (m[~zero] <= 2.0 ** 15)).all()


def out_dtype(sp):
    import torch
    return torch.bfloat16 if sp.dtype == mi.BF16 else torch.float32


def errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(d) / den) if den > 0 else float(np.linalg.norm(d))
    return max_abs, rel


def assert_close(got, ref, dtype: str, what: str = "out"):
    ma, rl = errors(got, ref)
    tol_abs, tol_rel = TOL[dtype]
    assert ma <= tol_abs and rl <= tol_rel, f"{what}: max-abs {ma:.3e} (<= {tol_abs}), rel-L2 {rl:.3e} (<= {tol_rel})"
    return ma, rl


def assert_close_scaled(got, ref, dtype: str, what: str):
    """Intermediates (h, y) of magnitude up to ~10: per-element bound scaled
    by the reference magnitude, plus the relative L2 bar."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    tol_abs, tol_rel = TOL[dtype]
    d = np.abs(got - ref)
    bound = tol_abs + tol_rel * np.abs(ref)
    bad = d > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements off, worst {float((d - bound).max()):.3e}"
    _, rl = errors(got, ref)
    assert rl <= tol_rel, f"{what}: rel-L2 {rl:.3e}"


def random_shapes(n=24, seed=2024):
    """Seeded layer shapes spread over the supported envelope (H % 64,
    Im % 32, 1-3 micros, 1-64 experts, k <= 8, fp32 and bf16, some with a
    shared expert of width Is % 32, skewed routing or no renormalisation),
    plus small-token bf16 shapes that take the decode path.  Sizes stay
    small enough for the oracle to run each in about a second."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = mi.F32 if rng.random() < 0.25 else mi.BF16
        E = int(rng.integers(1, 65))
        c = dict(T=int(rng.integers(1, 400)), H=64 * int(rng.integers(1, 9)), E=E,
                 k=int(rng.integers(1, min(E, 8) + 1)), Im=32 * int(rng.integers(1, 9)),
                 micro=int(rng.integers(1, 4)), dtype=dt, seed=300 + i, sigma_g=0.02, sigma_w=0.02,
                 renormalize=bool(rng.random() < 0.85))
        if rng.random() < 0.25:
            c["zipf"] = {"s": 1.2, "scale": 6.0, "seed": 300 + i}
        if rng.random() < 0.3:
            c["Is"] = 32 * int(rng.integers(1, 9))
        c["name"] = (f"r{i:02d}_T{c['T']}_H{c['H']}_E{E}_k{c['k']}_I{c['Im']}x{c['micro']}_{dt}"
                     + (f"_Is{c['Is']}" if "Is" in c else ""))
        out.append(c)
    # degenerate bf16 shapes: one expert, one token, every expert for every token
    for j, c in enumerate([dict(T=77, H=320, E=1, k=1, Im=96, micro=2),
                           dict(T=1, H=64, E=2, k=2, Im=32, micro=1),
                           dict(T=130, H=256, E=8, k=8, Im=160, micro=1, Is=32)]):
        c.update(dtype=mi.BF16, seed=380 + j, sigma_g=0.02, sigma_w=0.02, renormalize=True)
        c["name"] = (f"e{j}_T{c['T']}_H{c['H']}_E{c['E']}_k{c['k']}_I{c['Im']}x{c['micro']}_bf16"
                     + (f"_Is{c['Is']}" if "Is" in c else ""))
        out.append(c)
    for i in range(4):  # the decode path: T <= 16, bf16, H % 2048, Im % 256
        E = int(rng.integers(8, 65))
        c = dict(T=int(rng.integers(1, 17)), H=2048, E=E, k=int(rng.integers(1, min(E, 8) + 1)),
                 Im=256 * int(rng.integers(1, 3)), micro=int(rng.integers(1, 3)), dtype=mi.BF16,
                 seed=400 + i, sigma_g=0.02, sigma_w=0.02, renormalize=True)
        if i % 2:
            c["Is"] = 256 * int(rng.integers(1, 3))
        c["name"] = (f"d{i}_T{c['T']}_E{E}_k{c['k']}_I{c['Im']}x{c['micro']}"
                     + (f"_Is{c['Is']}" if "Is" in c else ""))
        out.append(c)
    return out
