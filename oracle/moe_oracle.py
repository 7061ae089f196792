"""CPU oracle of the routed Mixture-of-Experts FFN layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product path (the HIP library and
its Python binding) never calls it, and it shares no code with that path: the
only common module is ``moe_inputs``, which draws inputs and holds none of the
layer's arithmetic.

What is computed, and where the pages state it:

* Router: logits of a replicated router, computed in fp32 with fp32 weights
  ("HunyuanImage-3.0 on CANN NPU", section 5.2: the gate runs in fp32 with
  autocast disabled; "Hunyuan Image 3.0 hybrid parallelism", section 4.1:
  routers are replicated, not split).  The summation order is not stated; the
  reading taken here is: every product is formed in float64 (exact, because a
  bf16 or fp32 factor times an fp32 factor fits in 53 bits), summed in float64,
  the bias added in float64, and the sum rounded once to fp32.
* Gating: softmax over all experts, the k largest logits (ties to the lower
  expert index, slot j = j-th in that order), and weights renormalised over the
  selected experts (or, with renormalisation off, the softmax probabilities of
  the selected experts as they are).  The pages only say the router yields
  expert ids and routing scores of shape [num_tokens, top_k] (hybrid
  parallelism, section 6.1); k, softmax and renormalisation are the workload's
  definition.
* Route permutation: the flattened expert ids sorted by expert (stably, so
  each expert's rows keep token order), giving permuted_to_expanded; per-expert
  offsets from a bincount and a cumulative sum (hybrid parallelism, section 6.1;
  CANN NPU, section 4.2: init-routing / compute-expert-tokens).
* Gather: the input rows selected once by the permutation, shared by every
  micro-shard (hybrid parallelism, section 6.1).
* Expert FFN: down(SiLU(gate(x)) * up(x)) with gate and up fused as one w13
  projection whose first half is gate (CANN NPU, section 2.2, the swiglu fused
  operator takes chunk 0 through SiLU and multiplies by chunk 1).  Section 6.1
  of the hybrid-parallelism page prints the product the other way round; this
  oracle takes the CANN page's order, which the workload definition also uses.
* Micro-shards: micro m holds gate rows, up rows and down columns of its slice
  of the intermediate dimension (hybrid parallelism, sections 4.4 and 5); the
  micro outputs are summed before the routing scale (section 6.1, the
  finalize formula).
* Finalize: out[t] = sum_j w[t, j] * Y[row of route (t, j)], the scale applied
  once and the top-k reduction done once (hybrid parallelism, section 6.1).
* Shared expert: every token also passes through a shared expert whose output
  joins the routed experts' (CANN NPU, section 3.1, where it runs on a second
  stream).  No shape or gate is given for it; the reading taken here is an
  expert of the same SwiGLU form applied to every token and added with
  weight 1 after the routed sum.

Precision: float64 for everything after routing (the layer's own precision
is not fixed by the pages beyond the fp32 gate); routing weights are rounded
once to fp32, the type the routing scores are handed over in.

Parity status: every function is pinned by tests against brute force,
closed forms and invariants.  Absolute output values of the synthetic layers
are "parity unpinned" against the pages, which print no layer inputs or
outputs.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from moe_inputs import BF16, LayerInputs, bf16_bits_to_f32, expert_pack

# ---------------------------------------------------------------------------
# inputs


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp32 values of an fp32 array or of bf16 bit patterns."""
    if dtype == BF16:
        return bf16_bits_to_f32(a)
    return np.asarray(a, dtype=np.float32)


# ---------------------------------------------------------------------------
# router


def router_logits_f64(x32: np.ndarray, wg: np.ndarray, bias: Optional[np.ndarray]) -> np.ndarray:
    """Unrounded logits: float64 products and sums, bias added in float64."""
    L = x32.astype(np.float64) @ wg.astype(np.float64).T
    if bias is not None:
        L = L + bias.astype(np.float64)[None, :]
    return L


def router_logits(x32: np.ndarray, wg: np.ndarray, bias: Optional[np.ndarray]) -> np.ndarray:
    """fp32 router logits [T, E]: the float64 sum rounded once to fp32."""
    L = router_logits_f64(x32, wg, bias).astype(np.float32)
    assert np.all(np.isfinite(L)), "router logits must be finite"
    return L


def summation_bound_rel(n_terms: int) -> float:
    """2 * gamma_{n-1}, gamma_m = m u / (1 - m u), u = 2^-53: twice the
    worst-case error of a float64 sum of n exactly known terms taken in any
    order of pairwise additions, relative to the sum of their magnitudes (the
    standard bound of recursive summation, e.g. Higham, "Accuracy and
    Stability of Numerical Algorithms", section 4.2).  Two float64 sums of the
    same n terms in different orders can differ by at most this much."""
    m = max(int(n_terms) - 1, 0)
    u = 2.0 ** -53
    return 2.0 * m * u / (1.0 - m * u)


def logits_near_midpoint(x32, wg, bias, rel: Optional[float] = None) -> np.ndarray:
    """Flag logits whose float64 sum lies so close to an fp32 rounding
    midpoint that another float64 summation order could round it the other
    way: within rel * sum_h |x[t,h] wg[e,h]| (+ |bias[e]|) of a midpoint, rel
    by default the two-order bound of summation_bound_rel over the H products
    and the bias.  Every other logit has one fp32 value whatever float64
    order the sum is taken in, so it is pinned bit for bit."""
    H = x32.shape[1]
    if rel is None:
        rel = summation_bound_rel(H + (1 if bias is not None else 0))
    L64 = router_logits_f64(x32, wg, bias)
    L32 = L64.astype(np.float32)
    up = np.nextafter(L32, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(L32, np.float32(-np.inf)).astype(np.float64)
    c = L32.astype(np.float64)
    d = np.minimum(np.abs(L64 - (c + up) / 2), np.abs(L64 - (c + dn) / 2))
    mag = np.abs(x32.astype(np.float64)) @ np.abs(wg.astype(np.float64)).T
    if bias is not None:
        mag = mag + np.abs(bias.astype(np.float64))[None, :]
    return d <= rel * mag


def select_topk(L: np.ndarray, k: int) -> np.ndarray:
    """ids[t, j]: the j-th expert when experts are ordered by logit descending,
    equal logits by expert index ascending (-0.0 equals +0.0)."""
    T, E = L.shape
    assert 1 <= k <= E
    # numpy's stable sort keeps equal keys in index order, and compares with
    # '<', under which -0.0 and +0.0 are equal.
    order = np.argsort(-L.astype(np.float64), axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def topk_weights(L: np.ndarray, ids: np.ndarray, renormalize: bool = True) -> np.ndarray:
    """Softmax over all experts at the selected ones, in float64, rounded
    once to fp32; with renormalize, divided by their sum first (so the k
    weights of a token sum to 1)."""
    L64 = L.astype(np.float64)
    z = L64 - L64.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renormalize:
        sel = sel / sel.sum(axis=1, keepdims=True)
    return sel.astype(np.float32)


# ---------------------------------------------------------------------------
# counts, offsets, permutation


def expert_counts(ids: np.ndarray, E: int) -> np.ndarray:
    return np.bincount(ids.ravel().astype(np.int64), minlength=E).astype(np.int32)


def expert_offsets(counts: np.ndarray) -> np.ndarray:
    """Exclusive offsets [E + 1]: offsets[0] = 0, offsets[E] = T * k."""
    out = np.zeros(counts.shape[0] + 1, dtype=np.int64)
    out[1:] = np.cumsum(counts.astype(np.int64))
    return out.astype(np.int32)


def route_permutation(ids: np.ndarray):
    """perm[p] = expanded route index r = t*k + j of permuted row p (the
    expanded ids stably sorted by expert); inv[r] = p."""
    flat = ids.ravel()
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.shape[0], dtype=np.int32)
    return perm, inv


def gather_rows(x: np.ndarray, perm: np.ndarray, k: int) -> np.ndarray:
    """Permuted input: row p is the token of route perm[p]."""
    return x[perm.astype(np.int64) // k]


# ---------------------------------------------------------------------------
# expert FFN


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + e^-z)."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(xr: np.ndarray, w1s, w2s, Im: int) -> np.ndarray:
    """Y = sum over micros m of (SiLU(X G_m^T) * (X U_m^T)) D_m^T, float64.

    xr: [n, H] rows; w1s[m]: [2Im, H] (gate rows, then up rows);
    w2s[m]: [H, Im]."""
    X = np.asarray(xr, dtype=np.float64)
    Y = np.zeros((X.shape[0], w2s[0].shape[0]), dtype=np.float64)
    for w1, w2 in zip(w1s, w2s):
        w1 = np.asarray(w1, dtype=np.float64)
        G = X @ w1[:Im].T
        U = X @ w1[Im:].T
        A = silu(G) * U
        Y += A @ np.asarray(w2, dtype=np.float64).T
    return Y


def finalize(Y: np.ndarray, inv: np.ndarray, w: np.ndarray) -> np.ndarray:
    """out[t] = sum_{j < k} w[t, j] * Y[inv[t*k + j]], j ascending, float64."""
    T, k = w.shape
    out = np.zeros((T, Y.shape[1]), dtype=np.float64)
    for j in range(k):
        rows = inv.reshape(T, k)[:, j].astype(np.int64)
        out += w[:, j].astype(np.float64)[:, None] * Y[rows]
    return out


# ---------------------------------------------------------------------------
# whole layer


def route(inp: LayerInputs) -> dict:
    """Router, top-k, weights, counts, offsets, permutation of one call."""
    sp = inp.spec
    x32 = widen(inp.x, sp.dtype)
    L = router_logits(x32, inp.wg, inp.bias)
    ids = select_topk(L, sp.k)
    w = topk_weights(L, ids, sp.renormalize)
    counts = expert_counts(ids, sp.E)
    offsets = expert_offsets(counts)
    perm, inv = route_permutation(ids)
    return dict(logits=L, ids=ids, w=w, counts=counts, offsets=offsets, perm=perm, inv=inv)


def expert_weights_f32(inp: LayerInputs, e: int):
    """fp32 micro slices of expert e, from the packed arrays when present,
    else regenerated from the expert's own seed stream."""
    sp = inp.spec
    if inp.w1.shape[2] == 2 * sp.Im:
        w1s = [widen(inp.w1[m, e], sp.dtype) for m in range(sp.micro)]
        w2s = [widen(inp.w2[m, e], sp.dtype) for m in range(sp.micro)]
    else:
        a, b = expert_pack(sp, e)
        w1s = [widen(v, sp.dtype) for v in a]
        w2s = [widen(v, sp.dtype) for v in b]
    return w1s, w2s


def forward(inp: LayerInputs, routing: Optional[dict] = None) -> dict:
    """The whole layer through the permuted, segmented path.

    Returns the routing fields plus Y [T*k, H] and out [T, H] in float64."""
    sp = inp.spec
    r = route(inp) if routing is None else routing
    x32 = widen(inp.x, sp.dtype)
    Xp = gather_rows(x32, r["perm"], sp.k)
    Y = np.zeros((sp.T * sp.k, sp.H), dtype=np.float64)
    off = r["offsets"]
    for e in range(sp.E):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        w1s, w2s = expert_weights_f32(inp, e)
        Y[a:b] = expert_ffn(Xp[a:b], w1s, w2s, sp.Im)
    out = finalize(Y, r["inv"], r["w"])
    return dict(r, Y=Y, out=out)


def shared_expert(inp: LayerInputs, w1s: np.ndarray, w2s: np.ndarray, tokens=None) -> np.ndarray:
    """The shared expert on every token (or on the listed tokens): the expert
    FFN above with one micro of width Is, float64.  w1s [2Is, H] (gate rows,
    then up rows), w2s [H, Is]."""
    sp = inp.spec
    x32 = widen(inp.x, sp.dtype)
    if tokens is not None:
        x32 = x32[np.asarray(tokens, dtype=np.int64)]
    Is = w2s.shape[1]
    return expert_ffn(x32, [widen(w1s, sp.dtype)], [widen(w2s, sp.dtype)], Is)


def forward_shared(inp: LayerInputs, w1s: np.ndarray, w2s: np.ndarray,
                   routing: Optional[dict] = None) -> dict:
    """The layer with its shared expert: out = the routed output + the shared
    expert's output (float64).  Also returns Ys, the shared output alone."""
    r = forward(inp, routing)
    ys = shared_expert(inp, w1s, w2s)
    return dict(r, Ys=ys, out=r["out"] + ys)


def token_outputs(inp: LayerInputs, routing: dict, tokens) -> np.ndarray:
    """out[t] for a few tokens, evaluated token by token from the definition
    sum_j w[t, j] * FFN_{ids[t, j]}(x_t), j ascending (no permutation)."""
    sp = inp.spec
    x32 = widen(inp.x, sp.dtype)
    tokens = [int(t) for t in tokens]
    need = {}
    for t in tokens:
        for j in range(sp.k):
            need.setdefault(int(routing["ids"][t, j]), []).append((t, j))
    ys = {}
    for e, uses in sorted(need.items()):
        w1s, w2s = expert_weights_f32(inp, e)
        rows = np.stack([x32[t] for t, _ in uses])
        for (t, j), y in zip(uses, expert_ffn(rows, w1s, w2s, sp.Im)):
            ys[(t, j)] = y
    out = np.zeros((len(tokens), sp.H), dtype=np.float64)
    for i, t in enumerate(tokens):
        for j in range(sp.k):
            out[i] += np.float64(routing["w"][t, j]) * ys[(t, j)]
    return out


# ---------------------------------------------------------------------------
# independent brute forces (tiny shapes)


def brute_rank_topk(L: np.ndarray, k: int) -> np.ndarray:
    """Top-k by rank counting, no sort: expert e has rank
    #{e' : L[e'] > L[e] or (L[e'] == L[e] and e' < e)}; it is selected iff its
    rank is below k, and its slot is its rank."""
    T, E = L.shape
    ids = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        for e in range(E):
            rank = 0
            for f in range(E):
                if L[t, f] > L[t, e] or (L[t, f] == L[t, e] and f < e):
                    rank += 1
            if rank < k:
                ids[t, rank] = e
    return ids


def brute_dense(x32: np.ndarray, ids: np.ndarray, w: np.ndarray, w13_full, down_full) -> np.ndarray:
    """out[t] = sum_e c[t, e] * down_e(SiLU(gate_e x_t) * up_e x_t), every expert
    evaluated densely on every token in float64, c[t, e] = w[t, j] where
    ids[t, j] = e and 0 elsewhere.  w13_full[e]: [2I, H] unsharded (gate rows
    then up rows); down_full[e]: [H, I]."""
    T = x32.shape[0]
    E = len(w13_full)
    X = x32.astype(np.float64)
    c = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        for j in range(ids.shape[1]):
            c[t, ids[t, j]] += np.float64(w[t, j])
    out = np.zeros((T, down_full[0].shape[0]), dtype=np.float64)
    for e in range(E):
        w13 = np.asarray(w13_full[e], dtype=np.float64)
        I = w13.shape[0] // 2
        g = X @ w13[:I].T
        u = X @ w13[I:].T
        a = (g / (1.0 + np.exp(-g))) * u
        out += c[:, e:e + 1] * (a @ np.asarray(down_full[e], dtype=np.float64).T)
    return out
