"""Pins of the CPU oracle against things other than itself: hand-worked
examples, exact arithmetic, brute force, closed forms and invariants.

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, a non-stable sort, gate and up
swapped) fails at least one test."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import moe_inputs as mi
import oracle as o

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- router


def test_router_logits_exact_on_dyadic_inputs():
    """Integer activations and power-of-two weights make every logit exactly
    representable; compare with exact rational arithmetic element by
    element (catches transposed or mis-indexed operands and a lost bias)."""
    rng = np.random.default_rng(11)
    T, H, E = 7, 33, 5
    x = rng.integers(-2, 3, size=(T, H)).astype(np.float32)
    wg = (rng.choice([-1.0, 1.0], size=(E, H)) * 2.0 ** -rng.integers(0, 6, size=(E, H))).astype(np.float32)
    b = (np.arange(E) * 0.25 - 0.5).astype(np.float32)
    L = o.router_logits(x, wg, b)
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(float(x[t, h])) * Fraction(float(wg[e, h])) for h in range(H)) + Fraction(float(b[e]))
            assert Fraction(float(L[t, e])) == exact, (t, e)


def test_router_logits_match_exactly_rounded_sum():
    """For random bf16 x and fp32 Wg, the exact sum rounded to fp32 (via
    math.fsum, which is correctly rounded) equals the oracle's logits except
    where the oracle itself flags a near-midpoint value."""
    sp = mi.custom_spec(T=16, H=512, E=16, k=4, Im=32, dtype=mi.BF16, seed=5)
    inp = mi.make_layer(sp)
    x32 = o.widen(inp.x, sp.dtype)
    L = o.router_logits(x32, inp.wg, inp.bias)
    flags = o.logits_near_midpoint(x32, inp.wg, inp.bias)
    for t in range(sp.T):
        for e in range(sp.E):
            s = math.fsum(float(a) * float(b) for a, b in zip(x32[t], inp.wg[e]))
            if not flags[t, e]:
                assert np.float32(s) == L[t, e], (t, e)


def _f32_of_fraction(F):
    """The fp32 value nearest to the exact rational F, ties to the even
    significand: chosen among the fp32 neighbours of float(F) by exact
    rational distance (no double rounding through float64)."""
    c = np.float32(float(F))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    return min(cands, key=lambda v: (abs(Fraction(float(v)) - F), int(np.float32(v).view(np.uint32)) & 1))


def _dyadic_router(terms):
    """One token, one expert, H = len(terms) products x_h * w_h = terms[h],
    each term a power of two times +-1 split as x = 2^a, w = +-2^b."""
    x = np.array([[2.0 ** (math.frexp(abs(t))[1] // 2)] for t in terms], np.float64).T
    w = (np.array(terms, np.float64) / x[0])[None, :]
    return x.astype(np.float32), w.astype(np.float32)


def test_midpoint_guard_flags_exact_midpoint():
    """1 + 2^-24 is exactly halfway between the fp32 neighbours 1 and
    1 + 2^-23: its rounding depends on the last bit of any float64 sum, so
    the guard must flag it (and its negative, and 3 * 2^-30 + 2^-53, the
    midpoint above 3 * 2^-30 in a binade of ulp 2^-52); 1.5 is an fp32 value,
    half an ulp from either midpoint, and must not be flagged."""
    for terms, want in (([1.0, 2.0 ** -24], True), ([-1.0, -(2.0 ** -24)], True),
                        ([1.0, 0.5], False), ([3.0 * 2.0 ** -30, 2.0 ** -53], True)):
        x, w = _dyadic_router(terms)
        assert float((x.astype(np.float64) @ w.astype(np.float64).T)[0, 0]) == sum(terms)
        assert bool(o.logits_near_midpoint(x, w, None)[0, 0]) is want, terms


def test_midpoint_guard_bound_scales_with_terms():
    """Three exact terms 1 + 2^-24 + d: the sum is d from a midpoint and the
    bound of two float64 orders over three terms is 2 * 2u * (1 + ...) ~
    2^-51 of the magnitude.  d = 2^-51 must be flagged; d = 2^-50 and 2^-48
    (well inside a fixed 2^-40, which the bound reaches only at H ~ 4096)
    must not."""
    assert o.summation_bound_rel(3) == pytest.approx(2.0 ** -51, rel=1e-12)
    assert o.summation_bound_rel(4097) == pytest.approx(2.0 ** -40, rel=1e-12)
    for d, want in ((2.0 ** -51, True), (2.0 ** -50, False), (2.0 ** -48, False)):
        x, w = _dyadic_router([1.0, 2.0 ** -24, d])
        assert bool(o.logits_near_midpoint(x, w, None)[0, 0]) is want, d
    # a bias term is one more summand: 2^-51 away is still inside the bound
    x, w = _dyadic_router([1.0, 2.0 ** -24])
    assert bool(o.logits_near_midpoint(x, w, np.array([2.0 ** -51], np.float32))[0, 0])
    assert not o.logits_near_midpoint(x, w, np.array([2.0 ** -47], np.float32))[0, 0]


def test_unflagged_logits_are_the_exact_sum_correctly_rounded():
    """What the guard leaves unflagged is pinned: there, the oracle's logit
    is the exact rational sum rounded once to fp32 (round to nearest even),
    computed here without float64.  Activations are bf16 of N(0,1), router
    rows fp32 of N(0, 0.1), plus rows built to sit near midpoints.  The
    guard flags only a small fraction of random logits."""
    rng = np.random.default_rng(8)
    T, H, E = 12, 96, 10
    x = mi.bf16_bits_to_f32(mi.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)))
    wg = (rng.standard_normal((E, H)) * 0.1).astype(np.float32)
    b = (rng.standard_normal(E) * 0.5).astype(np.float32)
    # token 0 / expert 0: 1 + 2^-24 + 2^-60 exactly (a midpoint plus a hair)
    x[0] = 0.0
    wg[0] = 0.0
    x[0, :3] = [1.0, 2.0 ** -12, 2.0 ** -30]
    wg[0, :3] = [1.0, 2.0 ** -12, 2.0 ** -30]
    b[0] = 0.0
    L = o.router_logits(x, wg, b)
    flags = o.logits_near_midpoint(x, wg, b)
    assert flags[0, 0]
    assert flags.mean() < 0.02
    checked = 0
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(float(x[t, h])) * Fraction(float(wg[e, h])) for h in range(H)) + Fraction(float(b[e]))
            if not flags[t, e]:
                assert L[t, e].view(np.uint32) == _f32_of_fraction(exact).view(np.uint32), (t, e)
                checked += 1
    assert checked >= T * E - 3


def test_router_bias_shifts_logits():
    x = np.ones((2, 4), np.float32)
    wg = np.zeros((3, 4), np.float32)
    b = np.array([0.5, -1.0, 2.0], np.float32)
    assert np.array_equal(o.router_logits(x, wg, b), np.tile(b, (2, 1)))


# ---------------------------------------------------------------- top-k


def test_worked_routing_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "routing_worked_example.json")))
    L = np.array(g["logits"], np.float32)
    k = g["k"]
    ids = o.select_topk(L, k)
    assert ids.tolist() == g["ids"]
    w = o.topk_weights(L, ids)
    np.testing.assert_allclose(w, np.array(g["weights"]), rtol=1e-7, atol=0)
    counts = o.expert_counts(ids, L.shape[1])
    assert counts.tolist() == g["counts"]
    assert o.expert_offsets(counts).tolist() == g["offsets"]
    perm, inv = o.route_permutation(ids)
    assert perm.tolist() == g["perm"]
    assert inv.tolist() == g["inv"]


@pytest.mark.parametrize("E,k", [(8, 2), (8, 1), (8, 8), (16, 5), (64, 8), (3, 3)])
def test_topk_matches_rank_count_bruteforce(E, k):
    rng = np.random.default_rng(E * 100 + k)
    T = 24
    # quantised logits create many exact ties
    L = (rng.integers(-4, 5, size=(T, E)) * 0.5).astype(np.float32)
    assert np.array_equal(o.select_topk(L, k), o.brute_rank_topk(L, k))
    L2 = rng.standard_normal((T, E)).astype(np.float32)
    assert np.array_equal(o.select_topk(L2, k), o.brute_rank_topk(L2, k))


def test_topk_ties_and_signed_zero():
    # all equal -> 0..k-1
    assert o.select_topk(np.zeros((1, 6), np.float32), 3).tolist() == [[0, 1, 2]]
    # a tie straddling the k boundary: lower index wins
    L = np.array([[1.0, 2.0, 1.0, 1.0]], np.float32)
    assert o.select_topk(L, 2).tolist() == [[1, 0]]
    # -0.0 and +0.0 are equal: index order decides, both ways round
    L = np.array([[-0.0, 0.0, -1.0]], np.float32)
    assert o.select_topk(L, 1).tolist() == [[0]]
    L = np.array([[0.0, -0.0, -1.0]], np.float32)
    assert o.select_topk(L, 1).tolist() == [[0]]
    # k = E gives the full stable descending order
    L = np.array([[0.5, 2.0, 0.5, -3.0, 2.0]], np.float32)
    assert o.select_topk(L, 5).tolist() == [[1, 4, 0, 2, 3]]


def test_topk_weights_properties():
    rng = np.random.default_rng(3)
    L = (rng.standard_normal((50, 16)) * 2).astype(np.float32)
    for k in (1, 3, 16):
        ids = o.select_topk(L, k)
        w = o.topk_weights(L, ids)
        assert w.dtype == np.float32
        np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=2e-7 * k)
        assert np.all(np.diff(w, axis=1) <= 0)
        if k == 1:
            assert np.all(w == 1.0)
    # k = E: the plain softmax (scipy's, an independent routine), in expert order
    from scipy.special import softmax
    ids = o.select_topk(L, 16)
    w = o.topk_weights(L, ids)
    ref = softmax(L.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(ref, ids, axis=1), rtol=1e-6)
    # renormalisation off: scipy's softmax over all experts at the selected
    # ones, for every k (summing to less than 1 below k = E)
    for k in (1, 3, 16):
        ids = o.select_topk(L, k)
        w = o.topk_weights(L, ids, renormalize=False)
        np.testing.assert_allclose(w, np.take_along_axis(ref, ids, axis=1), rtol=1e-6)
        if k < 16:
            assert np.all(w.sum(axis=1) < 1.0)
    # two selected experts: closed form sigmoid of the logit gap
    L = np.array([[0.3, -1.2, 5.0]], np.float32)
    ids = o.select_topk(L, 2)
    assert ids.tolist() == [[2, 0]]
    w = o.topk_weights(L, ids)
    d = float(L[0, 2]) - float(L[0, 0])
    np.testing.assert_allclose(w[0], [1 / (1 + math.exp(-d)), 1 / (1 + math.exp(d))], rtol=1e-7)


# ---------------------------------------------------------------- permutation


def _perm_bruteforce(ids, E):
    """Expert by expert, walk the routes in order and append matches."""
    flat = ids.ravel().tolist()
    perm = []
    for e in range(E):
        for r, v in enumerate(flat):
            if v == e:
                perm.append(r)
    return perm


@pytest.mark.parametrize("T,E,k,seed", [(1, 4, 1, 0), (37, 8, 2, 1), (64, 64, 8, 2), (5, 6, 6, 3)])
def test_permutation_invariants_and_bruteforce(T, E, k, seed):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((T, E)).astype(np.float32)
    ids = o.select_topk(L, k)
    counts = o.expert_counts(ids, E)
    offsets = o.expert_offsets(counts)
    perm, inv = o.route_permutation(ids)
    assert counts.sum() == T * k
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.diff(offsets), counts)
    assert sorted(perm.tolist()) == list(range(T * k))
    assert np.array_equal(inv[perm], np.arange(T * k))
    flat = ids.ravel()
    assert np.all(np.diff(flat[perm]) >= 0)
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)
    for t in range(T):
        assert len(set(ids[t].tolist())) == k
    assert perm.tolist() == _perm_bruteforce(ids, E)


def test_gather_rows():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((6, 3)).astype(np.float32)
    ids = o.select_topk(rng.standard_normal((6, 4)).astype(np.float32), 2)
    perm, _ = o.route_permutation(ids)
    Xp = o.gather_rows(x, perm, 2)
    for p in range(12):
        assert np.array_equal(Xp[p], x[perm[p] // 2])


# ---------------------------------------------------------------- SwiGLU / FFN


def test_silu_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0, 3.5, -3.5, 800.0, -800.0])
    s = o.silu(z)
    assert s[0] == 0.0
    assert s[1] == pytest.approx(0.7310585786300049, rel=1e-15)   # 1 / (1 + e^-1)
    assert s[3] == pytest.approx(40.0, rel=1e-15)
    assert -1e-15 < s[4] < 0.0
    assert s[5] - s[6] == pytest.approx(3.5, rel=1e-15)           # SiLU(z) - SiLU(-z) = z
    assert s[7] == 800.0 and s[8] == 0.0


def test_swiglu_ffn_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "swiglu_ffn_worked_example.json")))
    x = np.array(g["x"])
    w13 = np.array(g["w13"])
    down = np.array(g["down"])
    y = o.expert_ffn(x, [w13], [down], Im=1)
    np.testing.assert_allclose(y, np.array(g["out"]), rtol=1e-15)
    # and through the whole routed path with E = k = 1
    sp = mi.custom_spec(T=1, H=2, E=1, k=1, Im=1, dtype=mi.F32)
    inp = mi.LayerInputs(sp, x.astype(np.float32), np.ones((1, 2), np.float32), None,
                         w13[None, None].astype(np.float32), down[None, None].astype(np.float32))
    r = o.forward(inp)
    np.testing.assert_allclose(r["out"], np.array(g["out"]), rtol=1e-15)


def test_gate_and_up_are_not_interchangeable():
    """SiLU goes on the first half (gate); swapping halves changes the result."""
    x = np.array([[1.0, 2.0]])
    w13 = np.array([[1.0, 0.0], [0.0, 1.0]])
    down = np.array([[1.0]])
    y = o.expert_ffn(x, [w13], [down], Im=1)
    assert y[0, 0] == pytest.approx(2.0 / (1.0 + math.exp(-1.0)))
    assert y[0, 0] != pytest.approx(1.0 * 2.0 / (1.0 + math.exp(-2.0)))


def test_e1_k1_reduces_to_textbook_ffn():
    """With one expert the routed layer is the plain SwiGLU FFN, written here
    with explicit Python loops."""
    sp = mi.custom_spec(T=3, H=5, E=1, k=1, Im=4, dtype=mi.F32, seed=9)
    inp = mi.make_layer(sp)
    r = o.forward(inp)
    W = inp.w1[0, 0].astype(np.float64)
    D = inp.w2[0, 0].astype(np.float64)
    for t in range(3):
        xv = inp.x[t].astype(np.float64)
        h = []
        for i in range(4):
            g = sum(W[i, c] * xv[c] for c in range(5))
            u = sum(W[4 + i, c] * xv[c] for c in range(5))
            h.append(g / (1 + math.exp(-g)) * u)
        for c in range(5):
            y = sum(D[c, i] * h[i] for i in range(4))
            assert r["out"][t, c] == pytest.approx(y, rel=1e-12, abs=1e-15)


def _unsharded(inp):
    """Rebuild each expert's unsharded w13 [2I, H] and down [H, I] from the
    micro pack by undoing the paired split."""
    sp = inp.spec
    w13s, downs = [], []
    for e in range(sp.E):
        w1s, w2s = o.expert_weights_f32(inp, e)
        gate = np.concatenate([w[:sp.Im] for w in w1s])
        up = np.concatenate([w[sp.Im:] for w in w1s])
        w13s.append(np.concatenate([gate, up]))
        downs.append(np.concatenate(w2s, axis=1))
    return w13s, downs


@pytest.mark.parametrize("cfg", [
    dict(T=40, H=48, E=8, k=2, Im=16, micro=1, seed=1),
    dict(T=33, H=64, E=6, k=3, Im=8, micro=2, seed=2),
    dict(T=17, H=32, E=5, k=5, Im=8, micro=1, seed=3),
    dict(T=50, H=32, E=8, k=2, Im=8, micro=2, seed=4, zipf={"s": 1.2, "scale": 6.0, "seed": 4}),
])
def test_forward_matches_dense_bruteforce(cfg):
    zipf = cfg.pop("zipf", None)
    sp = mi.custom_spec(dtype=mi.F32, zipf=zipf, **cfg)
    inp = mi.make_layer(sp)
    r = o.forward(inp)
    w13s, downs = _unsharded(inp)
    ref = o.brute_dense(o.widen(inp.x, sp.dtype), r["ids"], r["w"], w13s, downs)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-11, atol=1e-14)
    if zipf is not None:
        assert (r["counts"] == 0).any(), "skewed bias should leave an expert empty"


def test_tiny_layer_matches_dense_bruteforce():
    inp = mi.make_layer("tiny_fp32")
    r = o.forward(inp)
    w13s, downs = _unsharded(inp)
    ref = o.brute_dense(o.widen(inp.x, inp.spec.dtype), r["ids"], r["w"], w13s, downs)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-11, atol=1e-14)


# ---------------------------------------------------------------- shared expert


@pytest.mark.parametrize("cfg", [
    dict(T=40, H=48, E=8, k=2, Im=16, micro=1, seed=21),
    dict(T=25, H=64, E=6, k=3, Im=8, micro=2, seed=22),
    dict(T=30, H=32, E=5, k=2, Im=8, micro=1, seed=23, Is=24),  # shared width != routed width
])
def test_shared_expert_matches_dense_bruteforce(cfg):
    """The layer with its shared expert against the dense brute force with
    the shared expert as one more expert whose coefficient is 1 for every
    token (brute_dense's own FFN code, not the oracle's expert_ffn)."""
    cfg = dict(cfg)
    Is = cfg.pop("Is", None)
    sp = mi.custom_spec(dtype=mi.F32, **cfg)
    inp = mi.make_layer(sp)
    w1s, w2s = mi.make_shared(sp, Is)
    r = o.forward_shared(inp, w1s, w2s)
    w13s, downs = _unsharded(inp)
    ids = np.concatenate([r["ids"], np.full((sp.T, 1), sp.E, dtype=np.int32)], axis=1)
    w = np.concatenate([r["w"], np.ones((sp.T, 1), dtype=np.float32)], axis=1)
    ref = o.brute_dense(o.widen(inp.x, sp.dtype), ids, w, w13s + [w1s], downs + [w2s])
    np.testing.assert_allclose(r["out"], ref, rtol=1e-11, atol=1e-14)
    # the shared part is not negligible: dropping it fails the comparison
    assert np.abs(r["Ys"]).max() > 1e3 * np.abs(r["out"] - ref).max()


def test_shared_expert_gate_up_order_and_zero_down():
    """Gate rows first: swapping the halves of w1s changes the output (SiLU is
    not symmetric); a zero down projection leaves the routed layer exactly."""
    sp = mi.custom_spec(T=12, H=32, E=4, k=2, Im=8, dtype=mi.F32, seed=23)
    inp = mi.make_layer(sp)
    w1s, w2s = mi.make_shared(sp)
    Is = w2s.shape[1]
    base = o.forward(inp)["out"]
    r = o.forward_shared(inp, w1s, w2s)
    sw = o.forward_shared(inp, np.concatenate([w1s[Is:], w1s[:Is]]), w2s)
    assert np.abs(r["out"] - sw["out"]).max() > 1e-4
    z = o.forward_shared(inp, w1s, np.zeros_like(w2s))
    assert np.array_equal(z["out"], base)
    # one token by hand: ys[t] = w2s @ (SiLU(g) * u)
    x = inp.x[5].astype(np.float64)
    g = w1s[:Is].astype(np.float64) @ x
    u = w1s[Is:].astype(np.float64) @ x
    ys = w2s.astype(np.float64) @ ((g / (1.0 + np.exp(-g))) * u)
    np.testing.assert_allclose(r["Ys"][5], ys, rtol=1e-12, atol=1e-15)


def test_token_outputs_match_forward():
    sp = mi.custom_spec(T=30, H=32, E=8, k=3, Im=8, micro=2, dtype=mi.BF16, seed=8)
    inp = mi.make_layer(sp)
    r = o.forward(inp)
    toks = [0, 7, 29]
    np.testing.assert_allclose(o.token_outputs(inp, r, toks), r["out"][toks], rtol=1e-12, atol=1e-15)
    # and with weights regenerated per expert instead of read from the pack
    lean = mi.make_layer(sp, weights=False)
    np.testing.assert_allclose(o.token_outputs(lean, r, toks), r["out"][toks], rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- micro / TP2 invariants


def _micro_view(inp, m):
    sp = inp.spec
    vs = mi.LayerSpec(sp.name + f"_view{m}", sp.T, sp.H, sp.E, sp.k, sp.Im, 1, sp.dtype,
                      sp.x_seed, sp.layer_seed, sp.sigma_x, sp.sigma_g, sp.sigma_w, sp.zipf_bias)
    return mi.LayerInputs(vs, inp.x, inp.wg, inp.bias, inp.w1[m:m + 1], inp.w2[m:m + 1])


def test_micro_views_sum_to_multi_micro_and_expert_major():
    """fwd(micro0 view) + fwd(micro1 view) = fwd(2-micro pack) = fwd(the same
    shard stored expert-major as one micro of width 2*Im)."""
    two = mi.custom_spec(T=24, H=32, E=6, k=2, Im=8, micro=2, dtype=mi.F32, seed=21)
    one = mi.custom_spec(T=24, H=32, E=6, k=2, Im=16, micro=1, dtype=mi.F32, seed=21)
    a, b = mi.make_layer(two), mi.make_layer(one)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.wg, b.wg)
    ra, rb = o.forward(a), o.forward(b)
    for f in ("ids", "w", "perm", "inv", "offsets"):
        assert np.array_equal(ra[f], rb[f])
    np.testing.assert_allclose(ra["out"], rb["out"], rtol=1e-12, atol=1e-15)
    v0 = o.forward(_micro_view(a, 0))
    v1 = o.forward(_micro_view(a, 1))
    np.testing.assert_allclose(v0["out"] + v1["out"], ra["out"], rtol=1e-12, atol=1e-15)


def test_tp2_halves_sum_to_unsharded():
    """Split an unsharded layer (intermediate 2I) into storage shards A and B:
    the paired column split of w13 and the row split of down.  With the
    replicated router, fwd(A) + fwd(B) = fwd(full)."""
    full = mi.custom_spec(T=20, H=24, E=4, k=2, Im=12, micro=1, dtype=mi.F32, seed=31)
    inp = mi.make_layer(full)
    I = full.Im
    halves = []
    for s in range(2):
        lo, hi = s * I // 2, (s + 1) * I // 2
        w1 = np.concatenate([inp.w1[:, :, lo:hi], inp.w1[:, :, I + lo:I + hi]], axis=2)
        w2 = np.ascontiguousarray(inp.w2[:, :, :, lo:hi])
        hs = mi.custom_spec(T=20, H=24, E=4, k=2, Im=I // 2, micro=1, dtype=mi.F32, seed=31)
        halves.append(o.forward(mi.LayerInputs(hs, inp.x, inp.wg, None, w1, w2))["out"])
    np.testing.assert_allclose(halves[0] + halves[1], o.forward(inp)["out"], rtol=1e-12, atol=1e-15)


def test_token_permutation_equivariance():
    sp = mi.custom_spec(T=16, H=32, E=8, k=2, Im=8, micro=1, dtype=mi.F32, seed=41)
    inp = mi.make_layer(sp)
    r = o.forward(inp)
    pi = np.random.default_rng(0).permutation(sp.T)
    inp2 = mi.LayerInputs(sp, inp.x[pi], inp.wg, inp.bias, inp.w1, inp.w2)
    r2 = o.forward(inp2)
    assert np.array_equal(r2["ids"], r["ids"][pi])
    np.testing.assert_allclose(r2["out"], r["out"][pi], rtol=1e-12, atol=1e-15)


def test_expert_relabelling_invariance():
    sp = mi.custom_spec(T=16, H=32, E=8, k=2, Im=8, micro=1, dtype=mi.F32, seed=42)
    inp = mi.make_layer(sp)
    r = o.forward(inp)
    sigma = np.random.default_rng(1).permutation(sp.E)
    inp2 = mi.LayerInputs(sp, inp.x, inp.wg[sigma], None, inp.w1[:, sigma], inp.w2[:, sigma])
    r2 = o.forward(inp2)
    np.testing.assert_allclose(r2["out"], r["out"], rtol=1e-12, atol=1e-15)
