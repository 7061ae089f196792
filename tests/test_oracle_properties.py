"""Property tests of the CPU oracle (hypothesis): random tiny cases against
formulations that share no code with the oracle's path (rank counting
instead of sorting, dense evaluation of every expert instead of the
permuted segments) and against invariants that any correct result obeys."""
import math

import numpy as np
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

import moe_inputs as mi  # noqa: E402
import oracle as o  # noqa: E402

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

FAST = settings(max_examples=40, deadline=None, derandomize=True)


@st.composite
def logit_tables(draw):
    """[T, E] fp32 logits from a small value set, so exact ties and signed
    zeros are frequent, and a k in [1, E]."""
    T = draw(st.integers(1, 6))
    E = draw(st.integers(1, 12))
    k = draw(st.integers(1, E))
    vals = [-2.0, -1.0, -0.0, 0.0, 0.5, 1.0, 1.5, 3.0]
    flat = draw(st.lists(st.sampled_from(vals), min_size=T * E, max_size=T * E))
    return np.array(flat, dtype=np.float32).reshape(T, E), k


@FAST
@given(logit_tables())
def test_topk_equals_rank_count(case):
    L, k = case
    assert np.array_equal(o.select_topk(L, k), o.brute_rank_topk(L, k))


@FAST
@given(logit_tables())
def test_topk_weights_properties(case):
    L, k = case
    ids = o.select_topk(L, k)
    w = o.topk_weights(L, ids)
    T = L.shape[0]
    for t in range(T):
        # the selection is k distinct experts whose logits are non-increasing
        assert len(set(ids[t].tolist())) == k
        sel = [float(L[t, e]) for e in ids[t]]
        assert all(sel[j] >= sel[j + 1] for j in range(k - 1))
        # the weights: a distribution over the k, ordered like the logits, and
        # the softmax of the selected logits (written here with math.exp)
        assert abs(float(w[t].astype(np.float64).sum()) - 1.0) <= 2e-7 * k
        assert all(w[t, j] >= w[t, j + 1] for j in range(k - 1))
        m = max(sel)
        ex = [math.exp(v - m) for v in sel]
        ref = [v / sum(ex) for v in ex]
        assert np.allclose(w[t], ref, rtol=1e-6, atol=1e-7)


@st.composite
def id_tables(draw):
    """[T, k] expert ids, distinct within each token."""
    T = draw(st.integers(1, 20))
    E = draw(st.integers(1, 10))
    k = draw(st.integers(1, E))
    rows = [draw(st.permutations(list(range(E))))[:k] for _ in range(T)]
    return np.array(rows, dtype=np.int32).reshape(T, k), E


@FAST
@given(id_tables())
def test_permutation_invariants(case):
    ids, E = case
    R = ids.size
    counts = o.expert_counts(ids, E)
    offsets = o.expert_offsets(counts)
    perm, inv = o.route_permutation(ids)
    assert counts.sum() == R and offsets[0] == 0 and offsets[E] == R
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(np.sort(perm), np.arange(R))
    assert np.array_equal(inv[perm], np.arange(R))
    flat = ids.ravel()
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert (flat[seg] == e).all()
        assert (np.diff(seg) > 0).all()  # stable: routes of one expert in route order


@st.composite
def tiny_layers(draw):
    T = draw(st.integers(1, 10))
    H = draw(st.sampled_from([4, 8, 12]))
    E = draw(st.integers(1, 6))
    k = draw(st.integers(1, E))
    Im = draw(st.sampled_from([2, 4]))
    micro = draw(st.integers(1, 2))
    seed = draw(st.integers(0, 10_000))
    return mi.custom_spec(T=T, H=H, E=E, k=k, Im=Im, micro=micro, dtype=mi.F32, seed=seed)


def _unsharded(inp):
    sp = inp.spec
    w13s, downs = [], []
    for e in range(sp.E):
        w1s, w2s = o.expert_weights_f32(inp, e)
        gate = np.concatenate([w[:sp.Im] for w in w1s])
        up = np.concatenate([w[sp.Im:] for w in w1s])
        w13s.append(np.concatenate([gate, up]))
        downs.append(np.concatenate(w2s, axis=1))
    return w13s, downs


@FAST
@given(tiny_layers(), st.booleans())
def test_layer_equals_dense_bruteforce(sp, with_shared):
    """The permuted, segmented layer (with or without a shared expert)
    against every expert evaluated densely on every token."""
    inp = mi.make_layer(sp)
    w13s, downs = _unsharded(inp)
    x32 = o.widen(inp.x, sp.dtype)
    if with_shared:
        w1s, w2s = mi.make_shared(sp)
        r = o.forward_shared(inp, w1s, w2s)
        ids = np.concatenate([r["ids"], np.full((sp.T, 1), sp.E, dtype=np.int32)], axis=1)
        w = np.concatenate([r["w"], np.ones((sp.T, 1), dtype=np.float32)], axis=1)
        ref = o.brute_dense(x32, ids, w, w13s + [w1s], downs + [w2s])
    else:
        r = o.forward(inp)
        ref = o.brute_dense(x32, r["ids"], r["w"], w13s, downs)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-10, atol=1e-13)
