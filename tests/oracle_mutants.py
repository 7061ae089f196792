"""Plausible mistakes, planted in the CPU oracle (never in the HIP path), to
show that its pins catch each one.  ``apply(name)`` replaces one oracle
function, in the oracle module and in the package that re-exports it, with a
wrong version; the pins in test_oracle.py and test_oracle_properties.py must
then fail.  Used only by test_oracle_mutants.py, through the conftest hook
that reads MOE_ORACLE_MUTANT in a child pytest process."""
import numpy as np

import oracle
from oracle import moe_oracle as m

_orig = {name: getattr(m, name) for name in (
    "router_logits_f64", "select_topk", "topk_weights", "route_permutation", "silu", "expert_ffn",
    "finalize", "logits_near_midpoint")}


def _gate_up_swap(xr, w1s, w2s, Im):
    # SiLU on the up half instead of the gate half
    return _orig["expert_ffn"](xr, [np.concatenate([w[Im:], w[:Im]]) for w in w1s], w2s, Im)


def _unstable_sort(ids):
    # rows of one expert in decreasing route order
    flat = ids.ravel()
    R = flat.shape[0]
    perm = np.lexsort((-np.arange(R), flat)).astype(np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(R, dtype=np.int32)
    return perm, inv


def _dropped_bias(x32, wg, bias):
    return _orig["router_logits_f64"](x32, wg, None)


def _upper_index_ties(L, k):
    # equal logits go to the higher expert index
    E = L.shape[1]
    order = np.argsort(-L[:, ::-1].astype(np.float64), axis=1, kind="stable")
    return (E - 1 - order[:, :k]).astype(np.int32)


def _no_renormalisation(L, ids, renormalize=True):
    L64 = L.astype(np.float64)
    z = L64 - L64.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    return np.take_along_axis(p, ids.astype(np.int64), axis=1).astype(np.float32)


def _renormalise_always(L, ids, renormalize=True):
    # the flag ignored: weights renormalised even when it is off
    return _orig["topk_weights"](L, ids, True)


def _swapped_perm_inv(ids):
    perm, inv = _orig["route_permutation"](ids)
    return inv, perm


def _wrong_finalize_slot(Y, inv, w):
    # weight j applied to the row of slot (j + 1) mod k
    return _orig["finalize"](Y, inv, np.roll(w, 1, axis=1))


def _silu_sign(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(z))


def _dropped_micro(xr, w1s, w2s, Im):
    return _orig["expert_ffn"](xr, w1s[:1], w2s[:1], Im)


def _dropped_hidden_term(x32, wg, bias):
    # the last hidden column left out of the router sum
    return _orig["router_logits_f64"](x32[:, :-1], wg[:, :-1], bias)


def _guard_overflags(x32, wg, bias, rel=None):
    # a slip in the midpoint bound (2^-20 for 2^-40): every logit excused
    return _orig["logits_near_midpoint"](x32, wg, bias, rel=2.0 ** -20)


def _guard_fixed_bound(x32, wg, bias, rel=None):
    # the bound of 4096-term sums used whatever the number of terms
    return _orig["logits_near_midpoint"](x32, wg, bias, rel=2.0 ** -40)


def _guard_flags_nothing(x32, wg, bias, rel=None):
    return np.zeros((x32.shape[0], wg.shape[0]), dtype=bool)


MUTANTS = {
    "gate_up_swap": ("expert_ffn", _gate_up_swap),
    "unstable_sort": ("route_permutation", _unstable_sort),
    "dropped_bias": ("router_logits_f64", _dropped_bias),
    "upper_index_ties": ("select_topk", _upper_index_ties),
    "no_renormalisation": ("topk_weights", _no_renormalisation),
    "renormalise_always": ("topk_weights", _renormalise_always),
    "swapped_perm_inv": ("route_permutation", _swapped_perm_inv),
    "wrong_finalize_slot": ("finalize", _wrong_finalize_slot),
    "silu_sign": ("silu", _silu_sign),
    "dropped_micro": ("expert_ffn", _dropped_micro),
    "dropped_hidden_term": ("router_logits_f64", _dropped_hidden_term),
    "guard_overflags": ("logits_near_midpoint", _guard_overflags),
    "guard_fixed_bound": ("logits_near_midpoint", _guard_fixed_bound),
    "guard_flags_nothing": ("logits_near_midpoint", _guard_flags_nothing),
}


def apply(name: str) -> None:
    fn_name, fn = MUTANTS[name]
    setattr(m, fn_name, fn)
    setattr(oracle, fn_name, fn)
