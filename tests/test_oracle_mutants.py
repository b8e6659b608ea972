"""Planted mistakes in a private copy of the oracle (CPU only): each must be
caught by at least one pin, which shows the pins constrain what they claim."""
import importlib.util
import os

import numpy as np
import pytest

from pins import ALL_CHECKS

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "moe_oracle.py")


def _fresh_oracle():
    spec = importlib.util.spec_from_file_location("oracle_mutant_copy", ORACLE_SRC)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _renormalised_gates(O):
    orig = O.route

    def route(logits, k, acc=np.float64):
        idx, gate = orig(logits, k, acc)
        return idx, gate / gate.sum(axis=1, keepdims=True)
    return route


def _ties_to_higher_index(O):
    def route(logits, k, acc=np.float64):
        key = np.asarray(logits, np.float32)
        T, E = key.shape
        p = O.softmax(logits, acc)
        order = np.lexsort((-np.broadcast_to(np.arange(E), (T, E)), -key), axis=-1)
        idx = order[:, :k].astype(np.int32)
        return idx, np.take_along_axis(p, idx, axis=-1)
    return route


def _unstable_permute(O):
    orig = O.permute

    def permute(x, idx, E):
        xp, counts, offsets, rmap, src = orig(x, idx, E)
        # reverse token order inside each group
        rmap = rmap.copy()
        for e in range(E):
            lo, hi = offsets[e], offsets[e + 1]
            sel = (rmap >= lo) & (rmap < hi)
            rmap[sel] = lo + hi - 1 - rmap[sel]
        src = np.empty_like(src)
        src[rmap.ravel()] = np.repeat(np.arange(idx.shape[0]), idx.shape[1])
        return x[src], counts, offsets, rmap, src
    return permute


def _swapped_gate_up(O):
    def expert_forward(xr, w13, w2, acc=np.float64):
        I = w2.shape[1]
        w = np.concatenate([w13[I:], w13[:I]])
        xr = np.asarray(xr, acc)
        g = xr @ w[:I].T
        u = xr @ w[I:].T
        act = O.silu(g) * u
        return np.concatenate([u, g], axis=1), act, act @ np.asarray(w2, acc).T
    return expert_forward


def _silu_sign(O):
    return lambda z: z / (1.0 + np.exp(z))


def _combine_without_gate(O):
    orig = O.combine

    def combine(yp, rmap, gate, y_shared=None, acc=np.float64):
        return orig(yp, rmap, np.ones_like(gate), y_shared, acc)
    return combine


def _route_bwd_sign(O):
    orig = O.route_backward
    return lambda logits, idx, dgate, acc=np.float64: -orig(logits, idx, dgate, acc)


def _silu_grad_missing_term(O):
    orig = O.expert_backward

    def expert_backward(xr, w13, w2, dyr, acc=np.float64):
        xr, w13, w2, dyr = (np.asarray(a, acc) for a in (xr, w13, w2, dyr))
        I = w2.shape[1]
        g = xr @ w13[:I].T
        u = xr @ w13[I:].T
        sig = 1.0 / (1.0 + np.exp(-g))
        act = g * sig * u
        da = dyr @ w2
        dg = da * u * sig                       # drops the (1 + g(1 - sig)) factor
        du = da * g * sig
        dh13 = np.concatenate([dg, du], axis=1)
        return dh13, dh13 @ w13, dh13.T @ xr, dyr.T @ act
    return expert_backward


def _dropped_shared(O):
    orig = O.layer_forward

    def layer_forward(*a, **kw):
        kw = dict(kw)
        out = orig(*a, **kw)
        if kw.get("ws13") is not None:
            out["y"] = out["y"] - out["ys"]
        return out
    return layer_forward


def _sample_std_cv(O):
    orig = O.load_stats

    def load_stats(counts, experts_per_group=1):
        load, cv, g, gcv = orig(counts, experts_per_group)
        E, G = len(counts), len(g)
        fix = lambda v, n: v * np.sqrt(n / (n - 1)) if n > 1 else v
        return load, fix(cv, E), g, fix(gcv, G)
    return load_stats


def _strided_groups(O):
    orig = O.load_stats

    def load_stats(counts, experts_per_group=1):
        c = np.asarray(counts, np.int64)
        G = len(c) // experts_per_group
        load, cv, _, _ = orig(c, experts_per_group)
        g = c.reshape(experts_per_group, G).sum(axis=0)   # expert e in group e % G
        _, gcv, _, _ = orig(g, 1)
        return load, cv, g, gcv
    return load_stats


def _drop_last_pairs(O):
    orig = O.permute_capacity

    def permute_capacity(x, idx, E, C):
        # keeps each expert's last C pairs instead of its first C
        T, k = idx.shape
        xp, counts, offsets, rmap, src = orig(x[::-1], idx[::-1], E, C)
        rmap = rmap[::-1].copy()
        src = np.where(src >= 0, T - 1 - src, -1)
        return x[np.maximum(src, 0)] * (src >= 0)[:, None], counts, offsets, rmap, src
    return permute_capacity


def _dropped_pairs_combine(O):
    orig = O.combine

    def combine(yp, rmap, gate, y_shared=None, acc=np.float64):
        # a dropped pair (-1) is read as the last row
        return orig(yp, np.where(rmap < 0, yp.shape[0] - 1, rmap), gate, y_shared, acc)
    return combine


MUTANTS = {
    "renormalised_gates": ("route", _renormalised_gates),
    "ties_to_higher_index": ("route", _ties_to_higher_index),
    "unstable_permute": ("permute", _unstable_permute),
    "swapped_gate_up": ("expert_forward", _swapped_gate_up),
    "silu_sign": ("silu", _silu_sign),
    "combine_without_gate": ("combine", _combine_without_gate),
    "route_bwd_sign": ("route_backward", _route_bwd_sign),
    "silu_grad_missing_term": ("expert_backward", _silu_grad_missing_term),
    "dropped_shared": ("layer_forward", _dropped_shared),
    "sample_std_cv": ("load_stats", _sample_std_cv),
    "strided_groups": ("load_stats", _strided_groups),
    "drop_last_pairs": ("permute_capacity", _drop_last_pairs),
    "dropped_pairs_combine": ("combine", _dropped_pairs_combine),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    fn_name, make = MUTANTS[name]
    O = _fresh_oracle()
    setattr(O, fn_name, make(O))
    failed = []
    for check in ALL_CHECKS:
        try:
            check(O)
        except Exception:               # an assertion or a crash both count as caught
            failed.append(check.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
