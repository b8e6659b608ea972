"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each ``check_*`` takes the oracle module (or a planted-mistake copy of it) and
raises AssertionError when the oracle disagrees with a brute-force result, a
closed form, an invariant, a library routine or a finite difference.
``test_oracle_pins.py`` runs them on the oracle (all must pass);
``test_oracle_mutants.py`` runs them on copies with one planted mistake each
(at least one must fail), which shows that the pins can see such mistakes.
"""
from __future__ import annotations

import math

import numpy as np


def _rng(i):
    return np.random.default_rng(1000 + i)


# ----------------------------------------------------------------- routing


def check_route_bruteforce(O):
    """Top-k indices equal a per-token Python sort by (-logit, expert) on
    inputs with many exact ties (logits on a coarse grid)."""
    r = _rng(0)
    for E, k in [(1, 1), (2, 1), (5, 3), (8, 2), (8, 8), (33, 7)]:
        logits = (r.integers(-4, 5, size=(64, E)) * 0.25).astype(np.float32)
        idx, gate = O.route(logits, k)
        assert idx.shape == (64, k) and gate.shape == (64, k)
        for t in range(64):
            ref = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
            assert list(idx[t]) == ref, (E, k, t, list(idx[t]), ref)


def check_route_hand_example(O):
    """Probabilities 1:2:3:2 (logits ln1, ln2, ln3, ln2), k = 3: the order is
    expert 2, then the tie 1 vs 3 goes to 1, then 3; gates are the full
    softmax values 3/8, 2/8, 2/8 (not renormalised over the top-k)."""
    logits = np.log(np.array([[1.0, 2.0, 3.0, 2.0]])).astype(np.float32)
    # ln2 rounded to fp32 is the same number in both slots, so the tie is exact
    idx, gate = O.route(logits, 3)
    assert list(idx[0]) == [2, 1, 3], idx
    l = logits[0].astype(np.float64)
    z = np.exp(l - l.max())
    ref = [z[2] / z.sum(), z[1] / z.sum(), z[3] / z.sum()]
    assert np.allclose(gate[0], ref, rtol=1e-12, atol=0)
    assert np.allclose(gate[0], [3 / 8, 2 / 8, 2 / 8], rtol=1e-6, atol=0)


def check_gate_closed_forms(O):
    r = _rng(1)
    # k = E: the gates are the whole distribution
    logits = r.standard_normal((32, 9)).astype(np.float32) * 3
    _, gate = O.route(logits, 9)
    assert np.allclose(gate.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    # E = 2, k = 1: the chosen gate is the logistic function of the gap
    logits = r.standard_normal((32, 2)).astype(np.float32) * 3
    idx, gate = O.route(logits, 1)
    gap = np.abs(logits[:, 0].astype(np.float64) - logits[:, 1])
    assert np.allclose(gate[:, 0], 1.0 / (1.0 + np.exp(-gap)), rtol=1e-12, atol=0)
    assert np.array_equal(idx[:, 0], np.where(logits[:, 1] > logits[:, 0], 1, 0))
    # E = 1: a single expert with gate 1
    idx, gate = O.route(r.standard_normal((5, 1)).astype(np.float32), 1)
    assert np.all(idx == 0) and np.all(gate == 1.0)


def _separated_logits(r, T, E, k, gap=0.05):
    """Logits whose k-th and (k+1)-th values differ by more than ``gap``."""
    while True:
        l = r.standard_normal((T, E)).astype(np.float64) * 2
        s = -np.sort(-l, axis=1)
        if E == k or np.all(s[:, k - 1] - s[:, k] > gap):
            return l.astype(np.float32)


def check_route_backward_fd(O):
    """dlogits sums to zero per token and matches central finite differences
    of L(l) = sum_tj w[t,j] gate[t,j](l) with the selection held fixed."""
    r = _rng(2)
    T, E, k = 6, 7, 3
    l32 = _separated_logits(r, T, E, k)
    w = r.standard_normal((T, k))
    idx, _ = O.route(l32, k)
    dl = O.route_backward(l32, idx, w)
    assert np.allclose(dl.sum(axis=1), 0.0, atol=1e-12)
    l = l32.astype(np.float64)
    eps = 1e-6
    for t in range(T):
        for e in range(E):
            def L(delta):
                m = l.copy()
                m[t, e] += delta
                p = np.exp(m - m.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                return float((np.take_along_axis(p, idx.astype(np.int64), 1) * w).sum())
            fd = (L(eps) - L(-eps)) / (2 * eps)
            assert abs(fd - dl[t, e]) < 1e-7, (t, e, fd, dl[t, e])


# ----------------------------------------------------------------- permute


def check_permute_invariants(O):
    r = _rng(3)
    for T, E, k in [(50, 8, 2), (97, 16, 5), (40, 3, 3), (1, 4, 2)]:
        x = r.standard_normal((T, 6)).astype(np.float32)
        bias = np.where(np.arange(E) == 0, 4.0, 0.0)     # skew: expert 0 hot
        logits = (r.standard_normal((T, E)) + bias).astype(np.float32)
        idx, _ = O.route(logits, k)
        xp, counts, offsets, rmap, src = O.permute(x, idx, E)
        R = T * k
        assert counts.sum() == R and offsets[0] == 0 and offsets[E] == R
        assert np.all(np.diff(offsets) == counts) and np.all(counts >= 0)
        assert np.array_equal(np.sort(rmap.ravel()), np.arange(R))        # bijection
        for t in range(T):
            for j in range(k):
                row = rmap[t, j]
                e = idx[t, j]
                assert offsets[e] <= row < offsets[e + 1]
                assert src[row] == t
                assert xp[row].tobytes() == x[t].tobytes()
        for e in range(E):                                           # token order in a group
            s = src[offsets[e]:offsets[e + 1]]
            assert np.all(np.diff(s) > 0)
        # a library stable sort of the flattened expert ids gives the same rows
        order = np.argsort(idx.ravel(), kind="stable")
        assert np.array_equal(src, order // k)
        assert np.array_equal(np.bincount(idx.ravel(), minlength=E), counts)


def check_identity_experts(O):
    """With identity experts (yp = xp) the combine returns (sum_j gate) x; with
    all gates 1 it returns k x; and the permute adjoint of a permuted copy of
    dx returns k dx."""
    r = _rng(4)
    T, E, k, H = 40, 6, 3, 5
    x = r.standard_normal((T, H))
    idx, gate = O.route(r.standard_normal((T, E)).astype(np.float32), k)
    xp, counts, offsets, rmap, src = O.permute(x, idx, E)
    y = O.combine(xp, rmap, gate)
    assert np.allclose(y, gate.sum(axis=1)[:, None] * x, rtol=1e-12, atol=1e-12)
    y1 = O.combine(xp, rmap, np.ones_like(gate))
    assert np.allclose(y1, k * x, rtol=1e-12, atol=1e-12)
    ys = r.standard_normal((T, H))
    y2 = O.combine(xp, rmap, gate, ys)
    assert np.allclose(y2, ys + gate.sum(axis=1)[:, None] * x, rtol=1e-12, atol=1e-12)
    dx = O.permute_backward(xp, rmap)
    assert np.allclose(dx, k * x, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------- experts


def _silu(z):
    return z / (1.0 + math.exp(-z))


def check_expert_forward_bruteforce(O):
    """Scalar triple loops of the SwiGLU FFN (gate rows first, then up rows)."""
    r = _rng(5)
    n, H, I = 3, 5, 4
    xr = r.standard_normal((n, H))
    w13 = r.standard_normal((2 * I, H)) * 0.5
    w2 = r.standard_normal((H, I)) * 0.5
    h13, act, y = O.expert_forward(xr, w13, w2)
    for t in range(n):
        a = []
        for i in range(I):
            g = sum(xr[t, h] * w13[i, h] for h in range(H))
            u = sum(xr[t, h] * w13[I + i, h] for h in range(H))
            assert abs(h13[t, i] - g) < 1e-12 and abs(h13[t, I + i] - u) < 1e-12
            a.append(_silu(g) * u)
            assert abs(act[t, i] - a[-1]) < 1e-12
        for h in range(H):
            assert abs(y[t, h] - sum(a[i] * w2[h, i] for i in range(I))) < 1e-12


def check_dense_special_case(O):
    """E = 1, k = 1: every token goes to the one expert with gate 1, so the
    layer is a dense SwiGLU FFN (checked against torch's silu and matmul)."""
    import torch
    r = _rng(6)
    T, H, I = 17, 8, 6
    x = r.standard_normal((T, H))
    w13 = r.standard_normal((1, 2 * I, H)) * 0.3
    w2 = r.standard_normal((1, H, I)) * 0.3
    wg = r.standard_normal((H, 1)).astype(np.float32)
    out = O.layer_forward(x, 1, 1, w13, w2, wg=wg)
    xt = torch.from_numpy(x)
    g = xt @ torch.from_numpy(w13[0, :I]).T
    u = xt @ torch.from_numpy(w13[0, I:]).T
    ref = (torch.nn.functional.silu(g) * u) @ torch.from_numpy(w2[0]).T
    assert np.allclose(out["y"], ref.numpy(), rtol=1e-12, atol=1e-12)
    assert np.all(out["gate"] == 1.0) and np.all(out["idx"] == 0)


def check_grouped_matches_per_group(O):
    """Grouped forward equals the expert FFN applied to each group's slice;
    an empty group touches no rows and gets exactly zero weight gradients."""
    r = _rng(7)
    H, I = 6, 4
    counts = [3, 0, 5, 1]
    offsets = np.concatenate([[0], np.cumsum(counts)])
    R = offsets[-1]
    xp = r.standard_normal((R, H))
    w13 = r.standard_normal((4, 2 * I, H))
    w2 = r.standard_normal((4, H, I))
    h13, act, yp = O.grouped_forward(xp, offsets, w13, w2)
    for g in range(4):
        lo, hi = offsets[g], offsets[g + 1]
        if hi > lo:
            ref = xp[lo:hi] @ w13[g, :I].T
            assert np.allclose(h13[lo:hi, :I], ref, rtol=1e-12, atol=1e-12)
    dyp = r.standard_normal((R, H))
    dh13, dxp, dw13, dw2 = O.grouped_backward(xp, dyp, offsets, w13, w2)
    assert np.all(dw13[1] == 0) and np.all(dw2[1] == 0)
    # dW2[g] = dY_g^T act_g (a plain matmul identity)
    for g in (0, 2, 3):
        lo, hi = offsets[g], offsets[g + 1]
        assert np.allclose(dw2[g], dyp[lo:hi].T @ act[lo:hi], rtol=1e-12, atol=1e-12)


def check_expert_backward_fd(O):
    """Central finite differences of L = <dy, y(x, W13, W2)> for one expert."""
    r = _rng(8)
    n, H, I = 4, 5, 3
    xr = r.standard_normal((n, H))
    w13 = r.standard_normal((2 * I, H)) * 0.7
    w2 = r.standard_normal((H, I)) * 0.7
    dyr = r.standard_normal((n, H))
    dh13, dx, dw13, dw2 = O.expert_backward(xr, w13, w2, dyr)
    eps = 1e-6

    def L(a, b, c):
        I_ = c.shape[1]
        g = a @ b[:I_].T
        u = a @ b[I_:].T
        s = 1.0 / (1.0 + np.exp(-g))
        return float(((g * s * u) @ c.T * dyr).sum())

    for arr, grad, name in [(xr, dx, "x"), (w13, dw13, "w13"), (w2, dw2, "w2")]:
        for pos in np.ndindex(arr.shape):
            a = arr.copy()
            a[pos] += eps
            hi = L(*(a if nm == name else v for nm, v in (("x", xr), ("w13", w13), ("w2", w2))))
            a[pos] -= 2 * eps
            lo = L(*(a if nm == name else v for nm, v in (("x", xr), ("w13", w13), ("w2", w2))))
            fd = (hi - lo) / (2 * eps)
            assert abs(fd - grad[pos]) < 1e-6 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])


def check_remote_window(O):
    """Running only the window [g0, g0+G) equals the full run on its rows;
    other rows get zero expert output and zero input gradient."""
    r = _rng(9)
    T, H, I, E, k = 30, 6, 4, 6, 2
    x = r.standard_normal((T, H))
    w13 = r.standard_normal((E, 2 * I, H)) * 0.3
    w2 = r.standard_normal((E, H, I)) * 0.3
    idx, gate = O.route(r.standard_normal((T, E)).astype(np.float32), k)
    xp, counts, offsets, rmap, src = O.permute(x, idx, E)
    _, _, yp_all = O.grouped_forward(xp, offsets, w13, w2)
    g0, G = 2, 3
    _, _, yp = O.grouped_forward(xp, offsets, w13[g0:g0 + G], w2[g0:g0 + G], g0, G)
    lo, hi = offsets[g0], offsets[g0 + G]
    assert np.allclose(yp[lo:hi], yp_all[lo:hi], rtol=1e-12, atol=1e-12)
    assert np.all(yp[:lo] == 0) and np.all(yp[hi:] == 0)
    dyp = r.standard_normal(xp.shape)
    _, dxp, dw13, _ = O.grouped_backward(xp, dyp, offsets, w13[g0:g0 + G], w2[g0:g0 + G], g0, G)
    _, dxp_all, dw13_all, _ = O.grouped_backward(xp, dyp, offsets, w13, w2)
    assert np.all(dxp[:lo] == 0) and np.all(dxp[hi:] == 0)
    assert np.allclose(dxp[lo:hi], dxp_all[lo:hi], rtol=1e-12, atol=1e-12)
    assert np.allclose(dw13, dw13_all[g0:g0 + G], rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------- whole layer


def _torch_layer(x, wg, bias, w13, w2, k, ws13=None, ws2=None):
    """An independent dense-mask formulation of the layer with torch autograd."""
    import torch
    tt = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    X, WG, B, W13, W2 = tt(x), tt(wg), tt(bias), tt(w13), tt(w2)
    E, I2, H = W13.shape
    I = I2 // 2
    logits = X @ WG + B
    p = torch.softmax(logits, dim=-1)
    top = torch.topk(logits.detach(), k, dim=-1).indices
    mask = torch.zeros_like(p).scatter(1, top, 1.0)
    w = p * mask                                       # [T,E] gate of chosen experts, 0 elsewhere
    y = torch.zeros_like(X)
    for e in range(E):
        h = X @ W13[e].T
        y = y + w[:, e:e + 1] * ((torch.nn.functional.silu(h[:, :I]) * h[:, I:]) @ W2[e].T)
    extra = []
    if ws13 is not None:
        S13, S2 = tt(ws13), tt(ws2)
        hs = X @ S13.T
        y = y + (torch.nn.functional.silu(hs[:, :I]) * hs[:, I:]) @ S2.T
        extra = [S13, S2]
    return y, [X, WG, B, W13, W2] + extra


def check_layer_vs_torch_autograd(O):
    import torch
    r = _rng(10)
    T, H, I, E, k = 24, 8, 6, 5, 2
    x = r.standard_normal((T, H))
    wg = (r.standard_normal((H, E)) * 0.5).astype(np.float32)
    bias = (r.standard_normal(E) * 0.5).astype(np.float32)
    w13 = r.standard_normal((E, 2 * I, H)) * 0.3
    w2 = r.standard_normal((E, H, I)) * 0.3
    ws13 = r.standard_normal((2 * I, H)) * 0.3
    ws2 = r.standard_normal((H, I)) * 0.3
    dy = r.standard_normal((T, H))
    fwd = O.layer_forward(x, k, E, w13, w2, wg=wg, bias=bias, ws13=ws13, ws2=ws2)
    bwd = O.layer_backward(fwd, dy, x, w13, w2, wg=wg, ws13=ws13, ws2=ws2)
    # the torch model takes fp64 logits; the oracle rounds logits to fp32, so
    # compare at a tolerance that covers that rounding
    y, params = _torch_layer(x, wg, bias, w13, w2, k, ws13, ws2)
    (y * torch.from_numpy(dy)).sum().backward()
    tol = dict(rtol=1e-5, atol=1e-5)
    assert np.allclose(fwd["y"], y.detach().numpy(), **tol)
    names = ["dx", "dwg", "dbias", "dw13", "dw2", "dws13", "dws2"]
    for n, prm in zip(names, params):
        assert np.allclose(bwd[n], prm.grad.numpy(), **tol), n


def check_layer_fd(O):
    """Finite-difference gradcheck of the whole layer in fp64 with the
    routing held fixed (the perturbation never changes the selection)."""
    r = _rng(11)
    T, H, I, E, k = 10, 6, 4, 4, 2
    x = r.standard_normal((T, H))
    wg = (r.standard_normal((H, E)) * 0.5).astype(np.float32)
    w13 = r.standard_normal((E, 2 * I, H)) * 0.3
    w2 = r.standard_normal((E, H, I)) * 0.3
    dy = r.standard_normal((T, H))
    fwd = O.layer_forward(x, k, E, w13, w2, wg=wg)
    bwd = O.layer_backward(fwd, dy, x, w13, w2, wg=wg)
    idx0 = fwd["idx"]

    def L(xx, ww13):
        # fp64 logits so that the finite difference sees the exact function
        f = O.layer_forward(xx, k, E, ww13, w2, logits=(xx @ wg.astype(np.float64)))
        assert np.array_equal(f["idx"], idx0)
        return float((f["y"] * dy).sum())

    eps = 1e-6
    for pos in [(0, 0), (3, 2), (9, 5), (5, 1)]:
        a = x.copy(); a[pos] += eps; hi = L(a, w13)
        a[pos] -= 2 * eps; lo = L(a, w13)
        fd = (hi - lo) / (2 * eps)
        assert abs(fd - bwd["dx"][pos]) < 1e-5 * max(1, abs(fd)), (pos, fd, bwd["dx"][pos])
    for pos in [(0, 0, 0), (1, 5, 2), (3, 7, 5)]:
        a = w13.copy(); a[pos] += eps; hi = L(x, a)
        a[pos] -= 2 * eps; lo = L(x, a)
        fd = (hi - lo) / (2 * eps)
        assert abs(fd - bwd["dw13"][pos]) < 1e-5 * max(1, abs(fd)), (pos, fd, bwd["dw13"][pos])


def check_load_stats_closed_forms(O):
    """cv closed forms: equal loads 0; one expert holding every row sqrt(E-1);
    counts (1, 3) give 0.5 (population std 1 over mean 2, not the sample
    std's 0.707); group sums; loads sum to 1; no rows gives zeros."""
    load, cv, g, gcv = O.load_stats(np.full(8, 5), 2)
    assert cv == 0.0 and gcv == 0.0 and np.allclose(load, 1 / 8) and list(g) == [10] * 4
    for E in (2, 8, 256):
        c = np.zeros(E, np.int64)
        c[E // 3] = 1000
        _, cv, _, _ = O.load_stats(c)
        assert abs(cv - np.sqrt(E - 1)) < 1e-12 * np.sqrt(E)
    load, cv, g, gcv = O.load_stats(np.array([1, 3]), 1)
    assert abs(cv - 0.5) < 1e-15 and np.allclose(load, [0.25, 0.75]) and list(g) == [1, 3]
    load, cv, g, gcv = O.load_stats(np.array([1, 3, 2, 2]), 2)
    assert list(g) == [4, 4] and gcv == 0.0 and abs(cv - np.sqrt(0.5) / 2) < 1e-15
    r = np.random.default_rng(5)
    c = r.integers(0, 100, 64)
    load, cv, g, gcv = O.load_stats(c, 8)
    assert abs(load.sum() - 1) < 1e-12 and int(g.sum()) == int(c.sum())
    assert abs(cv - np.std(c) / np.mean(c)) < 1e-12
    load, cv, g, gcv = O.load_stats(np.zeros(4, np.int64), 4)
    assert cv == 0.0 and gcv == 0.0 and not load.any() and list(g) == [0]


def check_capacity_bruteforce(O):
    """Drop-and-pad permute against a direct listing: expert e's pairs in
    (token, slot) order, the first C keep rows e*C.., the rest are dropped;
    pad rows are zero with source -1; kept + dropped = T*k."""
    r = np.random.default_rng(41)
    T, k, E, C, H = 13, 2, 4, 3, 5
    logits = r.standard_normal((T, E)).astype(np.float32)
    logits[:, 1] += 1.5                                       # expert 1 overflows
    idx, _ = O.route(logits, k)
    x = r.standard_normal((T, H))
    xp, counts, offsets, rmap, src = O.permute_capacity(x, idx, E, C)
    assert list(offsets) == [0, 3, 6, 9, 12] and xp.shape == (E * C, H)
    kept = 0
    for e in range(E):
        pairs = [(t, j) for t in range(T) for j in range(k) if idx[t, j] == e]
        assert counts[e] == len(pairs)
        for n, (t, j) in enumerate(pairs):
            if n < C:
                assert rmap[t, j] == e * C + n and src[e * C + n] == t
                assert np.array_equal(xp[e * C + n], x[t])
                kept += 1
            else:
                assert rmap[t, j] == -1
        for n in range(len(pairs), C):
            assert src[e * C + n] == -1 and not xp[e * C + n].any()
    assert kept + int((rmap < 0).sum()) == T * k and kept == int((src >= 0).sum())
    assert max(counts) > C                                     # something was dropped
    assert O.capacity(8192, 8, 256, 1.2) == 308 and O.capacity(8192, 8, 256, 1.0) == 256
    # hand example: three tokens, one expert, one row -> only token 0 is served
    _, c1, _, m1, s1 = O.permute_capacity(np.eye(3), np.zeros((3, 1), np.int64), 1, 1)
    assert list(m1[:, 0]) == [0, -1, -1] and list(s1) == [0] and c1[0] == 3


def _small_layer(r, T=24, H=8, I=4, E=4, k=2, shared=True):
    x = r.standard_normal((T, H))
    w13 = r.standard_normal((E, 2 * I, H)) * 0.3
    w2 = r.standard_normal((E, H, I)) * 0.3
    logits = r.standard_normal((T, E)).astype(np.float32)
    ws13 = r.standard_normal((2 * I, H)) * 0.3 if shared else None
    ws2 = r.standard_normal((H, I)) * 0.3 if shared else None
    return x, w13, w2, logits, ws13, ws2


def check_capacity_limits(O):
    """A capacity of at least every count reduces to dropless (same outputs and
    gradients); capacity 0 drops every pair (output = shared expert only, no
    routed gradient, dgate 0)."""
    r = np.random.default_rng(43)
    T, k, E = 24, 2, 4
    x, w13, w2, logits, ws13, ws2 = _small_layer(r, T=T, k=k, E=E)
    dy = r.standard_normal(x.shape)
    ref = O.layer_forward(x, k, E, w13, w2, logits=logits, ws13=ws13, ws2=ws2)
    bref = O.layer_backward(ref, dy, x, w13, w2, ws13=ws13, ws2=ws2)
    big = O.layer_forward(x, k, E, w13, w2, logits=logits, ws13=ws13, ws2=ws2, C=T)
    bbig = O.layer_backward(big, dy, x, w13, w2, ws13=ws13, ws2=ws2)
    assert np.allclose(big["y"], ref["y"], rtol=0, atol=1e-12)
    for n in ("dx", "dw13", "dw2", "dgate", "dlogits"):
        assert np.allclose(bbig[n], bref[n], rtol=0, atol=1e-12), n
    # a capacity that drops some pairs: each token's output is the shared
    # expert plus its served pairs only, each expert run on the token alone
    mid = O.layer_forward(x, k, E, w13, w2, logits=logits, ws13=ws13, ws2=ws2, C=3)
    rm, idx, gate = mid["row_id_map"], mid["idx"], mid["gate"]
    assert (rm < 0).any() and (rm >= 0).any()
    ys = O.expert_forward(x, ws13, ws2)[2]
    for t in range(T):
        want = ys[t].copy()
        for j in range(k):
            if rm[t, j] >= 0:
                e = idx[t, j]
                want += gate[t, j] * O.expert_forward(x[t:t + 1], w13[e], w2[e])[2][0]
        assert np.allclose(mid["y"][t], want, rtol=0, atol=1e-12)
    zero = O.layer_forward(x, k, E, w13, w2, logits=logits, ws13=ws13, ws2=ws2, C=0)
    bz = O.layer_backward(zero, dy, x, w13, w2, ws13=ws13, ws2=ws2)
    assert np.allclose(zero["y"], O.expert_forward(x, ws13, ws2)[2], rtol=0, atol=1e-12)
    assert not bz["dgate"].any() and not bz["dw13"].any() and not bz["dw2"].any()
    assert np.allclose(bz["dx"], O.expert_backward(x, ws13, ws2, dy)[1], rtol=0, atol=1e-12)


ALL_CHECKS = [
    check_load_stats_closed_forms, check_capacity_bruteforce, check_capacity_limits,
    check_route_bruteforce, check_route_hand_example, check_gate_closed_forms,
    check_route_backward_fd, check_permute_invariants, check_identity_experts,
    check_expert_forward_bruteforce, check_dense_special_case, check_grouped_matches_per_group,
    check_expert_backward_fd, check_remote_window, check_layer_vs_torch_autograd, check_layer_fd,
]
