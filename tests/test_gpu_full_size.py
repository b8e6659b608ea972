"""Full-size parity of the DeepSeek-shaped layer and the small-expert stress
layer, GPU only, in the launch configuration the benchmark uses (two streams,
dynamic tile scheduler).

At these sizes the CPU oracle cannot run the whole layer in a test's time, so
the parts it can afford are checked in full and the rest on samples it
computes one by one:
  - in full: router logits (DeepSeek), route indices and gates, counts,
    offsets, row map and source tokens, route backward and router backward
    given the GPU's own upstream values;
  - sampled rows of the largest, the smallest and two random non-empty
    expert groups: the permuted copy, h13, act and yp (the oracle's expert on
    those rows), dyp, dh13 and dxp (its backward on those rows);
  - sampled tokens: y, dgate and dx (every row of the token through the
    oracle's expert, the oracle's combine, route and router backward);
  - whole weight gradients of the smallest non-empty group and of a group of
    about a hundred rows (every row of the group), and exact zeros for every
    empty group (DeepSeek's Zipf(1.2) skew leaves two at seed 0).
Tolerances as in the other layer tests: max|gpu - ref| <= 2e-2 max|ref| over
each checked tensor (bf16 storage), 1e-5 for gates and fp32 gradients.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import have_gpu, host, make_layer, rel_err

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

TOL = 2e-2


def log(*a):
    print("[full-size]", *a, flush=True)


def pick(t, rows):
    return host(t[torch.as_tensor(np.asarray(rows), dtype=torch.long, device=t.device)])


def group_of(offsets, rows):
    return np.searchsorted(offsets, rows, side="right") - 1


@pytest.mark.parametrize("name", ["deepseek", "stress"])
def test_layer_full_size_sampled(name):
    cfg = synth.get_config(name)
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    assert cfg.g0 == 0 and cfg.groups == E and not cfg.shared
    log(f"config={name} T={T} H={H} I={I} E={E} k={k}: drawing inputs")
    inp = synth.make_inputs(cfg, threads=16)
    L = make_layer(cfg, inp)
    log("inputs on the device; layer step")
    L.set_gemm_dynamic(True)
    L.forward()
    L.backward()
    torch.cuda.synchronize()
    acc = np.float32
    rep = {}

    # ---- routing, in full
    lg = host(L.logits)
    if cfg.router:
        ref_logits = oracle.router_logits(inp.x, inp.wg, inp.bias)
        rep["logits"] = rel_err(lg, ref_logits)
        assert rep["logits"] <= 1e-5
    idx, gate = oracle.route(lg, k)
    assert np.array_equal(host(L.idx), idx)
    assert rel_err(host(L.gate), gate) <= 1e-5
    # the maps do not depend on the rows, so a one-column stand-in for x
    _, counts, offsets, rmap, src = oracle.permute(np.zeros((T, 1), np.float32), idx, E)
    assert np.array_equal(host(L.counts), counts)
    assert np.array_equal(host(L.offsets), offsets)
    assert np.array_equal(host(L.row_id_map), rmap)
    assert np.array_equal(host(L.src_token), src)
    log("routing and maps bit-exact; counts min", counts.min(), "max", counts.max(),
        "empty", int((counts == 0).sum()))

    rng = np.random.default_rng(7)
    nonempty = np.flatnonzero(counts > 0)
    groups = {int(nonempty[np.argmax(counts[nonempty])]), int(nonempty[np.argmin(counts[nonempty])])}
    groups |= {int(g) for g in rng.choice(nonempty, 2, replace=False)}
    w13 = lambda e: inp.w13[e - cfg.g0]
    w2 = lambda e: inp.w2[e - cfg.g0]

    # ---- sampled rows of a few groups: forward and dX through the oracle's expert
    for e in sorted(groups):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        rows = np.unique(np.concatenate([[lo, hi - 1], rng.integers(lo, hi, 6)]))
        xr = inp.x[src[rows]]
        assert np.array_equal(pick(L.xp, rows), xr)                 # bit copy
        h13, act, yp = oracle.expert_forward(xr, w13(e), w2(e), acc=acc)
        # dyp of these rows: gate * dy of their token (the combine's backward)
        dyr, _ = oracle.combine_backward(inp.dy[src[rows]], np.zeros((len(rows), H), acc),
                                         np.arange(len(rows))[:, None],
                                         gate[src[rows], np.argmax(rmap[src[rows]] == rows[:, None],
                                                                   axis=1)][:, None], acc=acc)
        dh13, dxr, _, _ = oracle.expert_backward(xr, w13(e), w2(e), dyr, acc=acc)
        for n, g, r in (("h13", L.h13, h13), ("act", L.act, act), ("yp", L.yp, yp),
                        ("dyp", L.dyp, dyr), ("dh13", L.dh13, dh13), ("dxp", L.dxp, dxr)):
            v = rel_err(pick(g, rows), r)
            rep[f"{n}[{e}]"] = v
            assert v <= TOL, (n, e, v)
    log("sampled rows of groups", sorted(groups), "match")

    # ---- sampled tokens: y, dgate, dx
    top = int(nonempty[np.argmax(counts[nonempty])])
    toks = np.unique(np.concatenate([src[[offsets[top], offsets[top + 1] - 1]],
                                     rng.integers(0, T, 10)]))
    rows = rmap[toks].ravel()
    yp_sub = np.zeros((rows.size, H), acc)
    dxp_sub = np.zeros((rows.size, H), acc)
    ge = group_of(offsets, rows)
    gsub = gate[toks]
    dy_tok = inp.dy[toks]
    # every row of the sampled tokens through its expert (forward)
    for e in np.unique(ge):
        m = ge == e
        _, _, yp_sub[m] = oracle.expert_forward(inp.x[src[rows[m]]], w13(e), w2(e), acc=acc)
    rmap_sub = np.arange(rows.size).reshape(len(toks), k)
    y_ref = oracle.combine(yp_sub, rmap_sub, gsub, None, acc=acc)
    dyp_sub, dgate_ref = oracle.combine_backward(dy_tok, yp_sub, rmap_sub, gsub, acc=acc)
    for e in np.unique(ge):
        m = ge == e
        _, dxp_sub[m], _, _ = oracle.expert_backward(inp.x[src[rows[m]]], w13(e), w2(e),
                                                     dyp_sub[m], acc=acc)
    dx_ref = oracle.permute_backward(dxp_sub, rmap_sub, acc=acc)
    if cfg.router:
        dl_tok = oracle.route_backward(lg[toks], idx[toks], dgate_ref, acc=np.float64)
        dx_ref = dx_ref + oracle.router_backward(dl_tok, inp.x[toks], inp.wg)[0]
    rep["y(tokens)"] = rel_err(pick(L.y, toks), y_ref)
    rep["dgate(tokens)"] = rel_err(pick(L.dgate, toks), dgate_ref)
    rep["dx(tokens)"] = rel_err(pick(L.dx, toks), dx_ref)
    assert rep["y(tokens)"] <= TOL and rep["dx(tokens)"] <= TOL
    # dgate is an fp32 dot of stored values: the GPU's yp is bf16, the oracle's is not
    assert rep["dgate(tokens)"] <= TOL
    log("sampled tokens", toks.size, "match")

    # ---- route and router backward in full, given the GPU's own dgate / dlogits
    dgate_gpu = host(L.dgate)
    dl_ref = oracle.route_backward(lg, idx, dgate_gpu)
    rep["dlogits"] = rel_err(host(L.dlogits), dl_ref)
    assert rep["dlogits"] <= 1e-5
    if cfg.router:
        _, dwg_ref, db_ref = oracle.router_backward(host(L.dlogits), inp.x, inp.wg)
        rep["dwg"] = rel_err(host(L.dwg), dwg_ref)
        rep["dbias"] = rel_err(host(L.dbias), db_ref)
        assert rep["dwg"] <= 1e-5 and rep["dbias"] <= 1e-5

    # ---- whole weight gradients of the smallest, a ~100-row and the largest
    # group; empty groups exactly zero
    small = int(nonempty[np.argmin(counts[nonempty])])
    mid = int(nonempty[np.argmin(np.abs(counts[nonempty] - 100))])
    large = int(nonempty[np.argmax(counts[nonempty])])
    for e in sorted({small, mid, large}):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        r = np.arange(lo, hi)
        t_of = src[r]
        j_of = np.argmax(rmap[t_of] == r[:, None], axis=1)
        dyr, _ = oracle.combine_backward(inp.dy[t_of], np.zeros((r.size, H), acc),
                                         np.arange(r.size)[:, None], gate[t_of, j_of][:, None],
                                         acc=acc)
        _, _, dw13, dw2 = oracle.expert_backward(inp.x[t_of], w13(e), w2(e), dyr, acc=acc)
        rep[f"dw13[{e}]"] = rel_err(host(L.dw13[e - cfg.g0]), dw13)
        rep[f"dw2[{e}]"] = rel_err(host(L.dw2[e - cfg.g0]), dw2)
        assert rep[f"dw13[{e}]"] <= TOL and rep[f"dw2[{e}]"] <= TOL, e
    for e in np.flatnonzero(counts == 0):
        assert int(torch.count_nonzero(L.dw13[e - cfg.g0])) == 0
        assert int(torch.count_nonzero(L.dw2[e - cfg.g0])) == 0
    log(name, {n: f"{v:.2e}" for n, v in rep.items()})
