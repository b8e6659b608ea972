"""The drop-and-pad variant on the GPU against the oracle (GPU only).

Maps, counts, offsets and the padded row copy are compared bit for bit with
oracle.permute_capacity; the row kernels with dropped pairs and the whole
layer to the usual tolerance (2e-2 max|ref| for bf16, 1e-5 for fp32).  A
capacity that holds every expert's pairs must give the dropless layer's
results bit for bit (the same products, padded rows add exact zeros).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import dev, have_gpu, host, make_layer, rel_err

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

TOL = {"f32": 1e-5, "bf16": 2e-2}


@pytest.fixture(scope="module")
def abi():
    from routing_permute_grouped_moe_amd import abi as a
    return a


def _tdt(dt):
    return torch.bfloat16 if dt == "bf16" else torch.float32


def _store(a, dt):
    return synth.bf16_round(np.asarray(a, np.float32)) if dt == "bf16" else \
        np.asarray(a, np.float32)


def _route(abi, logits, k):
    T, E = logits.shape
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    gate = torch.empty(T, k, dtype=torch.float32, device="cuda")
    if T:
        abi.moe_route(dev(logits, torch.float32), T, E, k, idx, gate)
    return idx, gate


def _permute_cap(abi, x, dt, idx, T, H, E, k, C, with_xp=True):
    tdt = _tdt(dt)
    code = abi.MOE_BF16 if dt == "bf16" else abi.MOE_F32
    R = E * C
    xp = torch.full((R, H), 7.0, dtype=tdt, device="cuda") if with_xp else None
    counts = torch.full((E,), -5, dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), -5, dtype=torch.int32, device="cuda")
    rmap = torch.full((T, k), -5, dtype=torch.int32, device="cuda")
    src = torch.full((R,), -5, dtype=torch.int32, device="cuda")
    wsb = abi.moe_permute_workspace_bytes(T, E, k)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    abi.moe_permute_capacity(dev(x, tdt) if T else None, code, idx, T, H, E, k, C, xp, counts,
                             offsets, rmap, src, ws, wsb)
    torch.cuda.synchronize()
    return xp, counts, offsets, rmap, src


PERM_CASES = [  # T, E, k, C, skew, dt
    (300, 8, 2, 50, 2.0, "bf16"), (300, 8, 2, 75, 0.0, "f32"), (257, 64, 6, 30, 1.5, "bf16"),
    (1000, 256, 8, 1, 3.0, "bf16"), (64, 4, 2, 0, 0.0, "bf16"), (40, 4, 4, 64, 0.0, "bf16"),
    (0, 16, 2, 5, 0.0, "bf16")]


@pytest.mark.parametrize("T,E,k,C,skew,dt", PERM_CASES)
def test_permute_capacity_bit_exact(abi, T, E, k, C, skew, dt):
    print(f"case T={T} E={E} k={k} C={C} skew={skew} {dt}", flush=True)
    H = 128
    r = np.random.default_rng(T + E + k + C)
    logits = (r.standard_normal((T, E)) - skew * np.log1p(np.arange(E))).astype(np.float32)
    x = _store(r.standard_normal((T, H)), dt)
    idx, _ = _route(abi, logits, k)
    ridx = oracle.route(logits, k)[0] if T else np.zeros((0, k), np.int64)
    assert np.array_equal(host(idx), ridx)
    xp, counts, offsets, rmap, src = _permute_cap(abi, x, dt, idx, T, H, E, k, C)
    rxp, rc, ro, rm, rs = oracle.permute_capacity(x, ridx, E, C)
    assert np.array_equal(host(counts), rc) and np.array_equal(host(offsets), ro)
    assert np.array_equal(host(rmap), rm) and np.array_equal(host(src), rs)
    assert np.array_equal(host(xp).astype(np.float32), rxp.astype(np.float32))
    # maps only (no row copy) gives the same maps
    _, c2, o2, m2, s2 = _permute_cap(abi, x, dt, idx, T, H, E, k, C, with_xp=False)
    for a_, b_ in [(c2, counts), (o2, offsets), (m2, rmap), (s2, src)]:
        assert torch.equal(a_, b_)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_row_kernels_with_dropped_pairs(abi, dt):
    T, E, k, C, H = 500, 16, 4, 100, 256
    r = np.random.default_rng(77)
    logits = (r.standard_normal((T, E)) - 2.0 * np.log1p(np.arange(E))).astype(np.float32)
    idx, gate = _route(abi, logits, k)
    ridx, rgate = oracle.route(logits, k)
    _, _, _, rm, rs = oracle.permute_capacity(np.zeros((T, 1)), ridx, E, C)
    assert (rm < 0).any()
    R = E * C
    tdt, code, tol = _tdt(dt), (abi.MOE_BF16 if dt == "bf16" else abi.MOE_F32), TOL[dt]
    yp = _store(r.standard_normal((R, H)), dt)
    ys = _store(r.standard_normal((T, H)), dt)
    dy = _store(r.standard_normal((T, H)), dt)
    RM = dev(rm.astype(np.int32), torch.int32)
    y = torch.empty(T, H, dtype=tdt, device="cuda")
    abi.moe_unpermute_combine(dev(yp, tdt), RM, gate, dev(ys, tdt), code, T, H, k, R, y)
    dyp = torch.full((R, H), 3.0, dtype=tdt, device="cuda")
    dgate = torch.empty(T, k, dtype=torch.float32, device="cuda")
    abi.moe_unpermute_combine_bwd(dev(dy, tdt), dev(yp, tdt), RM, gate, code, T, H, k, R, dyp,
                                  dgate)
    dxp = _store(r.standard_normal((R, H)), dt)
    dx = torch.empty(T, H, dtype=tdt, device="cuda")
    abi.moe_permute_bwd(dev(dxp, tdt), RM, code, T, H, k, R, None, None, dx)
    torch.cuda.synchronize()
    g = host(gate)
    assert rel_err(host(y), oracle.combine(yp, rm, g, ys)) <= tol
    rdyp, rdgate = oracle.combine_backward(dy, yp, rm, g)
    filled = rs >= 0
    assert rel_err(host(dyp)[filled], rdyp[filled]) <= tol
    assert np.all(host(dyp)[~filled] == 3.0)          # rows no pair fills are not written
    assert rel_err(host(dgate), rdgate) <= 1e-5
    assert not host(dgate)[rm < 0].any()
    assert rel_err(host(dx), oracle.permute_backward(dxp, rm)) <= tol
    # clearing the unfilled rows leaves the filled ones alone
    before = host(dyp).copy()
    abi.moe_clear_empty_rows(dev(rs.astype(np.int32), torch.int32), R, code, H, dyp)
    torch.cuda.synchronize()
    after = host(dyp)
    assert not after[~filled].any() and np.array_equal(after[filled], before[filled])


@pytest.mark.parametrize("name,over,factor", [("tiny", {}, 1.0), ("small", {"T": 1024}, 1.0),
                                              ("pangu", {"T": 1024}, 1.2),
                                              # the benchmark's drop-and-pad run at full size
                                              ("pangu", {}, 1.2)])
def test_capacity_layer_matches_oracle(name, over, factor):
    cfg = synth.get_config(name, **over)
    C = oracle.capacity(cfg.T, cfg.k, cfg.E, factor)
    print(f"[capacity] config={cfg.name} T={cfg.T} C={C}", flush=True)
    inp = synth.make_inputs(cfg)
    L = make_layer(cfg, inp, capacity=C)
    L.forward()
    L.backward()
    torch.cuda.synchronize()
    acc = np.float64 if cfg.dtype == "f32" else np.float32
    # the oracle routes on the GPU's fp32 logits: indices then agree exactly
    lg = host(L.logits)
    fwd = oracle.layer_forward(inp.x, cfg.k, cfg.E, inp.w13, inp.w2, logits=lg, g0=cfg.g0,
                               G=cfg.G, ws13=inp.ws13, ws2=inp.ws2, acc=acc, C=C)
    assert np.array_equal(host(L.idx), fwd["idx"])
    assert np.array_equal(host(L.row_id_map), fwd["row_id_map"])
    assert np.array_equal(host(L.src_token), fwd["src_token"])
    assert (fwd["row_id_map"] < 0).any(), "the case should drop pairs"
    tol = TOL[cfg.dtype]
    assert rel_err(host(L.y), fwd["y"]) <= tol
    bwd = oracle.layer_backward(fwd, inp.dy, inp.x, inp.w13, inp.w2,
                                wg=inp.wg if cfg.router else None, g0=cfg.g0, G=cfg.G,
                                ws13=inp.ws13, ws2=inp.ws2, acc=acc)
    assert rel_err(host(L.dgate), bwd["dgate"]) <= tol
    assert rel_err(host(L.dw13), bwd["dw13"]) <= tol
    assert rel_err(host(L.dw2), bwd["dw2"]) <= tol
    # dx: routed, shared and router parts, all from the oracle
    assert rel_err(host(L.dx), bwd["dx"]) <= tol
    if cfg.router:   # through dgate, which carries the bf16 roundings of yp
        assert rel_err(host(L.dx_router), bwd["dx_router"]) <= tol
        assert rel_err(host(L.dwg), bwd["dwg"]) <= tol


def test_capacity_holding_every_pair_equals_dropless():
    cfg = synth.get_config("small", T=1024)
    inp = synth.make_inputs(cfg)
    A = make_layer(cfg, inp)
    A.step()
    torch.cuda.synchronize()
    C = int(host(A.counts).max())
    B = make_layer(cfg, inp, capacity=C)
    B.step()
    torch.cuda.synchronize()
    for n in ("y", "dx", "dw13", "dw2", "dgate", "dlogits", "dwg"):
        assert torch.equal(getattr(A, n), getattr(B, n)), n


def test_recompute_with_capacity_equals_saving_capacity():
    """Recompute on drop-and-pad: unfilled rows (src_token -1) gather zeros,
    so the results equal the saving drop-and-pad layer bit for bit."""
    cfg = synth.get_config("pangu", T=1024)
    C = oracle.capacity(cfg.T, cfg.k, cfg.E, 1.2)
    inp = synth.make_inputs(cfg)
    A = make_layer(cfg, inp, capacity=C)
    B = make_layer(cfg, inp, capacity=C, recompute=True)
    A.forward()
    B.forward()
    torch.cuda.synchronize()
    B.act.fill_(float("nan"))
    B.sh_act.fill_(float("nan"))
    A.backward()
    B.backward()
    torch.cuda.synchronize()
    assert (host(A.row_id_map) < 0).any()
    for n in ("y", "dx", "dw13", "dw2", "dgate", "dws13", "dws2", "dwg"):
        assert torch.equal(getattr(A, n), getattr(B, n)), n
