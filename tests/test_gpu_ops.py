"""Per-call parity of the HIP library against the CPU oracle (GPU only).

Integer and index outputs are compared bit for bit; floating-point outputs by
max|gpu - ref| <= tol * max|ref| per tensor, with tol = 1e-5 for fp32
storage and 2e-2 for bf16 storage (fp32 accumulation in both).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import dev, have_gpu, host, rel_err

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

TOL = {"f32": 1e-5, "bf16": 2e-2}


@pytest.fixture(scope="module")
def abi():
    from routing_permute_grouped_moe_amd import abi as a
    return a


def _rng(i):
    return np.random.default_rng(7000 + i)


def _tdt(dt):
    return torch.bfloat16 if dt == "bf16" else torch.float32


def _code(abi, dt):
    return abi.MOE_BF16 if dt == "bf16" else abi.MOE_F32


def _store(a, dt):
    return synth.bf16_round(np.asarray(a, np.float32)) if dt == "bf16" else np.asarray(a, np.float32)


# ---------------------------------------------------------------- routing

ROUTE_CASES = [(64, 8, 2, "normal"), (300, 64, 6, "normal"), (257, 256, 8, "ties"),
               (100, 1024, 8, "normal"), (33, 1024, 1024, "normal"), (50, 1, 1, "normal"),
               (70, 5, 5, "ties"), (129, 200, 3, "ties"),
               # every per-lane width of the kernels: E = 100 (2), E = 400 (8)
               (90, 100, 4, "ties"), (77, 400, 8, "normal"),
               # -0.0 and +0.0 are the same logit: ties broken by expert index
               (64, 64, 8, "signed_zeros"), (40, 300, 20, "signed_zeros")]


@pytest.mark.parametrize("T,E,k,kind", ROUTE_CASES)
def test_route_bit_exact_indices(abi, T, E, k, kind):
    r = _rng(T + E + k)
    if kind == "ties":
        logits = (r.integers(-3, 4, size=(T, E)) * 0.5).astype(np.float32)
    elif kind == "signed_zeros":
        # mostly zeros of either sign, a few +-1: the k-th place falls among zeros
        vals = np.array([-0.0, 0.0, -0.0, 0.0, -1.0, 1.0], np.float32)
        logits = vals[r.integers(0, len(vals), size=(T, E))]
        assert np.signbit(logits[logits == 0]).any() and (~np.signbit(logits[logits == 0])).any()
    else:
        logits = r.standard_normal((T, E)).astype(np.float32) * 2
    L = dev(logits, torch.float32)
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    gate = torch.empty(T, k, dtype=torch.float32, device="cuda")
    abi.moe_route(L, T, E, k, idx, gate)
    torch.cuda.synchronize()
    ridx, rgate = oracle.route(logits, k)
    assert np.array_equal(host(idx), ridx)
    assert rel_err(host(gate), rgate) <= 1e-5
    # backward
    dgate = r.standard_normal((T, k)).astype(np.float32)
    dl = torch.empty(T, E, dtype=torch.float32, device="cuda")
    abi.moe_route_bwd(L, idx, dev(dgate, torch.float32), T, E, k, dl)
    torch.cuda.synchronize()
    ref = oracle.route_backward(logits, ridx, dgate)
    assert rel_err(host(dl), ref) <= 1e-5
    assert np.abs(host(dl).astype(np.float64).sum(axis=1)).max() <= 1e-5 * max(1.0, np.abs(ref).max())


def test_route_deterministic(abi):
    r = _rng(99)
    T, E, k = 4096, 256, 8
    L = dev(r.standard_normal((T, E)).astype(np.float32), torch.float32)
    outs = []
    for _ in range(2):
        idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
        gate = torch.empty(T, k, dtype=torch.float32, device="cuda")
        abi.moe_route(L, T, E, k, idx, gate)
        outs.append((idx.clone(), gate.clone()))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


# ---------------------------------------------------------------- permute family

PERM_CASES = [(1, 8, 2, 128, "f32"), (31, 8, 2, 128, "f32"), (33, 16, 4, 256, "bf16"),
              (1000, 64, 6, 2048, "bf16"), (513, 256, 8, 7680, "bf16"), (40, 5, 5, 64, "f32"),
              (2048, 1024, 16, 128, "bf16"), (100, 3, 1, 8192, "f32"),
              # maximum sizes: every token picks all 1024 experts; bf16 rows
              # at the 32 KB a row kernel keeps in registers
              (8, 1024, 1024, 64, "bf16"), (77, 16, 4, 16384, "bf16"),
              # one expert; 32 rank blocks of 4096 pairs scanned in slices
              (50, 1, 1, 64, "f32"), (16384, 256, 8, 64, "bf16")]


def _perm_inputs(T, E, k, H, dt, seed):
    r = _rng(seed)
    bias = np.where(np.arange(E) < max(1, E // 16), 3.0, 0.0)   # a few hot experts
    logits = (r.standard_normal((T, E)) + bias).astype(np.float32)
    idx, gate = oracle.route(logits, k)
    x = _store(r.standard_normal((T, H)), dt)
    return r, idx, gate.astype(np.float32), x


@pytest.mark.parametrize("T,E,k,H,dt", PERM_CASES)
def test_permute_bit_exact(abi, T, E, k, H, dt):
    r, idx, gate, x = _perm_inputs(T, E, k, H, dt, T * 3 + E)
    R = T * k
    tdt = _tdt(dt)
    X = dev(x, tdt)
    xp = torch.empty(R, H, dtype=tdt, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    rmap = torch.empty(T, k, dtype=torch.int32, device="cuda")
    src = torch.empty(R, dtype=torch.int32, device="cuda")
    wsb = abi.moe_permute_workspace_bytes(T, E, k)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    abi.moe_permute(X, _code(abi, dt), dev(idx, torch.int32), T, H, E, k, xp, counts, offsets,
                    rmap, src, ws, wsb)
    torch.cuda.synchronize()
    rxp, rc, ro, rm, rs = oracle.permute(x, idx, E)
    assert np.array_equal(host(counts), rc)
    assert np.array_equal(host(offsets), ro)
    assert np.array_equal(host(rmap), rm)
    assert np.array_equal(host(src), rs)
    assert np.array_equal(host(xp), rxp)          # a bit copy of bf16/fp32 values
    # a second call on the same workspace (outputs cleared) gives the same maps
    for t in (counts, offsets, rmap, src):
        t.fill_(-1)
    abi.moe_permute(X, _code(abi, dt), dev(idx, torch.int32), T, H, E, k, xp, counts, offsets,
                    rmap, src, ws, wsb)
    torch.cuda.synchronize()
    for got, ref in ((counts, rc), (offsets, ro), (rmap, rm), (src, rs)):
        assert np.array_equal(host(got), ref)


@pytest.mark.parametrize("T,E,k,H,dt", PERM_CASES)
def test_combine_and_backward(abi, T, E, k, H, dt):
    r, idx, gate, x = _perm_inputs(T, E, k, H, dt, T * 5 + E)
    R = T * k
    tdt = _tdt(dt)
    _, _, _, rmap, _ = oracle.permute(x, idx, E)
    yp = _store(r.standard_normal((R, H)), dt)
    ys = _store(r.standard_normal((T, H)), dt)
    dy = _store(r.standard_normal((T, H)), dt)
    RM, G = dev(rmap, torch.int32), dev(gate, torch.float32)
    YP, YS, DY = dev(yp, tdt), dev(ys, tdt), dev(dy, tdt)
    code = _code(abi, dt)
    tol = TOL[dt]
    for with_shared in (False, True):
        y = torch.empty(T, H, dtype=tdt, device="cuda")
        abi.moe_unpermute_combine(YP, RM, G, YS if with_shared else None, code, T, H, k, T * k, y)
        torch.cuda.synchronize()
        ref = oracle.combine(yp, rmap, gate, ys if with_shared else None)
        assert rel_err(host(y), ref) <= tol
    dyp = torch.empty(R, H, dtype=tdt, device="cuda")
    dgate = torch.empty(T, k, dtype=torch.float32, device="cuda")
    abi.moe_unpermute_combine_bwd(DY, YP, RM, G, code, T, H, k, T * k, dyp, dgate)
    torch.cuda.synchronize()
    rdyp, rdg = oracle.combine_backward(dy, yp, rmap, gate)
    assert rel_err(host(dyp), rdyp) <= tol
    assert rel_err(host(dgate), rdg) <= 1e-5      # fp32 dot of storage values
    # permute backward with two addends
    dxp = _store(r.standard_normal((R, H)), dt)
    a0 = _store(r.standard_normal((T, H)), dt)
    a1 = _store(r.standard_normal((T, H)), dt)
    dx = torch.empty(T, H, dtype=tdt, device="cuda")
    abi.moe_permute_bwd(dev(dxp, tdt), RM, code, T, H, k, T * k, dev(a0, tdt), dev(a1, tdt), dx)
    torch.cuda.synchronize()
    ref = oracle.permute_backward(dxp, rmap) + a0 + a1
    assert rel_err(host(dx), ref) <= tol
    abi.moe_permute_bwd(dev(dxp, tdt), RM, code, T, H, k, T * k, None, None, dx)
    torch.cuda.synchronize()
    assert rel_err(host(dx), oracle.permute_backward(dxp, rmap)) <= tol


def test_permute_empty_input(abi):
    E = 16
    counts = torch.full((E,), 7, dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), 7, dtype=torch.int32, device="cuda")
    abi.moe_permute(None, abi.MOE_BF16, None, 0, 128, E, 2, None, counts, offsets, None, None,
                    None, 0)
    torch.cuda.synchronize()
    assert int(counts.abs().sum()) == 0 and int(offsets.abs().sum()) == 0


# ---------------------------------------------------------------- router projection

@pytest.mark.parametrize("T,H,E,dt", [(256, 128, 8, "f32"), (1000, 2048, 64, "bf16"),
                                      (300, 7680, 256, "bf16"), (2048, 2048, 64, "bf16"),
                                      (8192, 7680, 256, "bf16"), (512, 256, 128, "bf16")])
def test_router_projection(abi, T, H, E, dt):
    r = _rng(T + H)
    x = _store(r.standard_normal((T, H)), dt)
    wg = (r.standard_normal((H, E)) * 0.02).astype(np.float32)
    bias = (r.standard_normal(E) * 0.5).astype(np.float32)
    tdt = _tdt(dt)
    X, WG, B = dev(x, tdt), dev(wg, torch.float32), dev(bias, torch.float32)
    logits = torch.empty(T, E, dtype=torch.float32, device="cuda")
    wsb = abi.moe_router_workspace_bytes(T, H, E, _code(abi, dt))
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device="cuda")
    abi.moe_router_logits(X, _code(abi, dt), WG, B, T, H, E, logits, ws, wsb)
    torch.cuda.synchronize()
    assert rel_err(host(logits), oracle.router_logits(x, wg, bias)) <= 1e-5
    dl = r.standard_normal((T, E)).astype(np.float32)
    dx = torch.empty(T, H, dtype=tdt, device="cuda")
    dwg = torch.empty(H, E, dtype=torch.float32, device="cuda")
    db = torch.empty(E, dtype=torch.float32, device="cuda")
    DL = dev(dl, torch.float32)
    # right after the forward the workspace still holds wg's split: reusing
    # it gives the same bits
    abi.moe_router_logits_bwd(DL, X, _code(abi, dt), WG, T, H, E, dx, dwg, db, ws, wsb,
                              flags=abi.MOE_ROUTER_WG_SPLIT)
    dx2, dwg2, db2 = torch.empty_like(dx), torch.empty_like(dwg), torch.empty_like(db)
    abi.moe_router_logits_bwd(DL, X, _code(abi, dt), WG, T, H, E, dx2, dwg2, db2, ws, wsb)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx2) and torch.equal(dwg, dwg2) and torch.equal(db, db2)
    rdx, rdwg, rdb = oracle.router_backward(dl, x, wg)
    err_dx = rel_err(host(dx), rdx)
    assert err_dx <= TOL[dt]
    if dt == "bf16":
        # dx from the bf16 high parts of dlogits and wg, stored in bf16: its
        # error stays within a few times that of storing the exact product
        # in bf16 (the output rounding alone)
        err_store = rel_err(synth.bf16_round(rdx.astype(np.float32)), rdx)
        print(f"router dx: error {err_dx:.2e}, bf16 storage alone {err_store:.2e}")
        assert err_dx <= 3 * err_store
    assert rel_err(host(dwg), rdwg) <= 1e-5
    assert rel_err(host(db), rdb) <= 1e-5


# ---------------------------------------------------------------- grouped GEMM

GMM_CASES = [
    # counts per routed group, H, I, g0, G (None = all), shared rows, dtype
    ([300, 0, 17, 1, 256, 64, 0, 513], 256, 192, 0, None, 0, "bf16"),
    ([300, 0, 17, 1, 256, 64, 0, 513], 256, 192, 0, None, 0, "f32"),
    ([5, 40, 0, 700, 3, 90], 512, 128, 2, 3, 200, "bf16"),
    ([128, 64], 128, 64, 0, None, 77, "f32"),
    ([0, 0, 0], 128, 64, 0, None, 0, "bf16"),
    ([1000], 384, 320, 0, None, 0, "bf16"),
    ([], 256, 128, 0, 0, 300, "bf16"),
    # 150 small groups: several rounds of tiles on a 256-CU grid, so the
    # per-XCD counters hand out many tiles
    ([int(c) for c in np.random.default_rng(7).integers(0, 60, 150)], 1024, 512, 0, None, 40,
     "bf16"),
    # 40 groups of 100-600 rows with a shared expert: the paired backward
    # launches run several rounds of both products' tiles
    ([int(c) for c in np.random.default_rng(11).integers(100, 600, 40)], 512, 256, 0, None, 300,
     "bf16"),
    # 86 groups of 300 rows (H = 256): 172 dact tiles and 86 leading dW2
    # tiles are 258 long tiles, two past a round of a 256-workgroup grid, so
    # the first backward launch leaves two leading dW2 tiles to the second
    ([300] * 86, 256, 128, 0, None, 0, "bf16"),
    # the largest window: 1024 experts, most of them empty or tiny
    ([int(c) for c in np.random.default_rng(9).integers(0, 4, 1024) * (
        np.random.default_rng(10).random(1024) < 0.3)], 128, 64, 0, None, 0, "bf16"),
]


@pytest.mark.parametrize("dynamic", [True, False], ids=["dynamic", "static"])
@pytest.mark.parametrize("counts,H,I,g0,G,shT,dt", GMM_CASES)
def test_grouped_gemm(abi, counts, H, I, g0, G, shT, dt, dynamic):
    r = _rng(sum(counts) + H + I + g0)
    E = len(counts)
    G = E - g0 if G is None else G
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    R = int(offsets[-1]) + 5                 # a few rows past the last group
    tdt, code, tol = _tdt(dt), _code(abi, dt), TOL[dt]
    xp = _store(r.standard_normal((R, H)), dt)
    dyp = _store(r.standard_normal((R, H)), dt)
    w13 = _store(r.standard_normal((max(G, 1), 2 * I, H)) * 0.05, dt)
    w2 = _store(r.standard_normal((max(G, 1), H, I)) * 0.05, dt)
    sx = _store(r.standard_normal((shT, H)), dt)
    sdy = _store(r.standard_normal((shT, H)), dt)
    sw13 = _store(r.standard_normal((2 * I, H)) * 0.05, dt)
    sw2 = _store(r.standard_normal((H, I)) * 0.05, dt)

    def z(*s):
        return torch.zeros(*s, dtype=tdt, device="cuda")

    OFF = dev(offsets if E else np.zeros(1), torch.int32)
    XP, DYP, W13, W2 = dev(xp, tdt), dev(dyp, tdt), dev(w13, tdt), dev(w2, tdt)
    h13, act, yp = z(R, 2 * I), z(R, I), z(R, H)
    dh13, dxp = z(R, 2 * I), z(R, H)
    dw13, dw2 = torch.full((max(G, 1), 2 * I, H), 9.0, dtype=tdt, device="cuda"), \
        torch.full((max(G, 1), H, I), 9.0, dtype=tdt, device="cuda")
    sh = None
    if shT:
        SX, SDY = dev(sx, tdt), dev(sdy, tdt)
        shb = dict(x=SX, w13=dev(sw13, tdt), w2=dev(sw2, tdt), h13=z(shT, 2 * I), act=z(shT, I),
                   y=z(shT, H), dy=SDY, dh13=z(shT, 2 * I), dx=z(shT, H), dw13=z(2 * I, H),
                   dw2=z(H, I))
        sh = abi.shared_expert(T=shT, **shb)
    wsb = abi.moe_gmm_workspace_bytes() if dynamic else 0
    ws = torch.zeros(max(wsb, 256), dtype=torch.uint8, device="cuda") if dynamic else None
    abi.moe_grouped_gemm_fwd(XP, OFF, g0, G, R, code, H, I, W13, W2, h13, act, yp, sh, ws, wsb)
    torch.cuda.synchronize()
    rh13, ract, ryp = oracle.grouped_forward(xp, offsets, w13, w2, g0, G) if E else \
        (np.zeros((R, 2 * I)), np.zeros((R, I)), np.zeros((R, H)))
    assert rel_err(host(h13), rh13) <= tol
    assert rel_err(host(act), ract) <= tol
    assert rel_err(host(yp), ryp) <= tol
    if dynamic:
        # with the workspace both products run in one dependency-ordered
        # launch (groups above half a tile); without it, as two launches:
        # the same bits either way
        s_h13, s_act, s_yp = z(R, 2 * I), z(R, I), z(R, H)
        ssh = None
        if shT:
            sshb = dict(shb, h13=z(shT, 2 * I), act=z(shT, I), y=z(shT, H))
            ssh = abi.shared_expert(T=shT, **sshb)
        abi.moe_grouped_gemm_fwd(XP, OFF, g0, G, R, code, H, I, W13, W2, s_h13, s_act, s_yp, ssh,
                                 None, 0)
        torch.cuda.synchronize()
        for name, a, b in (("h13", h13, s_h13), ("act", act, s_act), ("yp", yp, s_yp)):
            assert torch.equal(a, b), name
        if shT:
            for n in ("h13", "act", "y"):
                assert torch.equal(shb[n], sshb[n]), "shared " + n
    # backward dX / dW on the GPU's own saved activations
    abi.moe_grouped_gemm_bwd_dx(DYP, OFF, g0, G, R, code, H, I, W13, W2, h13, dh13, dxp, sh, ws,
                                wsb)
    abi.moe_grouped_gemm_bwd_dw(XP, act, DYP, dh13, OFF, g0, G, R, code, H, I, dw13, dw2, sh, ws,
                                wsb)
    # dX and dW in one call (paired launches): the same bits
    c_dh13, c_dxp = z(R, 2 * I), z(R, H)
    c_dw13, c_dw2 = torch.full_like(dw13, 7.0), torch.full_like(dw2, 7.0)
    csh = None
    if shT:
        cshb = dict(shb, dh13=z(shT, 2 * I), dx=z(shT, H), dw13=z(2 * I, H), dw2=z(H, I))
        csh = abi.shared_expert(T=shT, **cshb)
    abi.moe_grouped_gemm_bwd(XP, act, DYP, OFF, g0, G, R, code, H, I, W13, W2, h13, c_dh13, c_dxp,
                             c_dw13, c_dw2, csh, ws, wsb)
    torch.cuda.synchronize()
    if dynamic:   # every call leaves the scheduler counters at zero
        assert int(ws.to(torch.int32).sum()) == 0
    for name, a, b in (("dh13", dh13, c_dh13), ("dxp", dxp, c_dxp), ("dw13", dw13[:G], c_dw13[:G]),
                       ("dw2", dw2[:G], c_dw2[:G])):
        assert torch.equal(a, b), name
    if shT:
        for n in ("dh13", "dx", "dw13", "dw2"):
            assert torch.equal(shb[n], cshb[n]), "shared " + n
    if E:
        rdh13, rdxp, rdw13, rdw2 = oracle.grouped_backward(xp, dyp, offsets, w13, w2, g0, G)
        assert rel_err(host(dh13), rdh13) <= tol
        assert rel_err(host(dxp), rdxp) <= tol
        assert rel_err(host(dw13)[:G], rdw13) <= tol
        assert rel_err(host(dw2)[:G], rdw2) <= tol
        for g in range(G):                     # empty groups: exact zeros
            if counts[g0 + g] == 0:
                assert not host(dw13)[g].any() and not host(dw2)[g].any()
    if shT:
        rh, ra, ry = oracle.expert_forward(sx, sw13, sw2)
        assert rel_err(host(shb["h13"]), rh) <= tol
        assert rel_err(host(shb["y"]), ry) <= tol
        rdh, rdx, rdw13s, rdw2s = oracle.expert_backward(sx, sw13, sw2, sdy)
        assert rel_err(host(shb["dh13"]), rdh) <= tol
        assert rel_err(host(shb["dx"]), rdx) <= tol
        assert rel_err(host(shb["dw13"]), rdw13s) <= tol
        assert rel_err(host(shb["dw2"]), rdw2s) <= tol
    # rows outside the window are untouched
    if E:
        lo, hi = int(offsets[g0]), int(offsets[g0 + G])
        for t in (yp, dxp, h13):
            hv = host(t)
            assert not hv[:lo].any() and not hv[hi:].any()


@pytest.mark.parametrize("kind", ["light_tiles", "half_tiles"])
def test_grouped_gemm_small_group_builds_are_bitwise_equal(abi, kind):
    """Calls whose groups average at most half a tile of rows launch the
    builds that skip the MFMAs of padding fragments.  The same groups with a
    larger row count R (so the host picks the full-tile builds) give the same
    bits in every output row, also through the gathering forward (which
    matches the forward on the gathered rows bit for bit).  light_tiles:
    most tiles hold at most 64 rows, so the waves take the short loops;
    half_tiles: every group holds 65-128 rows, so the small-group build runs
    its full loop (the device-side choice declines the short ones)."""
    r = _rng(4242)
    if kind == "light_tiles":
        counts = [int(c) for c in r.integers(0, 90, 96)]
        counts[5], counts[17] = 0, 300      # an empty group and a multi-tile one
    else:
        counts = [int(c) for c in r.integers(65, 129, 96)]
    G, H, I = len(counts), 512, 256
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    R = int(offsets[-1])
    assert R <= G * 128                     # small groups: light builds
    R_big = G * 256 + 1                     # same groups, full-tile builds
    xp = _store(r.standard_normal((R_big, H)), "bf16")
    dyp = _store(r.standard_normal((R_big, H)), "bf16")
    w13 = _store(r.standard_normal((G, 2 * I, H)) * 0.05, "bf16")
    w2 = _store(r.standard_normal((G, H, I)) * 0.05, "bf16")
    tdt, code = torch.bfloat16, abi.MOE_BF16
    OFF = dev(offsets, torch.int32)
    SRC = dev(np.arange(R_big), torch.int32)
    XP, DYP, W13, W2 = dev(xp, tdt), dev(dyp, tdt), dev(w13, tdt), dev(w2, tdt)
    wsb = abi.moe_gmm_workspace_bytes()
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    outs = []
    for rows in (R, R_big):
        h13 = torch.zeros(R_big, 2 * I, dtype=tdt, device="cuda")
        act = torch.zeros(R_big, I, dtype=tdt, device="cuda")
        yp = torch.zeros(R_big, H, dtype=tdt, device="cuda")
        dh13 = torch.zeros(R_big, 2 * I, dtype=tdt, device="cuda")
        dxp = torch.zeros(R_big, H, dtype=tdt, device="cuda")
        abi.moe_grouped_gemm_fwd(XP, OFF, 0, G, rows, code, H, I, W13, W2, h13, act, yp, None,
                                 ws, wsb)
        abi.moe_grouped_gemm_bwd_dx(DYP, OFF, 0, G, rows, code, H, I, W13, W2, h13, dh13, dxp,
                                    None, ws, wsb)
        # the gathering forward, with row r reading token r (so its inputs are xp's)
        gh13 = torch.zeros(R_big, 2 * I, dtype=tdt, device="cuda")
        gact = torch.zeros(R_big, I, dtype=tdt, device="cuda")
        gyp = torch.zeros(R_big, H, dtype=tdt, device="cuda")
        abi.moe_grouped_gemm_fwd_gather(XP, SRC, R_big, OFF, 0, G, rows, code, H, I, W13, W2,
                                        gh13, gact, gyp, None, ws, wsb)
        torch.cuda.synchronize()
        outs.append([t[:R].clone() for t in (h13, act, yp, dh13, dxp, gh13, gact, gyp)])
    names = ("h13", "act", "yp", "dh13", "dxp", "gather h13", "gather act", "gather yp")
    for name, a, b in zip(names, outs[0], outs[1]):
        assert torch.equal(a, b), name
    for a, b in zip(outs[0][:3], outs[0][5:]):
        assert torch.equal(a, b)


def test_chained_forwards_on_two_streams(abi):
    """Two chained forward launches at once, on two streams of the same
    priority with a workspace each: every workgroup of one can be held up
    while the other holds its CU, so this runs the protocol's no-deadlock
    property on the hardware (a stuck wait gives up after one second and
    sets the workspace's error word, which fails here rather than hanging).
    Both results equal the same calls run one after the other, bit for bit,
    over several rounds."""
    r = _rng(777)
    H, I = 1024, 512
    probs = []
    for counts in ([int(c) for c in r.integers(100, 900, 12)],
                   [int(c) for c in r.integers(200, 1200, 10)]):
        G = len(counts)
        offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
        R = int(offsets[-1])
        tdt = torch.bfloat16
        p = dict(G=G, R=R, OFF=dev(offsets, torch.int32),
                 XP=dev(_store(r.standard_normal((R, H)), "bf16"), tdt),
                 W13=dev(_store(r.standard_normal((G, 2 * I, H)) * 0.05, "bf16"), tdt),
                 W2=dev(_store(r.standard_normal((G, H, I)) * 0.05, "bf16"), tdt))
        probs.append(p)
    wsb = abi.moe_gmm_workspace_bytes()

    def outputs(p):
        return [torch.zeros(p["R"], 2 * I, dtype=torch.bfloat16, device="cuda"),
                torch.zeros(p["R"], I, dtype=torch.bfloat16, device="cuda"),
                torch.zeros(p["R"], H, dtype=torch.bfloat16, device="cuda")]

    def fwd(p, out, ws, stream=None):
        abi.moe_grouped_gemm_fwd(p["XP"], p["OFF"], 0, p["G"], p["R"], abi.MOE_BF16, H, I,
                                 p["W13"], p["W2"], *out, None, ws, wsb, stream)

    wss = [torch.zeros(wsb, dtype=torch.uint8, device="cuda") for _ in probs]
    ref = []
    for p, ws in zip(probs, wss):
        out = outputs(p)
        fwd(p, out, ws)
        ref.append(out)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(4):
        got = [outputs(p) for p in probs]
        torch.cuda.synchronize()
        for p, out, ws, st in zip(probs, got, wss, streams):
            fwd(p, out, ws, st)
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            for x, y in zip(a, b):
                assert torch.equal(x, y)
        for ws in wss:   # counters back at zero, no wait gave up
            assert int(ws.view(torch.int32).abs().sum()) == 0
