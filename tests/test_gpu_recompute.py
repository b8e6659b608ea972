"""The recompute variant (no saved xp / act): the grouped GEMMs gather token
rows through src_token and dW recomputes act from h13 (GPU only).

Per call: the gathering calls on (x, src_token) must give the same bits as
the saving calls on xp = x[src_token], and match the oracle to the bf16
tolerance.  Whole layer: every output and gradient of a recompute layer must
equal the saving layer's bit for bit, with act overwritten by NaN between the
forward and the backward (so nothing can come from the forward's act).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import dev, have_gpu, host, make_layer, rel_err

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

TOL = 2e-2


@pytest.fixture(scope="module")
def abi():
    from routing_permute_grouped_moe_amd import abi as a
    return a


CASES = [
    # counts per routed group, H, I, g0, G (None = all), shared rows, tokens
    ([300, 0, 17, 1, 256, 64, 0, 513], 256, 192, 0, None, 0, 700),
    ([5, 40, 0, 700, 3, 90], 512, 128, 2, 3, 200, 500),
    ([1000], 384, 320, 0, None, 0, 1000),
    ([], 256, 128, 0, 0, 300, 300),
    ([int(c) for c in np.random.default_rng(8).integers(0, 60, 150)], 1024, 512, 0, None, 40,
     900),
]


def _bf(a):
    return synth.bf16_round(np.asarray(a, np.float32))


@pytest.mark.parametrize("dynamic", [True, False], ids=["dynamic", "static"])
@pytest.mark.parametrize("counts,H,I,g0,G,shT,T", CASES)
def test_gather_calls_match_saving_calls(abi, counts, H, I, g0, G, shT, T, dynamic):
    print(f"case counts={len(counts)} groups H={H} I={I} g0={g0} G={G} shT={shT} T={T}",
          flush=True)
    r = np.random.default_rng(sum(counts) + H + I + T)
    E = len(counts)
    G = E - g0 if G is None else G
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    R = int(offsets[-1]) + 5
    code, bf = abi.MOE_BF16, torch.bfloat16
    x = _bf(r.standard_normal((T, H)))
    src = r.integers(0, T, R).astype(np.int32)
    src[::97] = T + 3                        # out of range: reads a zero row
    xp = np.where((src < T)[:, None], x[np.minimum(src, T - 1)], 0).astype(np.float32)
    dyp = _bf(r.standard_normal((R, H)))
    w13 = _bf(r.standard_normal((max(G, 1), 2 * I, H)) * 0.05)
    w2 = _bf(r.standard_normal((max(G, 1), H, I)) * 0.05)
    sw13 = _bf(r.standard_normal((2 * I, H)) * 0.05)
    sw2 = _bf(r.standard_normal((H, I)) * 0.05)
    sx = _bf(r.standard_normal((shT, H)))
    sdy = _bf(r.standard_normal((shT, H)))

    def z(*s):
        return torch.zeros(*s, dtype=bf, device="cuda")

    OFF = dev(offsets if E else np.zeros(1), torch.int32)
    X, SRC, XP, DYP = dev(x, bf), dev(src, torch.int32), dev(xp, bf), dev(dyp, bf)
    W13, W2 = dev(w13, bf), dev(w2, bf)

    def shared():
        if not shT:
            return None, None
        b = dict(x=dev(sx, bf), w13=dev(sw13, bf), w2=dev(sw2, bf), h13=z(shT, 2 * I),
                 act=z(shT, I), y=z(shT, H), dy=dev(sdy, bf), dh13=z(shT, 2 * I), dx=z(shT, H),
                 dw13=z(2 * I, H), dw2=z(H, I))
        return abi.shared_expert(T=shT, **b), b

    wsb = abi.moe_gmm_workspace_bytes() if dynamic else 0

    def ws():
        return torch.zeros(max(wsb, 256), dtype=torch.uint8, device="cuda") if dynamic else None

    # saving path on xp
    sh, shb = shared()
    h13, act, yp, dh13, dxp = z(R, 2 * I), z(R, I), z(R, H), z(R, 2 * I), z(R, H)
    dw13, dw2 = z(max(G, 1), 2 * I, H), z(max(G, 1), H, I)
    w = ws()
    abi.moe_grouped_gemm_fwd(XP, OFF, g0, G, R, code, H, I, W13, W2, h13, act, yp, sh, w, wsb)
    abi.moe_grouped_gemm_bwd_dx(DYP, OFF, g0, G, R, code, H, I, W13, W2, h13, dh13, dxp, sh, w,
                                wsb)
    abi.moe_grouped_gemm_bwd_dw(XP, act, DYP, dh13, OFF, g0, G, R, code, H, I, dw13, dw2, sh, w,
                                wsb)
    # gathering path on x, act poisoned before dW
    sh2, shb2 = shared()
    h13b, actb, ypb, dh13b, dxpb = z(R, 2 * I), z(R, I), z(R, H), z(R, 2 * I), z(R, H)
    dw13b, dw2b = z(max(G, 1), 2 * I, H), z(max(G, 1), H, I)
    w2s = ws()
    abi.moe_grouped_gemm_fwd_gather(X, SRC, T, OFF, g0, G, R, code, H, I, W13, W2, h13b, actb,
                                    ypb, sh2, w2s, wsb)
    torch.cuda.synchronize()
    act_fwd = host(actb).copy()
    actb.fill_(float("nan"))
    if shT:
        sh_act_fwd = host(shb2["act"]).copy()
        shb2["act"].fill_(float("nan"))
    abi.moe_grouped_gemm_bwd_dx(DYP, OFF, g0, G, R, code, H, I, W13, W2, h13b, dh13b, dxpb, sh2,
                                w2s, wsb)
    abi.moe_grouped_gemm_bwd_dw_recompute(X, SRC, T, h13b, actb, DYP, dh13b, OFF, g0, G, R, code,
                                          H, I, dw13b, dw2b, sh2, w2s, wsb)
    torch.cuda.synchronize()
    for a_, b_ in [(h13, h13b), (yp, ypb), (dh13, dh13b), (dxp, dxpb), (dw13, dw13b),
                   (dw2, dw2b)]:
        assert torch.equal(a_, b_)
    assert np.array_equal(host(act), act_fwd)
    lo, hi = (int(offsets[g0]), int(offsets[g0 + G])) if E else (0, 0)
    # the recomputed act equals the forward's on the window rows
    assert np.array_equal(host(actb)[lo:hi], act_fwd[lo:hi])
    if shT:
        for k_ in ("h13", "y", "dh13", "dx", "dw13", "dw2"):
            assert torch.equal(shb[k_], shb2[k_])
        assert np.array_equal(host(shb2["act"]), sh_act_fwd)
    if dynamic:
        assert int(w2s.to(torch.int32).sum()) == 0
    if E:
        rh13, ract, ryp = oracle.grouped_forward(xp, offsets, w13, w2, g0, G)
        assert rel_err(host(h13b), rh13) <= TOL
        assert rel_err(host(ypb), ryp) <= TOL
        _, _, rdw13, rdw2 = oracle.grouped_backward(xp, dyp, offsets, w13, w2, g0, G)
        assert rel_err(host(dw13b)[:G], rdw13) <= TOL
        assert rel_err(host(dw2b)[:G], rdw2) <= TOL


def test_permute_without_copy_writes_the_same_maps(abi):
    T, E, k, H = 1500, 64, 6, 256
    r = np.random.default_rng(31)
    logits = r.standard_normal((T, E)).astype(np.float32)
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    gate = torch.empty(T, k, dtype=torch.float32, device="cuda")
    abi.moe_route(dev(logits, torch.float32), T, E, k, idx, gate)
    x = dev(_bf(r.standard_normal((T, H))), torch.bfloat16)
    wsb = abi.moe_permute_workspace_bytes(T, E, k)
    outs = []
    for xp in (torch.empty(T * k, H, dtype=torch.bfloat16, device="cuda"), None):
        o = [torch.full((E,), -1, dtype=torch.int32, device="cuda"),
             torch.full((E + 1,), -1, dtype=torch.int32, device="cuda"),
             torch.full((T, k), -1, dtype=torch.int32, device="cuda"),
             torch.full((T * k,), -1, dtype=torch.int32, device="cuda")]
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
        abi.moe_permute(x if xp is not None else None, abi.MOE_BF16, idx, T, H, E, k, xp, *o, ws,
                        wsb)
        torch.cuda.synchronize()
        outs.append([host(t) for t in o])
    for a_, b_ in zip(*outs):
        assert np.array_equal(a_, b_)
    ridx, _ = oracle.route(logits, k)
    _, counts, offsets, rmap, src = oracle.permute(np.zeros((T, 1)), ridx, E)
    assert np.array_equal(outs[1][0], counts) and np.array_equal(outs[1][1], offsets)
    assert np.array_equal(outs[1][2], rmap) and np.array_equal(outs[1][3], src)


@pytest.mark.parametrize("name,over", [("small", {}), ("pangu", {"T": 2048}),
                                       ("deepseek", {"T": 1024}),
                                       # the benchmark's workload at full size
                                       ("pangu", {})])
def test_recompute_layer_equals_saving_layer(name, over):
    cfg = synth.get_config(name, **over)
    print(f"[recompute] config={cfg.name} T={cfg.T}", flush=True)
    inp = synth.make_inputs(cfg)
    A = make_layer(cfg, inp)
    B = make_layer(cfg, inp, recompute=True)
    assert B.xp is None and B.saved_bytes() < A.saved_bytes()
    A.forward()
    B.forward()
    torch.cuda.synchronize()
    B.act.fill_(float("nan"))
    if cfg.shared:
        B.sh_act.fill_(float("nan"))
    A.backward()
    B.backward()
    torch.cuda.synchronize()
    names = ["y", "dx", "dw13", "dw2", "dgate", "dlogits"]
    if cfg.router:
        names += ["dwg"]
    if cfg.shared:
        names += ["ys", "dws13", "dws2"]
    for n in names:
        assert torch.equal(getattr(A, n), getattr(B, n)), n
    G = cfg.groups
    off = host(A.offsets)
    lo, hi = int(off[cfg.g0]), int(off[cfg.g0 + G])
    # rows of remote experts are never written: compare the window
    assert torch.equal(A.h13[lo:hi], B.h13[lo:hi])
    assert torch.equal(A.act[lo:hi], B.act[lo:hi])
