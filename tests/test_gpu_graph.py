"""The layer's whole step captured in a HIP graph, GPU only.

No entry point allocates, copies to or from the host, clears memory or
synchronizes inside a call, and the grouped GEMM's scheduler workspace is
left zero by every call, so a step captured once replays as a fixed
sequence of kernels.  Each replay must give the eager step's bits: the
outputs are overwritten with a marker before every replay, with unrelated
eager work and synchronizations between the replays.
"""
import pytest
import torch

import synth
from gpu_util import have_gpu, make_layer

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

OUTPUTS = ("logits", "idx", "gate", "counts", "offsets", "row_id_map", "src_token", "y",
           "dgate", "dlogits", "dx", "dw13", "dw2", "dws13", "dws2", "dwg", "dbias", "load")


@pytest.mark.parametrize("name", ["small", "pangu"])
def test_layer_step_replays_from_a_hip_graph(name):
    cfg = synth.get_config(name)
    print(f"\n[graph] config={cfg.name} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k}", flush=True)
    L = make_layer(cfg, synth.make_inputs(cfg))
    # (logits are an input of the configs without a router)
    names = [n for n in OUTPUTS
             if getattr(L, n, None) is not None and (cfg.router or n != "logits")]
    L.step()
    torch.cuda.synchronize()
    ref = {n: getattr(L, n).clone() for n in names}

    def mark():
        for n in names:
            t = getattr(L, n)
            t.fill_(-7 if t.dtype == torch.int32 else float("nan"))

    # warm-up on a side stream, then capture (torch's recipe for graphs)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        L.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    mark()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.step()
    torch.cuda.synchronize()
    junk = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        mark()
        junk.mul_(1.5).sum().item()           # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(getattr(L, n), ref[n]), (rep, n)
    # and the eager step still gives the same bits after the replays
    mark()
    L.step()
    torch.cuda.synchronize()
    for n in names:
        assert torch.equal(getattr(L, n), ref[n]), ("eager", n)
