"""Upload seeded synthetic inputs into a device-resident MoE layer.

Used by the benchmark, the GPU tests and the smoke run.  It only copies the
arrays ``synth.make_inputs`` drew into the buffers of a
``routing_permute_grouped_moe_amd.layer.MoeLayer`` (torch handles the device
memory); no arithmetic of the layer happens here.
"""
from __future__ import annotations

import numpy as np

from . import Inputs, MoeConfig


def torch_dtype(cfg: MoeConfig):
    import torch
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def dev(a: np.ndarray, dtype):
    """numpy array (fp32 values, bf16-exact for bf16 storage) -> cuda tensor."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device="cuda").to(dtype)


def shape_of(cfg: MoeConfig, capacity=None):
    from routing_permute_grouped_moe_amd.layer import LayerShape
    return LayerShape(T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, k=cfg.k, dtype=torch_dtype(cfg),
                      g0=cfg.g0, G=cfg.G, shared=cfg.shared, router=cfg.router,
                      capacity=capacity)


def make_layer(cfg: MoeConfig, inp: Inputs, overlap: bool = False, recompute: bool = False,
               capacity=None):
    """A ``MoeLayer`` of ``cfg``'s shape holding ``inp``'s parameters and inputs."""
    import torch

    from routing_permute_grouped_moe_amd.layer import MoeLayer
    L = MoeLayer(shape_of(cfg, capacity), overlap=overlap, recompute=recompute)
    dt = torch_dtype(cfg)
    L.x.copy_(dev(inp.x, dt))
    L.dy.copy_(dev(inp.dy, dt))
    if cfg.router:
        L.wg.copy_(dev(inp.wg, torch.float32))
        if inp.bias is not None:
            L.bias = dev(inp.bias, torch.float32)
    else:
        L.logits.copy_(dev(inp.logits, torch.float32))
    L.w13.copy_(dev(inp.w13, dt))
    L.w2.copy_(dev(inp.w2, dt))
    if cfg.shared:
        L.ws13.copy_(dev(inp.ws13, dt))
        L.ws2.copy_(dev(inp.ws2, dt))
    torch.cuda.synchronize()
    return L
