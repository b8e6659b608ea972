"""Helpers shared by the GPU tests: upload seeded inputs, compare tensors."""
from __future__ import annotations

import numpy as np
import torch

import synth


def have_gpu() -> bool:
    return torch.cuda.is_available()


def torch_dtype(cfg: synth.MoeConfig):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def dev(a: np.ndarray, dtype) -> torch.Tensor:
    """numpy (fp32 values, bf16-exact for bf16 storage) -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device="cuda").to(dtype)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def rel_err(gpu, ref) -> float:
    """max|gpu - ref| / max|ref| (0 when both are zero)."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    scale = np.abs(r).max() if r.size else 0.0
    diff = np.abs(g - r).max() if r.size else 0.0
    if scale == 0.0:
        return float(diff)
    return float(diff / scale)


def shape_of(cfg: synth.MoeConfig, capacity=None):
    from routing_permute_grouped_moe_amd.layer import LayerShape
    return LayerShape(T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, k=cfg.k, dtype=torch_dtype(cfg),
                      g0=cfg.g0, G=cfg.G, shared=cfg.shared, router=cfg.router,
                      capacity=capacity)


def make_layer(cfg: synth.MoeConfig, inp: synth.Inputs, overlap: bool = True,
               recompute: bool = False, capacity=None):
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
