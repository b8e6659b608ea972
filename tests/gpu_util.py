"""Helpers shared by the GPU tests: compare tensors; the input upload lives
in ``synth.device`` (shared with the benchmark)."""
from __future__ import annotations

import numpy as np
import torch

from synth.device import dev, make_layer, shape_of, torch_dtype  # noqa: F401


def have_gpu() -> bool:
    return torch.cuda.is_available()


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
