"""Seeded synthetic inputs for the MoE expert layer.

This module is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark.  It holds no arithmetic of the layer itself: it only draws
seeded normal variates, scales them, and rounds them to bf16 where a config
stores tensors in bf16.  Neither the oracle nor the HIP library imports it;
callers pass its arrays to one or the other.

Recipe (one numpy ``SeedSequence([seed, stream, i])`` per tensor, always
``standard_normal(dtype=float32)`` and then scaled):

====== ======================= ============================================
stream tensor                  recipe
====== ======================= ============================================
0      x          [T,H]        N(0,1)
1      Wg         [H,E]        x0.02, kept fp32
2      router bias [E]         normal: x0.5; zipf(a): rank r = permutation
                               of 1..E, bias = -a*ln(r)
3, e   W13[e]     [2I,H]       x0.02 (rows 0..I-1 gate, I..2I-1 up)
4, e   W2[e]      [H,I]        x0.02
5      dY         [T,H]        N(0,1)
6, 7   shared W13, W2          x0.02
8      logits     [T,E]        N(0,1) (configs that skip the router)
====== ======================= ============================================

Shapes come from the pages: the Pangu Ultra MoE shape (hidden 7680, 256
routed experts + 1 shared expert, expert hidden 2048) is given by the
reportify.cn summaries of the Pangu Ultra MoE reports; DeepSeek-V3's 256
experts by the MindSpore/China Telecom Cloud article, section 01.1.  The
remaining sizes (token counts, top-k, the DeepSeek and small-config widths)
are the fixed benchmark configurations of this project.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

__all__ = [
    "MoeConfig", "CONFIGS", "get_config", "rng", "bf16_round", "bf16_bits",
    "bits_to_f32", "Inputs", "make_inputs", "expert_w13", "expert_w2",
]


@dataclasses.dataclass(frozen=True)
class MoeConfig:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    dtype: str                 # "f32" or "bf16": storage type of x, weights, dY
    bias: str                  # "none", "normal", "zipf"
    bias_param: float = 0.0    # std for "normal", alpha for "zipf"
    router: bool = True        # False: logits are drawn directly (stream 8)
    g0: int = 0                # first expert run by the grouped GEMM
    G: Optional[int] = None    # number of experts run by the grouped GEMM (None = all)
    shared: bool = False       # one always-on shared expert of width I
    description: str = ""

    @property
    def groups(self) -> int:
        return self.E if self.G is None else self.G

    @property
    def R(self) -> int:
        return self.T * self.k


CONFIGS = {
    "tiny": MoeConfig("tiny", 256, 128, 64, 8, 2, "f32", "none",
                      description="tiny fp32 oracle case"),
    "small": MoeConfig("small", 4096, 2048, 1408, 64, 6, "bf16", "normal", 0.5,
                       description="small bf16 fwd+bwd, mild skew"),
    "pangu": MoeConfig("pangu", 8192, 7680, 2048, 256, 8, "bf16", "zipf", 1.1,
                       g0=0, G=8, shared=True,
                       description="Pangu-Ultra-shaped one-device share: 8 local experts + shared"),
    "deepseek": MoeConfig("deepseek", 4096, 7168, 2048, 256, 8, "bf16", "zipf", 1.2,
                          description="DeepSeek-V3-shaped full layer, heavy skew"),
    "stress": MoeConfig("stress", 16384, 7680, 256, 256, 8, "bf16", "none", router=False,
                        description="small-expert stress, logits drawn directly"),
    # the per-device shape of the Pangu layer under expert parallelism after
    # the all-to-all, with balanced peers: the 8 local experts receive T*k
    # rows in all, T each (every token picks all 8 experts here, which gives
    # exactly those group sizes), plus the shared expert on the T tokens
    # (logits drawn directly: the router of that deployment runs over all
    # 256 experts before the all-to-all, as in the pangu config)
    "pangu_received": MoeConfig("pangu_received", 8192, 7680, 2048, 8, 8, "bf16", "none",
                                router=False, shared=True,
                                description="Pangu share as received under balanced EP: "
                                            "8 local experts x T rows + shared, logits drawn "
                                            "directly"),
}


def get_config(name: str, **overrides) -> MoeConfig:
    cfg = CONFIGS[name]
    return dataclasses.replace(cfg, **overrides) if overrides else cfg


def rng(seed: int, stream: int, i: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, stream, i]))


def _normal(seed, stream, i, shape, scale=1.0) -> np.ndarray:
    a = rng(seed, stream, i).standard_normal(int(np.prod(shape)), dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return a.reshape(shape)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """IEEE round-to-nearest-even of fp32 to bf16, returned as uint16 bits.

    Finite inputs only (the generators never produce non-finite values)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    flat_in = a.reshape(-1).view(np.uint32)
    flat_out = out.reshape(-1)
    step = 1 << 20
    for s in range(0, flat_in.size, step):
        # finite values stay below 2**32 after adding at most 0x8000
        u = flat_in[s:s + step].copy()
        lsb = (u >> 16) & 1
        u += 0x7FFF
        u += lsb
        u >>= 16
        flat_out[s:s + step] = u
    return out


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """fp32 array holding the bf16-rounded values of ``a``."""
    return bits_to_f32(bf16_bits(a))


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round to the config's storage type; returns fp32 values (bf16-exact for bf16)."""
    return bf16_round(a) if dtype == "bf16" else a


def router_bias(cfg: MoeConfig, seed: int = 0) -> Optional[np.ndarray]:
    if not cfg.router or cfg.bias == "none":
        return None
    if cfg.bias == "normal":
        return _normal(seed, 2, 0, (cfg.E,), cfg.bias_param)
    if cfg.bias == "zipf":
        r = rng(seed, 2, 0).permutation(cfg.E).astype(np.float64) + 1.0
        return (-cfg.bias_param * np.log(r)).astype(np.float32)
    raise ValueError(cfg.bias)


def expert_w13(cfg: MoeConfig, e: int, seed: int = 0) -> np.ndarray:
    """W13[e] [2I,H] (gate rows then up rows), in fp32 holding storage-type values."""
    return _store(_normal(seed, 3, e, (2 * cfg.I, cfg.H), 0.02), cfg.dtype)


def expert_w2(cfg: MoeConfig, e: int, seed: int = 0) -> np.ndarray:
    return _store(_normal(seed, 4, e, (cfg.H, cfg.I), 0.02), cfg.dtype)


def shared_w13(cfg: MoeConfig, seed: int = 0) -> np.ndarray:
    return _store(_normal(seed, 6, 0, (2 * cfg.I, cfg.H), 0.02), cfg.dtype)


def shared_w2(cfg: MoeConfig, seed: int = 0) -> np.ndarray:
    return _store(_normal(seed, 7, 0, (cfg.H, cfg.I), 0.02), cfg.dtype)


@dataclasses.dataclass
class Inputs:
    cfg: MoeConfig
    x: np.ndarray                      # [T,H] fp32 (bf16-exact for bf16 configs)
    wg: Optional[np.ndarray]           # [H,E] fp32 (None if the router is skipped)
    bias: Optional[np.ndarray]         # [E] fp32 or None
    logits: Optional[np.ndarray]       # [T,E] fp32, only when the router is skipped
    w13: Optional[np.ndarray]          # [G,2I,H] or None when not materialised
    w2: Optional[np.ndarray]           # [G,H,I]
    dy: np.ndarray                     # [T,H]
    ws13: Optional[np.ndarray] = None  # shared expert [2I,H]
    ws2: Optional[np.ndarray] = None   # shared expert [H,I]


def make_inputs(cfg: MoeConfig, seed: int = 0, experts: bool = True,
                threads: int = 8) -> Inputs:
    """Build every input of one config.  ``experts=False`` skips the per-expert
    weights (callers can draw single experts with :func:`expert_w13`)."""
    x = _store(_normal(seed, 0, 0, (cfg.T, cfg.H)), cfg.dtype)
    dy = _store(_normal(seed, 5, 0, (cfg.T, cfg.H)), cfg.dtype)
    if cfg.router:
        wg = _normal(seed, 1, 0, (cfg.H, cfg.E), 0.02)
        logits = None
    else:
        wg = None
        logits = _normal(seed, 8, 0, (cfg.T, cfg.E))
    bias = router_bias(cfg, seed)
    w13 = w2 = None
    if experts:
        G = cfg.groups
        w13 = np.empty((G, 2 * cfg.I, cfg.H), np.float32)
        w2 = np.empty((G, cfg.H, cfg.I), np.float32)

        def fill(g):
            w13[g] = expert_w13(cfg, cfg.g0 + g, seed)
            w2[g] = expert_w2(cfg, cfg.g0 + g, seed)

        with ThreadPoolExecutor(max(1, threads)) as ex:
            list(ex.map(fill, range(G)))
    ws13 = ws2 = None
    if cfg.shared:
        ws13 = shared_w13(cfg, seed)
        ws2 = shared_w2(cfg, seed)
    return Inputs(cfg, x, wg, bias, logits, w13, w2, dy, ws13, ws2)
