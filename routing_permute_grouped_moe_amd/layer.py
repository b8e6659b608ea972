"""The MoE expert layer as a sequence of C-ABI calls on one GPU.

This module only allocates device buffers (through torch) and calls the
library entry points in order; every step of the layer runs in the HIP
kernels of ``libmoe.so``.

Forward:  router logits -> route -> permute -> grouped GEMM (+ shared expert)
          -> unpermute/combine.
Backward: combine bwd -> grouped GEMM dX and dW (one call, paired launches)
          -> route bwd -> router bwd -> permute bwd (which also adds the
          shared expert's and the router's input gradients).

The forward runs on one stream: with the grouped GEMM's workspace, the
routed and the shared expert's gate/up and down products are one persistent
launch, which leaves no idle CUs for a second stream to use (a persistent
GEMM holds every CU it gets, and a GEMM workgroup fills its CU's registers).
With ``overlap`` the backward runs the route and router backward on a second
stream of the same priority, beside the grouped GEMM's dX and dW; that
measured within noise of one stream, so it is off by default.  Results are
bitwise identical either way.

With ``shape.capacity`` = C the layer is the drop-and-pad variant: every
expert owns C rows, pairs past an expert's first C (in token order) are
dropped, unfilled rows are zero, and the grouped GEMM runs on the padded
groups.

Experts outside ``[g0, g0+G)`` are remote: their rows are moved by the
permute and the combine, their expert outputs and input gradients are zero
(the buffers are cleared once at allocation and never written), and they get
no weight gradients.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

from . import abi


@dataclass
class LayerShape:
    T: int
    H: int
    I: int
    E: int
    k: int
    dtype: torch.dtype          # torch.bfloat16 or torch.float32
    g0: int = 0
    G: Optional[int] = None     # experts run by the grouped GEMM (None = all E)
    shared: bool = False
    router: bool = True         # False: logits are an input
    capacity: Optional[int] = None   # drop-and-pad: rows per expert (None = dropless)

    @property
    def groups(self) -> int:
        return self.E - self.g0 if self.G is None else self.G

    @property
    def R(self) -> int:
        """Rows of the permuted buffers."""
        return self.T * self.k if self.capacity is None else self.E * self.capacity


class MoeLayer:
    """Device buffers of one layer plus the forward/backward call sequences."""

    def __init__(self, shape: LayerShape, device="cuda", overlap: bool = False,
                 recompute: bool = False):
        s = self.s = shape
        self.overlap = overlap
        # recompute: no permuted copy of x (the grouped GEMMs gather token
        # rows through src_token) and act is recomputed from h13 for dW
        self.recompute = recompute
        dev = self.device = torch.device(device)
        dt, f32, i32 = s.dtype, torch.float32, torch.int32
        self.dt = abi.MOE_BF16 if dt == torch.bfloat16 else abi.MOE_F32
        T, H, I, E, k, R, G = s.T, s.H, s.I, s.E, s.k, s.R, s.groups
        e = lambda *shp, d=dt: torch.empty(shp, dtype=d, device=dev)
        z = lambda *shp, d=dt: torch.zeros(shp, dtype=d, device=dev)
        # parameters / inputs (filled by the caller)
        self.x = e(T, H)
        self.wg = e(H, E, d=f32) if s.router else None
        self.bias = None
        self.logits = e(T, E, d=f32)
        self.w13 = e(G, 2 * I, H)
        self.w2 = e(G, H, I)
        self.ws13 = e(2 * I, H) if s.shared else None
        self.ws2 = e(H, I) if s.shared else None
        self.dy = e(T, H)
        # forward state
        self.idx = e(T, k, d=i32)
        self.gate = e(T, k, d=f32)
        self.xp = None if recompute else e(R, H)
        self.counts = e(E, d=i32)
        self.offsets = e(E + 1, d=i32)
        self.row_id_map = e(T, k, d=i32)
        # load statistics; an EP group is the window of experts one device runs
        self.epg = s.groups if E % s.groups == 0 else E
        self.load = e(E, d=f32)
        self.cv = e(2, d=f32)
        self.group_counts = e(E // self.epg, d=i32)
        self.src_token = e(R, d=i32)
        self.ws_bytes = abi.moe_permute_workspace_bytes(T, E, k)
        self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device=dev)
        self.rws_bytes = abi.moe_router_workspace_bytes(T, H, E, self.dt) if s.router else 0
        self.rws = torch.empty(max(self.rws_bytes, 256), dtype=torch.uint8, device=dev)
        self._wg_split = False
        # tile scheduler counters of the grouped GEMM (zero-filled once; every
        # call leaves them zero); set_gemm_dynamic(False) selects the static order
        self.gws_bytes = abi.moe_gmm_workspace_bytes()
        self.gws = torch.zeros(self.gws_bytes, dtype=torch.uint8, device=dev)
        self.aux = torch.cuda.Stream(device=dev) if overlap else None
        self._ev = [torch.cuda.Event() for _ in range(2)] if overlap else None
        self.h13 = e(R, 2 * I)
        self.act = e(R, I)
        self.yp = z(R, H)            # remote rows stay zero
        self.y = e(T, H)
        if s.shared:
            self.sh_h13 = e(T, 2 * I)
            self.sh_act = e(T, I)
            self.ys = e(T, H)
        # backward state
        self.dyp = e(R, H)
        self.dgate = e(T, k, d=f32)
        self.dh13 = e(R, 2 * I)
        self.dxp = z(R, H)           # remote rows stay zero
        self.dw13 = e(G, 2 * I, H)
        self.dw2 = e(G, H, I)
        self.dlogits = e(T, E, d=f32)
        self.dx = e(T, H)
        if s.router:
            self.dx_router = e(T, H)
            self.dwg = e(H, E, d=f32)
            self.dbias = e(E, d=f32)
        if s.shared:
            self.sh_dh13 = e(T, 2 * I)
            self.sh_dx = e(T, H)
            self.dws13 = e(2 * I, H)
            self.dws2 = e(H, I)

    # ------------------------------------------------------------------ helpers
    def set_gemm_dynamic(self, on: bool = True):
        """Grouped GEMM tiles from per-XCD counters (True) or a fixed share (False)."""
        if on:
            self.gws_bytes = abi.moe_gmm_workspace_bytes()
            self.gws = torch.zeros(self.gws_bytes, dtype=torch.uint8, device=self.device)
        else:
            self.gws_bytes, self.gws = 0, None

    def shared_desc(self):
        if not self.s.shared:
            return None
        return abi.shared_expert(
            T=self.s.T, x=self.x, w13=self.ws13, w2=self.ws2, h13=self.sh_h13, act=self.sh_act,
            y=self.ys, dy=self.dy, dh13=self.sh_dh13, dx=self.sh_dx, dw13=self.dws13,
            dw2=self.dws2)

    # ------------------------------------------------------------------ steps
    def router_fwd(self, stream=None):
        s = self.s
        abi.moe_router_logits(self.x, self.dt, self.wg, self.bias, s.T, s.H, s.E, self.logits,
                              self.rws, self.rws_bytes, stream)
        self._wg_split = True    # the router workspace now holds wg's split

    def route(self, stream=None):
        s = self.s
        abi.moe_route(self.logits, s.T, s.E, s.k, self.idx, self.gate, stream)

    def permute(self, stream=None):
        s = self.s
        if s.capacity is not None:
            abi.moe_permute_capacity(self.x, self.dt, self.idx, s.T, s.H, s.E, s.k, s.capacity,
                                     self.xp, self.counts, self.offsets, self.row_id_map,
                                     self.src_token, self.ws, self.ws_bytes, stream)
            return
        abi.moe_permute(self.x, self.dt, self.idx, s.T, s.H, s.E, s.k, self.xp, self.counts,
                        self.offsets, self.row_id_map, self.src_token, self.ws, self.ws_bytes,
                        stream)

    def load_stats(self, stream=None):
        abi.moe_load_stats(self.counts, self.s.E, self.epg, self.load, self.cv, self.group_counts,
                           stream)

    def saved_bytes(self) -> int:
        """Bytes of activations kept from the forward for the backward (beyond
        the layer input, the weights and the routing maps)."""
        b = self.x.element_size()
        s = self.s
        n = s.R * 2 * s.I + (s.T * 2 * s.I if s.shared else 0)        # h13
        if not self.recompute:
            n += s.R * s.H + s.R * s.I + (s.T * s.I if s.shared else 0)  # xp, act
        return n * b

    def _gmm_sel(self):
        """(G, shared descriptor, workspace) of the grouped-GEMM calls."""
        return self.s.groups, self.shared_desc(), self.gws

    def gmm_fwd(self, stream=None):
        s = self.s
        G, sh, ws = self._gmm_sel()
        if self.recompute:
            abi.moe_grouped_gemm_fwd_gather(self.x, self.src_token, s.T, self.offsets, s.g0, G,
                                            s.R, self.dt, s.H, s.I, self.w13, self.w2, self.h13,
                                            self.act, self.yp, sh, ws, self.gws_bytes, stream)
            return
        abi.moe_grouped_gemm_fwd(self.xp, self.offsets, s.g0, G, s.R, self.dt, s.H, s.I,
                                 self.w13, self.w2, self.h13, self.act, self.yp, sh, ws,
                                 self.gws_bytes, stream)

    def combine(self, stream=None):
        s = self.s
        abi.moe_unpermute_combine(self.yp, self.row_id_map, self.gate,
                                  self.ys if s.shared else None, self.dt, s.T, s.H, s.k, s.R,
                                  self.y, stream)

    def combine_bwd(self, stream=None):
        s = self.s
        abi.moe_unpermute_combine_bwd(self.dy, self.yp, self.row_id_map, self.gate, self.dt, s.T,
                                      s.H, s.k, s.R, self.dyp, self.dgate, stream)
        if s.capacity is not None:   # padded rows of dyp: exact zeros through dX and dW
            abi.moe_clear_empty_rows(self.src_token, s.R, self.dt, s.H, self.dyp, stream)

    def gmm_bwd_dx(self, stream=None):
        s = self.s
        G, sh, ws = self._gmm_sel()
        abi.moe_grouped_gemm_bwd_dx(self.dyp, self.offsets, s.g0, G, s.R, self.dt, s.H, s.I,
                                    self.w13, self.w2, self.h13, self.dh13, self.dxp, sh, ws,
                                    self.gws_bytes, stream)

    def gmm_bwd_dw(self, stream=None):
        s = self.s
        G, sh, ws = self._gmm_sel()
        if self.recompute:
            abi.moe_grouped_gemm_bwd_dw_recompute(self.x, self.src_token, s.T, self.h13, self.act,
                                                  self.dyp, self.dh13, self.offsets, s.g0, G,
                                                  s.R, self.dt, s.H, s.I, self.dw13, self.dw2,
                                                  sh, ws, self.gws_bytes, stream)
            return
        abi.moe_grouped_gemm_bwd_dw(self.xp, self.act, self.dyp, self.dh13, self.offsets, s.g0,
                                    G, s.R, self.dt, s.H, s.I, self.dw13, self.dw2, sh, ws,
                                    self.gws_bytes, stream)

    def gmm_bwd(self, stream=None):
        """dX and dW in one call (paired launches); the recompute variant
        keeps its two calls (dW recomputes act and gathers x)."""
        if self.recompute:
            self.gmm_bwd_dx(stream)
            self.gmm_bwd_dw(stream)
            return
        s = self.s
        G, sh, ws = self._gmm_sel()
        abi.moe_grouped_gemm_bwd(self.xp, self.act, self.dyp, self.offsets, s.g0, G, s.R, self.dt,
                                 s.H, s.I, self.w13, self.w2, self.h13, self.dh13, self.dxp,
                                 self.dw13, self.dw2, sh, ws, self.gws_bytes, stream)

    def route_bwd(self, stream=None):
        s = self.s
        abi.moe_route_bwd(self.logits, self.idx, self.dgate, s.T, s.E, s.k, self.dlogits, stream)

    def router_bwd(self, stream=None):
        """Reuses the split of wg that router_fwd left in the router
        workspace (the step order: wg does not change between the two)."""
        s = self.s
        flags = abi.MOE_ROUTER_WG_SPLIT if self._wg_split else 0
        abi.moe_router_logits_bwd(self.dlogits, self.x, self.dt, self.wg, s.T, s.H, s.E,
                                  self.dx_router, self.dwg, self.dbias, self.rws, self.rws_bytes,
                                  stream, flags=flags)

    def permute_bwd(self, stream=None):
        s = self.s
        abi.moe_permute_bwd(self.dxp, self.row_id_map, self.dt, s.T, s.H, s.k, s.R,
                            self.sh_dx if s.shared else None,
                            self.dx_router if s.router else None, self.dx, stream)

    # ------------------------------------------------------------------ passes
    def _streams(self, stream):
        main = torch.cuda.current_stream(self.device) if stream is None else stream
        return main, self.aux

    def forward(self, stream=None):
        s = self.s
        if s.router:
            self.router_fwd(stream)
        self.route(stream)
        self.permute(stream)
        self.load_stats(stream)
        self.gmm_fwd(stream)
        self.combine(stream)

    def backward(self, stream=None):
        s = self.s
        if self.overlap and s.router:
            main, aux = self._streams(stream)
            ev_c, ev_aux = self._ev[0], self._ev[1]
            self.combine_bwd(main)
            ev_c.record(main)
            aux.wait_event(ev_c)
            self.route_bwd(aux)                         # needs dgate
            self.router_bwd(aux)
            ev_aux.record(aux)
            self.gmm_bwd(main)
            main.wait_event(ev_aux)
            self.permute_bwd(main)
            return
        self.combine_bwd(stream)
        self.gmm_bwd(stream)
        self.route_bwd(stream)
        if s.router:
            self.router_bwd(stream)
        self.permute_bwd(stream)

    def step(self, stream=None):
        self.forward(stream)
        self.backward(stream)
