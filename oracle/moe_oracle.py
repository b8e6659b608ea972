"""Plain CPU oracle of the single-GPU MoE expert layer, forward and backward.

TEST INFRASTRUCTURE.  This module is the slow, obviously correct statement of
what the layer computes.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may use it; the HIP library shares no code with it.

Sources (the web pages this project follows; cited by title and section):

* [CANN-MoE]   "MoE算子优化：动态路由硬件加速与零拷贝通信实践" (gtnt.cn):
  s2.1 routing is Softmax -> Top-k selection -> mask generation;
  s2.2 an expert is a stack of fully-connected layers;
  s4.2 the router network is kept in FP32;
  s4.3 a load-balancing term, 0.01 times the coefficient of variation of the
  experts' loads, is added to the loss.
* [MoE-ops]    Huawei MoE training operator article (feedman.me): the
  VectorSort section (Fig. 3) names the reorder and anti-reorder of tokens
  around the expert matmuls; the Host-Device section (Fig. 4) removes the host
  wait on the token-dispatch preprocessing (per-expert counts).
* [Pangu-QA]   QbitAI article on the Pangu Ultra MoE technical report
  (rjtj.cn): "MoE training analysis" (dropless beats drop-and-pad and was
  adopted), the parallel-overlap part (expert backward split into dW and dX),
  "Experimental results" (the layer output is a weighted sum of the shared
  expert's and the routed experts' contributions).
* [MindSpore-DSv3] "昇思MindSpore助力天翼云提供极致MoE大模型训练性能"
  (mindspore.cn): 01.1 tokens are sorted inside a machine before AlltoAll;
  03.3 GroupedMatmul (GMM) runs all experts' matmuls as one operator.

Readings where the pages are silent (each one is also listed in the design
notes of the repository):

1. gates are the full-softmax probabilities of the chosen experts, not
   renormalised over the top-k;
2. top-k is taken on the fp32 logits (same set as on the probabilities since
   exp is monotone), ties to the lower expert index, slots in descending score;
3. the rows of one expert group keep token order (a stable sort by expert);
4. the expert FFN is SwiGLU without biases: W13[e] = [gate rows; up rows]
   [2I,H], W2[e] [H,I], ``a = silu(x W_gate^T) * (x W_up^T)``, ``y = a W2^T``;
5. the shared expert enters the combine with weight 1;
6. dropless: every one of the T*k (token, slot) pairs gets a row;
7. experts outside the window ``[g0, g0+G)`` are remote: their rows are moved
   by permute/combine but their expert output (and its input gradient) is zero
   and they get no weight gradient;
8. an expert's load is its share of the T*k rows, cv is the population
   standard deviation over the mean, an EP group is a run of consecutive
   experts;
9. drop-and-pad (the variant the pages compare dropless with): capacity
   C = ceil(factor * T*k / E) rows per expert, an expert keeps its first C
   pairs in token order, dropped pairs contribute nothing, empty rows are
   zero.

Precision: every function computes in the dtype ``acc`` it is given (float64
by default).  Router logits are rounded to fp32 because [CANN-MoE] s4.2 keeps
the router in FP32.  Large bf16 configurations may pass ``acc=np.float32``:
products of bf16 values are exact in fp32, only the summation rounds.
"""
from __future__ import annotations

from typing import Callable, Optional, Sequence, Union

import numpy as np

__all__ = [
    "router_logits", "softmax", "route", "permute", "silu", "expert_forward",
    "grouped_forward", "combine", "combine_backward", "expert_backward",
    "grouped_backward", "permute_backward", "route_backward",
    "router_backward", "layer_forward", "layer_backward", "load_stats",
    "capacity", "permute_capacity",
]

WeightSource = Union[np.ndarray, Callable[[int], np.ndarray]]


def _weight(src: WeightSource, g: int) -> np.ndarray:
    return src(g) if callable(src) else src[g]


# --------------------------------------------------------------------------
# forward


def router_logits(x: np.ndarray, wg: np.ndarray, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """``logits = x Wg + bias``: computed in fp64, rounded to fp32 ([CANN-MoE] s4.2)."""
    out = np.asarray(x, np.float64) @ np.asarray(wg, np.float64)
    if bias is not None:
        out = out + np.asarray(bias, np.float64)[None, :]
    return out.astype(np.float32)


def softmax(logits: np.ndarray, acc=np.float64) -> np.ndarray:
    """Row softmax with the row maximum subtracted first."""
    l = np.asarray(logits, acc)
    z = np.exp(l - l.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def route(logits: np.ndarray, k: int, acc=np.float64):
    """Softmax -> top-k -> selection mask ([CANN-MoE] s2.1).

    Returns ``idx`` [T,k] int32 (descending fp32 logit, ties to the lower
    expert index) and ``gate`` [T,k] = softmax probability of each chosen
    expert, computed from the logits as given (fp32 in the layer).
    """
    key = np.asarray(logits, np.float32)
    T, E = key.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    p = softmax(logits, acc)
    # lexsort: the last key is the primary one -> (-logit, expert index)
    experts = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((experts, -key), axis=-1)
    idx = order[:, :k].astype(np.int32)
    gate = np.take_along_axis(p, idx, axis=-1)
    return idx, gate


def permute(x: np.ndarray, idx: np.ndarray, E: int):
    """Sort the T*k (token, slot) pairs into contiguous per-expert groups.

    ``counts[e]`` is the number of pairs routed to e, ``offsets`` its exclusive
    scan (``offsets[E] = T*k``), ``row_id_map[t,j]`` the row that pair (t,j)
    occupies, ``src_token[row]`` the token a row came from, and
    ``xp[row] = x[src_token[row]]`` (the reorder of [MoE-ops], VectorSort,
    Fig. 3).  Rows of one group keep token order (reading 3).
    """
    T, k = idx.shape
    counts = np.zeros(E, np.int64)
    for t in range(T):
        for j in range(k):
            counts[idx[t, j]] += 1
    offsets = np.zeros(E + 1, np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    next_row = offsets[:E].copy()
    row_id_map = np.empty((T, k), np.int64)
    src_token = np.empty(T * k, np.int64)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            row_id_map[t, j] = next_row[e]
            src_token[next_row[e]] = t
            next_row[e] += 1
    xp = x[src_token]
    return xp, counts, offsets, row_id_map, src_token


def capacity(T: int, k: int, E: int, factor: float) -> int:
    """Rows per expert of the drop-and-pad variant: ``ceil(factor * T*k / E)``
    ([CANN-MoE] s4.3 sets a capacity factor of 1.2; the pages give no
    formula, this is the reading in which factor 1 is the mean load)."""
    return int(np.ceil(factor * T * k / E))


def permute_capacity(x: np.ndarray, idx: np.ndarray, E: int, C: int):
    """Drop-and-pad permute ([CANN-MoE] s4.3 capacity factor; [Pangu-QA] MoE
    training analysis compares it with dropless): expert e owns rows
    ``[e*C, (e+1)*C)``; its first C pairs in token order keep a row, the rest
    are dropped (``row_id_map = -1``); rows nobody fills are zero
    (``src_token = -1``).  ``counts[e]`` counts every pair routed to e,
    dropped or not; ``offsets[e] = e*C``.
    """
    T, k = idx.shape
    counts = np.zeros(E, np.int64)
    row_id_map = np.full((T, k), -1, np.int64)
    src_token = np.full(E * C, -1, np.int64)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            rank = counts[e]
            counts[e] += 1
            if rank < C:
                row_id_map[t, j] = e * C + rank
                src_token[e * C + rank] = t
    offsets = np.arange(E + 1, dtype=np.int64) * C
    xp = np.zeros((E * C,) + x.shape[1:], x.dtype)
    kept = src_token >= 0
    xp[kept] = x[src_token[kept]]
    return xp, counts, offsets, row_id_map, src_token


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def expert_forward(xr: np.ndarray, w13: np.ndarray, w2: np.ndarray, acc=np.float64):
    """One SwiGLU expert on its rows (reading 4). Returns (h13, act, y)."""
    xr = np.asarray(xr, acc)
    w13 = np.asarray(w13, acc)
    w2 = np.asarray(w2, acc)
    I = w2.shape[1]
    g = xr @ w13[:I].T
    u = xr @ w13[I:].T
    act = silu(g) * u
    return np.concatenate([g, u], axis=1), act, act @ w2.T


def grouped_forward(xp: np.ndarray, offsets: np.ndarray, w13: WeightSource, w2: WeightSource,
                    g0: int = 0, G: Optional[int] = None, acc=np.float64):
    """GroupedMatmul SwiGLU over the groups ``[g0, g0+G)`` ([MindSpore-DSv3] 03.3).

    Rows of other groups (remote experts, reading 7) get zero outputs.
    ``w13``/``w2`` are indexed by ``g - g0`` (arrays or callables)."""
    R, H = xp.shape
    E = len(offsets) - 1
    G = E - g0 if G is None else G
    I = _weight(w2, 0).shape[1]
    h13 = np.zeros((R, 2 * I), acc)
    act = np.zeros((R, I), acc)
    yp = np.zeros((R, H), acc)
    for g in range(G):
        lo, hi = int(offsets[g0 + g]), int(offsets[g0 + g + 1])
        if hi == lo:
            continue
        h13[lo:hi], act[lo:hi], yp[lo:hi] = expert_forward(
            xp[lo:hi], _weight(w13, g), _weight(w2, g), acc)
    return h13, act, yp


def combine(yp: np.ndarray, row_id_map: np.ndarray, gate: np.ndarray,
            y_shared: Optional[np.ndarray] = None, acc=np.float64) -> np.ndarray:
    """Anti-reorder and weighted sum: ``y[t] = ys[t] + sum_j gate[t,j] yp[row(t,j)]``
    ([MoE-ops] VectorSort; [Pangu-QA] experimental results, shared weight 1).
    A dropped pair (row -1, drop-and-pad variant) adds nothing."""
    T, k = row_id_map.shape
    y = np.zeros((T, yp.shape[1]), acc) if y_shared is None else np.array(y_shared, acc)
    for j in range(k):
        rows = row_id_map[:, j]
        keep = rows >= 0
        y[keep] += np.asarray(gate[keep, j], acc)[:, None] * np.asarray(yp[rows[keep]], acc)
    return y


# --------------------------------------------------------------------------
# backward


def combine_backward(dy: np.ndarray, yp: np.ndarray, row_id_map: np.ndarray,
                     gate: np.ndarray, acc=np.float64):
    """``dyp[row(t,j)] = gate[t,j] dy[t]``, ``dgate[t,j] = <dy[t], yp[row(t,j)]>``;
    a dropped pair (row -1) gets dgate 0 and no row."""
    T, k = row_id_map.shape
    dy = np.asarray(dy, acc)
    dyp = np.zeros((yp.shape[0], dy.shape[1]), acc)
    dgate = np.zeros((T, k), acc)
    for j in range(k):
        rows = row_id_map[:, j]
        keep = rows >= 0
        dyp[rows[keep]] = np.asarray(gate[keep, j], acc)[:, None] * dy[keep]
        dgate[keep, j] = np.einsum("th,th->t", dy[keep], np.asarray(yp[rows[keep]], acc))
    return dyp, dgate


def expert_backward(xr: np.ndarray, w13: np.ndarray, w2: np.ndarray, dyr: np.ndarray,
                    acc=np.float64):
    """Backward of one SwiGLU expert, split into the input gradient (dX) and
    the weight gradients (dW) as [Pangu-QA] separates them.

    Returns (dh13, dx, dw13, dw2)."""
    xr = np.asarray(xr, acc)
    w13 = np.asarray(w13, acc)
    w2 = np.asarray(w2, acc)
    dyr = np.asarray(dyr, acc)
    I = w2.shape[1]
    g = xr @ w13[:I].T
    u = xr @ w13[I:].T
    act = silu(g) * u
    da = dyr @ w2                                   # d act
    sig = 1.0 / (1.0 + np.exp(-g))
    dg = da * u * sig * (1.0 + g * (1.0 - sig))     # d silu(g)/dg = sig (1 + g (1 - sig))
    du = da * (g * sig)
    dh13 = np.concatenate([dg, du], axis=1)
    dx = dh13 @ w13
    dw2 = dyr.T @ act
    dw13 = dh13.T @ xr
    return dh13, dx, dw13, dw2


def grouped_backward(xp: np.ndarray, dyp: np.ndarray, offsets: np.ndarray,
                     w13: WeightSource, w2: WeightSource, g0: int = 0,
                     G: Optional[int] = None, acc=np.float64, weight_grads: bool = True):
    """Backward of :func:`grouped_forward`.

    Returns (dh13, dxp, dw13 [G,2I,H], dw2 [G,H,I]); an empty group's weight
    gradients are exactly zero; remote rows get ``dxp = 0``."""
    R, H = xp.shape
    E = len(offsets) - 1
    G = E - g0 if G is None else G
    I = _weight(w2, 0).shape[1]
    dh13 = np.zeros((R, 2 * I), acc)
    dxp = np.zeros((R, H), acc)
    dw13 = np.zeros((G, 2 * I, H), acc) if weight_grads else None
    dw2 = np.zeros((G, H, I), acc) if weight_grads else None
    for g in range(G):
        lo, hi = int(offsets[g0 + g]), int(offsets[g0 + g + 1])
        if hi == lo:
            continue
        a, b, c, d = expert_backward(xp[lo:hi], _weight(w13, g), _weight(w2, g), dyp[lo:hi], acc)
        dh13[lo:hi], dxp[lo:hi] = a, b
        if weight_grads:
            dw13[g], dw2[g] = c, d
    return dh13, dxp, dw13, dw2


def permute_backward(dxp: np.ndarray, row_id_map: np.ndarray, acc=np.float64) -> np.ndarray:
    """``dx[t] = sum_j dxp[row(t,j)]`` (the adjoint of the row copy); dropped
    pairs (row -1) add nothing."""
    T, k = row_id_map.shape
    dx = np.zeros((T, dxp.shape[1]), acc)
    for j in range(k):
        rows = row_id_map[:, j]
        keep = rows >= 0
        dx[keep] += np.asarray(dxp[rows[keep]], acc)
    return dx


def route_backward(logits: np.ndarray, idx: np.ndarray, dgate: np.ndarray,
                   acc=np.float64) -> np.ndarray:
    """Gradient through the gate values only (the selection has none):
    ``dlogits = p * (dp - sum_e p_e dp_e)`` with ``dp`` = dgate at the chosen
    experts and 0 elsewhere."""
    p = softmax(logits, acc)
    T, E = p.shape
    dp = np.zeros((T, E), acc)
    for j in range(idx.shape[1]):
        dp[np.arange(T), idx[:, j]] += np.asarray(dgate[:, j], acc)
    s = (p * dp).sum(axis=1, keepdims=True)
    return p * (dp - s)


def router_backward(dlogits: np.ndarray, x: np.ndarray, wg: np.ndarray, acc=np.float64):
    """Backward of ``x Wg + b``: (dx, dWg, dbias)."""
    dl = np.asarray(dlogits, acc)
    return dl @ np.asarray(wg, acc).T, np.asarray(x, acc).T @ dl, dl.sum(axis=0)


# --------------------------------------------------------------------------
# routing statistics


def load_stats(counts: np.ndarray, experts_per_group: int = 1):
    """Per-expert load and its spread, from the permute's histogram.

    [CANN-MoE] s4.3 adds a balance term ``0.01 * cv(experts_load)`` to the
    loss; [Pangu-QA] "MoE training analysis" balances per EP group and plans
    expert placement from the experts' observed loads.  Readings (the pages
    define none of these): ``load[e] = counts[e] / sum(counts)``; cv is the
    population standard deviation over the mean (divide by the number of
    experts, not one less); EP group g holds the experts
    ``[g*epg, (g+1)*epg)``.  Returns ``(load [E], cv_experts, group_counts
    [E/epg], cv_groups)``; cv is 0 when every count is 0.
    """
    c = np.asarray(counts, np.int64)
    E = c.shape[0]
    if E % experts_per_group:
        raise ValueError("experts_per_group must divide E")
    total = int(c.sum())
    load = c.astype(np.float64) / total if total else np.zeros(E)

    def cv(v):
        v = np.asarray(v, np.float64)
        mean = v.mean()
        if mean == 0:
            return 0.0
        return float(np.sqrt(((v - mean) ** 2).mean()) / mean)

    groups = c.reshape(E // experts_per_group, experts_per_group).sum(axis=1)
    return load, cv(c), groups, cv(groups)


# --------------------------------------------------------------------------
# whole layer


def layer_forward(x, k: int, E: int, w13: WeightSource, w2: WeightSource,
                  wg=None, bias=None, logits=None, g0: int = 0, G: Optional[int] = None,
                  ws13=None, ws2=None, acc=np.float64, C: Optional[int] = None) -> dict:
    """Route -> permute -> grouped SwiGLU -> unpermute/combine (+ shared expert).

    Either ``wg`` (router weights) or ``logits`` must be given.  ``C`` (rows
    per expert) selects the drop-and-pad variant; None is dropless."""
    if logits is None:
        logits = router_logits(x, wg, bias)
    idx, gate = route(logits, k, acc)
    if C is None:
        xp, counts, offsets, row_id_map, src_token = permute(x, idx, E)
    else:
        xp, counts, offsets, row_id_map, src_token = permute_capacity(x, idx, E, C)
    h13, act, yp = grouped_forward(xp, offsets, w13, w2, g0, G, acc)
    ys = None
    if ws13 is not None:
        ys = expert_forward(x, ws13, ws2, acc)[2]
    y = combine(yp, row_id_map, gate, ys, acc)
    return dict(logits=logits, idx=idx, gate=gate, xp=xp, counts=counts, offsets=offsets,
                row_id_map=row_id_map, src_token=src_token, h13=h13, act=act, yp=yp,
                ys=ys, y=y)


def layer_backward(fwd: dict, dy, x, w13: WeightSource, w2: WeightSource, wg=None,
                   g0: int = 0, G: Optional[int] = None, ws13=None, ws2=None,
                   acc=np.float64) -> dict:
    """Backward of :func:`layer_forward` given the upstream gradient ``dy``."""
    dyp, dgate = combine_backward(dy, fwd["yp"], fwd["row_id_map"], fwd["gate"], acc)
    dh13, dxp, dw13, dw2 = grouped_backward(fwd["xp"], dyp, fwd["offsets"], w13, w2, g0, G, acc)
    dx = permute_backward(dxp, fwd["row_id_map"], acc)
    out = dict(dyp=dyp, dgate=dgate, dh13=dh13, dxp=dxp, dw13=dw13, dw2=dw2)
    if ws13 is not None:
        dh13s, dxs, dws13, dws2 = expert_backward(x, ws13, ws2, dy, acc)
        dx = dx + dxs
        out.update(dh13_shared=dh13s, dx_shared=dxs, dws13=dws13, dws2=dws2)
    dlogits = route_backward(fwd["logits"], fwd["idx"], dgate, acc)
    out["dlogits"] = dlogits
    if wg is not None:
        dxr, dwg, dbias = router_backward(dlogits, x, wg, acc)
        dx = dx + dxr
        out.update(dx_router=dxr, dwg=dwg, dbias=dbias)
    out["dx"] = dx
    return out
