#!/usr/bin/env python3
"""Benchmark: one MoE expert layer forward + backward on one MI355X.

Workload: the Pangu-Ultra-shaped one-device share -- T = 8192 tokens (one
8K sequence), hidden 7680, 256 routed experts with top-8 softmax gating and a
Zipf(1.1) router bias; the grouped GEMM runs the 8 local experts (expert
intermediate 2048, SwiGLU) plus one always-on shared expert (intermediate
2048) on every token.  bf16 storage, fp32 accumulation, fp32 router.
Inputs are seeded synthetic tensors (no dataset), resident in HBM before the
timed region.

A step is the whole path: router projection, route, permute, load statistics, grouped GEMM
forward (+ shared expert), unpermute/combine, combine backward, grouped GEMM
dX and dW (+ shared expert), route backward, router backward, permute
backward.  ``value`` is tokens per second over the timed steps.

Prints one JSON line.  ``--gpus`` above 1 is refused: this build runs on
one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd+bwd tokens/s on 1 GPU; GMM % MFMA peak; permute % HBM BW"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
FLUSH_BYTES = 1 << 30          # scratch read before each call of the per-call breakdown


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", default="pangu")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-variants", action="store_true",
                   help="skip the timing of the recompute variant")
    p.add_argument("--overlap", action="store_true",
                   help="time steps with the route and router backward on a second stream "
                        "(default: every call on one stream, as the per-call breakdown)")
    p.add_argument("--cpu-tokens", type=int, default=8192,
                   help="tokens in the oracle's timed sample")
    p.add_argument("--no-dense-ref", action="store_true",
                   help="skip timing torch.matmul (hipBLASLt) on the dense equivalents and the "
                        "reference HBM copies")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="run one device-to-device copy of this many MiB before the timed "
                        "region (a known-size reference for HBM byte counters)")
    return p.parse_args()


# the calls of one step, in order; the dX and dW products run in one call
# (gmm_bwd); gmm_bwd_dx and gmm_bwd_dw, its two halves as separate calls,
# are timed after the step's calls for reference
CALLS = ["router_fwd", "route", "permute", "load_stats", "gmm_fwd", "combine", "combine_bwd",
         "gmm_bwd", "route_bwd", "router_bwd", "permute_bwd"]
REFERENCE_CALLS = ["gmm_bwd_dx", "gmm_bwd_dw"]


def algorithmic(cfg, rows_local, active_local):
    """Algorithmic flops / bytes per call (routed rows only, no padding).

    An expert's weights are W13 [2I, H] and W2 [H, I]: 3 H I elements, read
    once by the forward and by dX (experts that received rows), written once
    as weight gradients by dW (every expert of the window, empty ones as
    zeros)."""
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    b = 2 if cfg.dtype == "bf16" else 4
    rows = rows_local + (T if cfg.shared else 0)
    gmm_flops = 6.0 * rows * H * I
    sh = 1 if cfg.shared else 0
    w_read = (active_local + sh) * 3.0 * H * I * b
    w_write = (cfg.groups + sh) * 3.0 * H * I * b
    out = {
        "router_fwd": {"flops": 2.0 * T * H * E, "bytes": T * H * b + H * E * 4 + T * E * 4},
        "route": {"bytes": 4.0 * T * E + 8.0 * T * k},
        "permute": {"bytes": (1 + k) * T * H * b + 12.0 * T * k},
        "load_stats": {"bytes": 8.0 * E + 8 + 4.0 * (E // (cfg.groups if E % cfg.groups == 0 else E))},
        "gmm_fwd": {"flops": gmm_flops, "bytes": w_read + rows * (2 * H + 3 * I) * b},
        "combine": {"bytes": (k + 1) * T * H * b + 8.0 * T * k + (T * H * b if cfg.shared else 0)},
        "combine_bwd": {"bytes": T * H * b + 2.0 * T * k * H * b + 12.0 * T * k},
        "gmm_bwd_dx": {"flops": gmm_flops, "bytes": w_read + rows * (2 * H + 4 * I) * b},
        "gmm_bwd_dw": {"flops": gmm_flops, "bytes": w_write + rows * (2 * H + 3 * I) * b},
        "gmm_bwd": {"flops": 2 * gmm_flops,
                    "bytes": w_read + w_write + rows * (4 * H + 7 * I) * b},
        "route_bwd": {"bytes": 8.0 * T * E + 12.0 * T * k},
        "router_bwd": {"flops": 4.0 * T * H * E, "bytes": 2 * T * H * b + H * E * 4 + T * E * 4},
        "permute_bwd": {"bytes": (k + 1) * T * H * b + 4.0 * T * k
                        + (T * H * b if cfg.shared else 0) + (T * H * b if cfg.router else 0)},
    }
    return out


def cpu_baseline(cfg_name, tokens, min_seconds=10.0, max_reps=8):
    """Time the CPU oracle (as it stands) on a bounded sample of the workload:
    the layer fwd+bwd on ``tokens`` tokens, repeated until about
    ``min_seconds`` of CPU work have been timed."""
    import numpy as np

    import oracle
    import synth
    cfg = synth.get_config(cfg_name, T=tokens)
    inp = synth.make_inputs(cfg)
    acc = np.float32 if cfg.dtype == "bf16" else np.float64
    reps, spent, t_fwd, t_bwd = 0, 0.0, 0.0, 0.0
    while reps < max_reps and (reps == 0 or spent < min_seconds):
        t0 = time.perf_counter()
        fwd = oracle.layer_forward(inp.x, cfg.k, cfg.E, inp.w13, inp.w2, wg=inp.wg,
                                   bias=inp.bias, logits=inp.logits, g0=cfg.g0, G=cfg.G,
                                   ws13=inp.ws13, ws2=inp.ws2, acc=acc)
        t1 = time.perf_counter()
        oracle.layer_backward(fwd, inp.dy, inp.x, inp.w13, inp.w2, wg=inp.wg, g0=cfg.g0,
                              G=cfg.G, ws13=inp.ws13, ws2=inp.ws2, acc=acc)
        t2 = time.perf_counter()
        t_fwd += t1 - t0
        t_bwd += t2 - t1
        spent += t2 - t0
        reps += 1
        del fwd
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    cpu_model = platform.processor() or platform.machine()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        deps = np.show_config(mode="dicts")["Build Dependencies"]
        blas = ", ".join(f"{k}: {deps[k].get('name', '?')} {deps[k].get('version', '')}".strip()
                         for k in ("blas", "lapack") if k in deps)
    except Exception:
        blas = "unknown"
    return {"value": tokens * reps / spent, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{cfg_name} layer fwd+bwd on {tokens} tokens (same H/I/E/k and seeds as "
                      f"the workload), numpy "
                      + ("fp32 on bf16 inputs" if cfg.dtype == "bf16" else "fp64") +
                      f", {reps} repetitions, "
                      f"{spent:.1f} s", "seconds": spent, "forward_s_per_rep": t_fwd / reps,
            "backward_s_per_rep": t_bwd / reps, "cpu": cpu_model, "blas": blas}


def dense_reference(cfg, reps=10):
    """The library bar for the grouped GEMM: torch.matmul (hipBLASLt) in bf16
    on the dense products of one expert that receives all T tokens (for the
    Pangu share: exactly the shared expert's six products), operands in the
    layouts the layer stores them in.  Reports TFLOP/s per product and per
    call (the call's two products back to back)."""
    import torch
    T, H, I = cfg.T, cfg.H, cfg.I
    bf = torch.bfloat16
    r = lambda *shp: torch.randn(*shp, device="cuda", dtype=bf)
    x, dy, act, dh13 = r(T, H), r(T, H), r(T, I), r(T, 2 * I)
    w13, w2 = r(2 * I, H), r(H, I)
    prods = {
        "fwd1": (lambda: x @ w13.t(), 2.0 * T * 2 * I * H),     # h13 = x W13^T
        "fwd2": (lambda: act @ w2.t(), 2.0 * T * H * I),        # y = act W2^T
        "dx1": (lambda: dy @ w2, 2.0 * T * I * H),              # dact = dy W2
        "dx2": (lambda: dh13 @ w13, 2.0 * T * H * 2 * I),       # dx = dh13 W13
        "dw2": (lambda: dy.t() @ act, 2.0 * H * I * T),         # dW2 = dy^T act
        "dw13": (lambda: dh13.t() @ x, 2.0 * 2 * I * H * T),    # dW13 = dh13^T x
    }
    ms = {}
    for n, (fn, _) in prods.items():
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms[n] = e0.elapsed_time(e1) / reps
    out = {"what": f"torch.matmul (hipBLASLt) bf16, dense products of one expert on all "
                   f"{T} tokens (H={H}, I={I}), operands in the layer's layouts",
           "products": {n: {"ms": round(ms[n], 4),
                            "tflops": round(f / (ms[n] * 1e-3) / 1e12, 1),
                            "frac_bf16_peak": round(f / (ms[n] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
                        for n, (_, f) in prods.items()}}
    for call, (a, b) in {"gmm_fwd": ("fwd1", "fwd2"), "gmm_bwd_dx": ("dx1", "dx2"),
                         "gmm_bwd_dw": ("dw2", "dw13")}.items():
        t = ms[a] + ms[b]
        tf = 6.0 * T * H * I / (t * 1e-3) / 1e12
        out[call] = {"ms": round(t, 4), "tflops": round(tf, 1),
                     "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)}
    del x, dy, act, dh13, w13, w2
    torch.cuda.empty_cache()
    return out


def hbm_reference(reps=10):
    """Reference HBM rates of plain torch kernels on this GPU, each timed with
    HIP events after the same 1 GiB cache flush as the per-call breakdown: a
    1 GiB device copy (1 GiB read + 1 GiB written) and a 1 GiB fill (write
    only).  The copy gives the practical bar for the permute family, whose
    calls mix reads and writes the same way."""
    import torch
    n = (1 << 30) // 2
    a = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    out = {}
    for name, fn, nbytes in (("copy_1GiB", lambda: b.copy_(a), 2 << 30),
                             ("fill_1GiB", lambda: b.fill_(1.0), 1 << 30)):
        fn()
        ts = []
        for _ in range(reps):
            torch.amax(flush, dim=0, out=sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = sorted(ts)[reps // 2]
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 4), "gbs": round(gbs, 1),
                     "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    del a, b, flush
    torch.cuda.empty_cache()
    return out


def measured_traffic(call):
    """HBM bytes per launch of ``call`` from the committed rocprofv3 byte
    counters, if they were taken on the current kernel source (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic_pangu.json")
    try:
        rec = json.load(open(path))["calls"][call]
        src = os.path.join(ROOT, "routing_permute_grouped_moe_amd", "csrc", rec["source"])
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["source_sha256"]:
            return None
        return rec["hbm_bytes"]
    except (OSError, KeyError, ValueError):
        return None


def variant(L, steps, warmup, recompute=False, capacity=None):
    """Time the same step in a variant of the layer on the same parameters
    and inputs: the recompute variant (no saved xp / act; reports the
    activation bytes each path keeps from the forward for the backward) or
    drop-and-pad with ``capacity`` rows per expert (reports the pairs
    dropped)."""
    import dataclasses

    import numpy as np
    import torch

    from routing_permute_grouped_moe_amd.layer import MoeLayer
    shape = dataclasses.replace(L.s, capacity=capacity)
    B = MoeLayer(shape, overlap=L.overlap, recompute=recompute)
    for n in ("x", "dy", "w13", "w2", "wg", "logits", "ws13", "ws2"):
        if getattr(L, n) is not None:
            getattr(B, n).copy_(getattr(L, n))
    B.bias = L.bias
    for _ in range(warmup):
        B.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        B.step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the calls that differ from the saving path, one stream, HIP events
    calls = ["permute", "gmm_fwd", "gmm_bwd_dw"]
    B.overlap = False
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(calls) * steps)]
    for s in range(steps):
        for i, c in enumerate(calls):
            ev[2 * (s * len(calls) + i)].record(stream)
            getattr(B, c)()
            ev[2 * (s * len(calls) + i) + 1].record(stream)
    torch.cuda.synchronize()
    per_call = {c: round(sum(ev[2 * (s * len(calls) + i)].elapsed_time(
        ev[2 * (s * len(calls) + i) + 1]) for s in range(steps)) / steps, 4)
        for i, c in enumerate(calls)}
    out = {"ms_per_step": round(wall * 1e3 / steps, 4),
           "tokens_per_s": round(L.s.T * steps / wall, 1),
           "ms_per_call": per_call}
    if recompute:
        out["activation_bytes_kept"] = B.saved_bytes()
        out["saving_path_activation_bytes_kept"] = L.saved_bytes()
    if capacity is not None:
        counts = B.counts.cpu().numpy().astype(np.int64)
        g0, G = L.s.g0, L.s.groups
        out.update(capacity_rows_per_expert=capacity,
                   dropped_pairs=int(np.maximum(counts - capacity, 0).sum()),
                   pairs=int(counts.sum()),
                   gemm_rows_local=G * capacity,
                   gemm_rows_local_dropless=int(counts[g0:g0 + G].sum()))
    del B
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (the layer "
              f"here is one device's share; the design notes describe how it would shard)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    from synth.device import make_layer

    torch.cuda.set_device(0)
    cfg = synth.get_config(args.config)
    t_setup = time.time()
    inp = synth.make_inputs(cfg)
    L = make_layer(cfg, inp)
    del inp
    print(f"[bench] setup {time.time() - t_setup:.1f}s config={cfg.name}", file=sys.stderr,
          flush=True)

    calls = [c for c in CALLS if not (c.startswith("router") and not cfg.router)]
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    L.overlap = args.overlap
    for _ in range(args.warmup):
        L.step()
    torch.cuda.synchronize()
    rows = L.offsets.cpu().numpy()
    rows_local = int(rows[cfg.g0 + cfg.groups] - rows[cfg.g0])
    active_local = int((L.counts.cpu().numpy()[cfg.g0:cfg.g0 + cfg.groups] > 0).sum())

    # timed region: K whole steps (the route and router backward on a second
    # stream with --overlap), bracketed by device synchronisation
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        L.step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0

    # per-call breakdown: the same steps with every call on the working
    # stream; before each call a 1 GiB scratch read streams through the 256 MB
    # last-level cache (MALL) and the L2s, so no call reads its inputs from
    # the cache its predecessor left warm (a read, not a write: the lines it
    # leaves are clean, so the timed call does not pay for writing back the
    # flush; the predecessor's own dirty lines are written back during it);
    # HIP events bracket the call alone
    overlap, L.overlap = L.overlap, False
    stream = torch.cuda.current_stream()
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    timed = calls + REFERENCE_CALLS
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(len(timed))] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        for i, c in enumerate(timed):
            torch.amax(flush, dim=0, out=sink)
            ev[s][i][0].record(stream)
            getattr(L, c)()
            ev[s][i][1].record(stream)
    torch.cuda.synchronize()
    # the same calls back to back without the flush (inputs partly warm in
    # the MALL from the call before, as in a step)
    evw = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(len(timed))] for _ in range(args.steps)]
    for s in range(args.steps):
        for i, c in enumerate(timed):
            evw[s][i][0].record(stream)
            getattr(L, c)()
            evw[s][i][1].record(stream)
    torch.cuda.synchronize()
    del flush, sink
    L.overlap = overlap
    # median over the steps of each call's event-to-event time
    per_call = {c: float(np.median([ev[s][i][0].elapsed_time(ev[s][i][1])
                                    for s in range(args.steps)]))
                for i, c in enumerate(timed)}
    ms_per_step = wall * 1e3 / args.steps
    tokens_per_s = cfg.T * args.steps / wall

    per_call_warm = {c: float(np.median([evw[s][i][0].elapsed_time(evw[s][i][1])
                                         for s in range(args.steps)]))
                     for i, c in enumerate(timed)}
    alg = algorithmic(cfg, rows_local, active_local)
    phases = {}
    for c in timed:
        ms = per_call[c]
        d = {"ms": round(ms, 4)}
        if "flops" in alg[c]:
            tf = alg[c]["flops"] / (ms * 1e-3) / 1e12
            d["tflops"] = round(tf, 1)
            d["frac_bf16_peak"] = round(tf / BF16_PEAK_TFLOPS, 4)
        gbs = alg[c]["bytes"] / (ms * 1e-3) / 1e9
        d["gbs"] = round(gbs, 1)
        d["frac_hbm"] = round(gbs / HBM_PEAK_GBS, 4)
        d["ms_warm"] = round(per_call_warm[c], 4)
        d["frac_hbm_warm"] = round(alg[c]["bytes"] / (per_call_warm[c] * 1e-3) / 1e9
                                   / HBM_PEAK_GBS, 4)
        phases[c] = d
    dom = max((c for c in calls if c.startswith("gmm")), key=lambda c: per_call[c])
    dom_call = "moe_grouped_gemm_" + dom[4:]
    traffic = measured_traffic(dom_call) if cfg.name == "pangu" else None
    launches = {"gmm_bwd": "2 persistent launches, gmm_pair_kernel [dact + SwiGLU bwd | dW2] "
                           "then [dX | dW13]",
                "gmm_fwd": "1 persistent launch, gmm_chain_kernel (gate/up + SwiGLU, then down)"}
    # the binding roofline: whichever of the MFMA peak and HBM takes longer
    # for the call's algorithmic flops and bytes
    hbm_bound = alg[dom]["bytes"] / HBM_PEAK_GBS > alg[dom]["flops"] / BF16_PEAK_TFLOPS / 1e3
    roof = {"kernel": f"{dom_call} ({launches.get(dom, 'one call')})",
            "bound": "hbm" if hbm_bound else "mfma",
            "achieved": phases[dom]["gbs"] if hbm_bound else phases[dom]["tflops"],
            "peak": HBM_PEAK_GBS if hbm_bound else BF16_PEAK_TFLOPS,
            "unit": "GB/s" if hbm_bound else "TFLOP/s",
            "frac": phases[dom]["frac_hbm"] if hbm_bound else phases[dom]["frac_bf16_peak"],
            "traffic": round(traffic) if traffic else None,
            "flops_per_launch": alg[dom]["flops"], "ms_per_launch": round(per_call[dom], 4),
            "algorithmic_bytes": alg[dom]["bytes"],
            "frac_bf16_peak": phases[dom]["frac_bf16_peak"],
            "frac_hbm": phases[dom]["frac_hbm"]}

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.description}; T={cfg.T} H={cfg.H} I={cfg.I} "
                               f"E={cfg.E} top-{cfg.k}, grouped GEMM over experts "
                               f"[{cfg.g0},{cfg.g0 + cfg.groups})"
                               + (" + shared expert" if cfg.shared else "") + ", fwd+bwd",
                   "tokens": cfg.T, "rows_local": rows_local, "parallelism": "none (1 GPU)",
                   "streams": 2 if overlap else 1},
        "roofline": roof,
        "phases": phases,
    }
    if not args.no_dense_ref and cfg.dtype == "bf16":
        out["dense_ref"] = dense_reference(cfg)
        out["hbm_ref"] = hbm_reference()
    if not args.no_variants and cfg.dtype == "bf16":
        import math
        C = math.ceil(1.2 * cfg.T * cfg.k / cfg.E)   # capacity factor 1.2
        out["variants"] = {
            "recompute": variant(L, args.steps, args.warmup, recompute=True),
            "drop_and_pad_cf1.2": variant(L, args.steps, args.warmup, capacity=C)}
    del L
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.config, min(args.cpu_tokens, cfg.T))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
