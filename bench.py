#!/usr/bin/env python3
"""Benchmark of the dropless-MoE expert layer on one MI355X.

One step = routing metadata + forward + backward of the whole layer (every
kernel of the path) on one batch of seeded synthetic input already resident
in HBM.  Default workload: the fine-grained layer T=4096 (2x2048 tokens),
H=2048, F=1024, E=64, top-8, bf16, Gaussian router.

Prints ONE JSON line with tokens/s, the per-kernel times (HIP events that
the library records between its kernels: around every kernel in an untimed
pass, and around the dominant kernel in the timed steps, each interval less
the measured cost of one record), the roofline of the dominant kernel and
the CPU oracle's rate on the host.  The same line carries a compact record
of the other seeded workloads (``workloads``), the step with the
activation-lean backward (``lean_backward``), cold-cache figures, the layer
on tile-aware token-rounded routing (``token_rounding``) and the dMoA map /
reduce pair with its backward (``moa``).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
                    [--workloads zipf_e64,coarse_e8,... | none]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 matrix / vector
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

METRIC = "dMoE fwd+bwd tokens/s and useful TFLOP/s (% bf16 MFMA peak), E=64 k=8"

META_KERNELS = ["meta_hist", "meta_scan", "meta_place"]
FWD_KERNELS = ["padded_gather", "gemm_up_gate", "gemm_down", "padded_scatter"]
BWD_KERNELS = ["scatter_backward", "gemm_down_dgrad_wgrad_down", "gemm_up_dgrad",
               "gather_backward", "gemm_wgrad_up"]


def kernel_work(cfg, P, fused=False):
    """Algorithmic FLOPs and bytes of each kernel for P padded rows.

    Bytes are unique reads plus writes; weights are counted once per kernel
    for the experts that have rows.  GEMM FLOPs are the executed (padded)
    multiply-adds x2.  fused: the gather fused into the up projection's
    operand loads, so that product reads the T token rows of x instead of
    the P rows of x_perm (the gather then runs in the backward)."""
    s = 4 if cfg.dtype == "f32" else 2
    T, H, F, E, k = cfg.T, cfg.H, cfg.F, cfg.E, cfg.k
    N = T * k
    Ea = E  # every expert is active in the timed workloads
    w = {}
    w["meta_hist"] = (0, 4 * N + 4 * E)
    w["meta_scan"] = (0, 16 * E)
    w["meta_place"] = (0, 4 * N + 12 * N)
    w["padded_gather"] = (0, (T * H + P * H) * s)
    X = T * H if fused else P * H     # rows the up projection reads
    w["gemm_up_gate"] = (4 * P * H * F, (X + 2 * Ea * H * F + 3 * P * F) * s)
    w["gemm_down"] = (2 * P * F * H, (P * F + Ea * F * H + P * H) * s)
    w["padded_scatter"] = (0, (N * H + T * H) * s + 4 * N)
    w["scatter_backward"] = (0, (T * H + N * H + P * H) * s + 8 * N)
    # down dgrad + gate backward and dw2, one launch: dy_perm is read once
    w["gemm_down_dgrad_wgrad_down"] = (
        4 * P * H * F, (P * H + 2 * Ea * F * H + 5 * P * F) * s)
    w["gemm_up_dgrad"] = (4 * P * H * F, (2 * P * F + 2 * Ea * H * F + P * H) * s)
    w["gemm_wgrad_up"] = (4 * P * H * F, (P * H + 2 * P * F + 2 * Ea * H * F) * s)
    w["gather_backward"] = (0, (N * H + T * H) * s)
    return w


MOA_CALLS = ["moa_map", "moa_reduce", "moa_reduce_backward", "moa_map_backward"]


def moa_work(cfg, P):
    """Algorithmic FLOPs and bytes of each dMoA entry point for P padded rows
    (bf16): the sum over the kernels the call launches, each counted as in
    kernel_work (unique reads plus writes, weights once)."""
    s = 2
    T, H, F, E, k = cfg.T, cfg.H, cfg.F, cfg.E, cfg.k
    N = T * k
    w = {}
    # gather x; q_perm = x_perm w1[e]; q in slot order
    w["moa_map"] = (2 * P * H * F,
                    ((T * H + P * H) + (P * H + E * H * F + P * F) + 2 * N * F) * s)
    # y in padded order; o_perm = y_perm w2[e]; out = weighted top-k sum
    w["moa_reduce"] = (2 * P * F * H,
                       ((N * F + P * F) + (P * F + E * F * H + P * H) + (N * H + T * H)) * s
                       + 4 * N)
    # do_perm = w dout and d_weights; dy_perm = do_perm w2^T; dw2; dy in slot order
    w["moa_reduce_backward"] = (
        4 * P * F * H,
        ((T * H + N * H + P * H) + (P * H + E * F * H + P * F) + (P * F + P * H + E * F * H)
         + 2 * N * F) * s + 8 * N)
    # dq in padded order; dx_perm = dq_perm w1^T; dx = unit top-k sum; dw1
    w["moa_map_backward"] = (
        4 * P * H * F,
        ((N * F + P * F) + (P * F + E * H * F + P * H) + (N * H + T * H)
         + (P * H + P * F + E * H * F)) * s)
    return w


def roof_time(flop, nbytes, peak_tflops):
    """Seconds a kernel takes at its roofline: the larger of its FLOP at the
    matrix-core peak and its algorithmic bytes at the HBM peak."""
    return max((flop or 0.0) / (peak_tflops * 1e12), nbytes / (PEAK_HBM_GBS * 1e9))


def committed_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summaries under
    profiles/ (FETCH_SIZE + WRITE_SIZE, calibrated on a plain copy), or None
    if there is none for this kernel and workload or the kernel's source
    changed since the counters were taken."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*traffic*.json"))):
        try:
            with open(path) as fh:
                d = json.load(fh)
        except (OSError, ValueError):
            continue
        if d.get("bench_name") != kernel or d.get("workload") != workload:
            continue
        src = os.path.join(ROOT, d.get("source", ""))
        if not os.path.isfile(src):
            return None
        with open(src, "rb") as fh:
            if hashlib.sha256(fh.read()).hexdigest() != d.get("source_sha256"):
                return None
        return float(d["traffic_bytes_per_launch"])
    return None


def cpu_baseline(inp, budget_s=30.0):
    """Time the fp64 CPU oracle (metadata + forward + backward) on the host."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    t0 = time.perf_counter()
    y, saved = oracle.forward_padded(inp.x, inp.top_experts, inp.weights,
                                     inp.w1, inp.w3, inp.w2)
    g = oracle.backward_padded(inp.x, inp.top_experts, inp.weights, inp.w1,
                               inp.w3, inp.w2, inp.dy, saved)
    dt = time.perf_counter() - t0
    assert np.isfinite(y).all() and np.isfinite(g["dx"]).all()
    T = inp.cfg.T
    return {"value": T / dt, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"one full step (metadata + forward + backward, fp64 numpy, "
                       f"expert-batched) of the same {T}-token workload: {dt:.2f} s; "
                       f"host os.cpu_count()={os.cpu_count()}"),
            "literal_loop": cpu_literal_loop(inp, threads)}


def cpu_literal_loop(inp, threads, max_tokens=64, budget_s=20.0):
    """The oracle's per-(token, slot) loop, forward and backward, over the
    workload's first tokens, one token per call, until max_tokens or the time
    budget is reached; tokens/s of that sample."""
    import numpy as np
    import oracle
    n, dt = 0, 0.0
    while n < min(max_tokens, inp.cfg.T) and dt < budget_s:
        sl = slice(n, n + 1)
        t0 = time.perf_counter()
        y, _ = oracle.forward_loop(inp.x[sl], inp.top_experts[sl], inp.weights[sl],
                                   inp.w1, inp.w3, inp.w2)
        g = oracle.backward_loop(inp.x[sl], inp.top_experts[sl], inp.weights[sl],
                                 inp.w1, inp.w3, inp.w2, inp.dy[sl])
        dt += time.perf_counter() - t0
        assert np.isfinite(y).all() and np.isfinite(g["dx"]).all()
        n += 1
    return {"value": n / dt, "unit": "tokens/s", "cores": int(threads),
            "sample": (f"per-token loop (fp64 numpy, forward + backward) over the first "
                       f"{n} tokens of the workload, one token per call: {dt:.2f} s")}


def event_overhead_ms(stream, n=40):
    """Median interval between two HIP event records with nothing between
    them on the stream: what every bracketed interval carries on top of
    the kernel it brackets (about 4.5 us on MI355X)."""
    import statistics
    import torch
    from dropless_mixture_experts_amd.hip_events import EventArray
    torch.cuda.synchronize()
    ev = EventArray(n)
    for i in range(n):
        ev.record(i, stream)
    torch.cuda.synchronize()
    gaps = [ev.elapsed_ms(i, i + 1) for i in range(n - 1)]
    ev.close()
    return statistics.median(gaps)


def cold_steps(step, stream, n, flush_mb=512):
    """Median milliseconds of n steps, each started after a flush_mb write
    that evicts the last-level cache (256 MB), so that every input and weight
    comes from HBM.  The flush sits between the two events, not inside them."""
    import statistics
    import torch
    scratch = torch.empty(flush_mb << 18, dtype=torch.float32, device=stream.device)
    times = []
    for _ in range(n):
        scratch.fill_(1.0)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    del scratch
    return statistics.median(times)


def router_time(dm, cfg, dev, stream, steps):
    """Mean microseconds of the router's forward (top-k, softmax, z-loss) and
    backward on this workload's seeded logits.  Reported beside the layer's
    step, not part of it: the layer takes ids and weights as inputs."""
    import torch
    from workloads import make_logits
    logits, d_weights = make_logits(cfg)
    l = torch.from_numpy(logits).to(dev)
    g = torch.from_numpy(d_weights).to(dev)
    D = dm.Dims(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, dm.DMOE_F32)
    ids = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device=dev)
    w = torch.empty(cfg.T, cfg.k, dtype=torch.float32, device=dev)
    z = torch.empty(cfg.T, dtype=torch.float32, device=dev)
    zl = torch.empty(1, dtype=torch.float32, device=dev)
    dl = torch.empty(cfg.T, cfg.E, dtype=torch.float32, device=dev)

    def once():
        dm.dmoe_router_forward(D, l, ids, w, zloss_coef=0.001, z=z, zloss=zl, stream=stream)
        dm.dmoe_router_backward(D, l, ids, w, g, dl, zloss_coef=0.001, stream=stream)

    for _ in range(3):
        once()
    with torch.cuda.stream(stream):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            once()
        e1.record(stream)
    torch.cuda.synchronize()
    return round(e0.elapsed_time(e1) * 1e3 / steps, 1)



def moa_leg(dm, dev, ovh, K=10, W=3):
    """The dMoA map / reduce pair (mixture of attention heads) on moa_e16:
    per step the metadata, map, reduce, reduce_backward and map_backward.
    The attention between map and reduce is outside the library and not
    timed; its output (y) and the map's upstream gradient (dq) are seeded
    N(0,1) stand-ins of their shapes."""
    import torch
    from dropless_mixture_experts_amd.hip_events import EventArray
    from workloads import CONFIGS, make_inputs
    cfg = CONFIGS["moa_e16"]
    inp = make_inputs(cfg)
    print(f"bench: dMoA map/reduce on {cfg.name}", file=sys.stderr, flush=True)
    D = dm.Dims(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, dm.DMOE_BF16)
    L = dm.DMoALayer(D, dev)
    bf = torch.bfloat16
    up = lambda a, dt=bf: torch.from_numpy(a).to(dev).to(dt).contiguous()
    x, w1, w2, dout = up(inp.x), up(inp.w1), up(inp.w2), up(inp.dy)
    ids = up(inp.top_experts, torch.int32)
    wts = up(inp.weights, torch.float32)
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed_id)
    y = torch.randn(cfg.T * cfg.k, cfg.F, generator=gen, device=dev).to(bf)
    dq = torch.randn(cfg.T * cfg.k, cfg.F, generator=gen, device=dev).to(bf)
    stream = torch.cuda.current_stream(dev)
    calls = [lambda: L.map(x, w1), lambda: L.reduce(y, wts, w2),
             lambda: L.reduce_backward(dout, wts, w2), lambda: L.map_backward(dq, w1)]

    def step(ev=None):
        L.metadata(ids)
        for i, f in enumerate(calls):
            if ev is not None:
                ev.record(i, stream)
            f()
        if ev is not None:
            ev.record(len(calls), stream)

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    P = int(L.meta.num_padded_rows.item())
    evs = [EventArray(len(calls) + 1) for _ in range(K)]
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    per = {n: max(sum(ev.elapsed_ms(i, i + 1) for ev in evs) / K - ovh, 0.0)
           for i, n in enumerate(MOA_CALLS)}
    for ev in evs:
        ev.close()
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / K
    work = moa_work(cfg, P)
    N = cfg.T * cfg.k
    table = {}
    for n in MOA_CALLS:
        fl, by = work[n]
        t = per[n] * 1e-3
        table[n] = {"ms": round(per[n], 4), "tflops": round(fl / t / 1e12, 1),
                    "gbs": round(by / t / 1e9, 1),
                    "roofline_frac": round(roof_time(fl, by, PEAK_BF16_TFLOPS) / t, 4)}
    dom = max(MOA_CALLS, key=lambda n: per[n])
    fl, by = work[dom]
    ai = fl / by
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    t = per[dom] * 1e-3
    roof = ({"call": dom, "bound": "hbm", "achieved": round(by / t / 1e9, 1),
             "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(by / t / 1e9 / PEAK_HBM_GBS, 4)}
            if ai < ridge else
            {"call": dom, "bound": "mfma", "achieved": round(fl / t / 1e12, 1),
             "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
             "frac": round(fl / t / 1e12 / PEAK_BF16_TFLOPS, 4)})
    roof["intensity_flop_per_byte"] = round(ai, 1)
    gemm_flop = sum(work[n][0] for n in MOA_CALLS)
    rec = {"config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "F": cfg.F, "E": cfg.E,
                      "k": cfg.k, "dtype": cfg.dtype, "routing": cfg.routing, "P": P},
           "steps": K, "warmup": W, "ms_per_step": round(ms, 4),
           "tokens_s": round(cfg.T / (ms * 1e-3), 1),
           "useful_tflops": round(12.0 * N * cfg.H * cfg.F / (ms * 1e-3) / 1e12, 1),
           "gemm_executed_tflops": round(gemm_flop / (ms * 1e-3) / 1e12, 1),
           "calls": table, "roofline": roof,
           "note": ("metadata + map + reduce + reduce_backward + map_backward per step; the "
                    "attention between map and reduce is not part of the library and not "
                    "timed; per-call ms from K steps with an event around every call")}
    del L
    return rec


def saved_bytes_per_token(cfg, P):
    """Bytes of activations kept from the forward for the backward, per
    token: the plain backward keeps x_perm, h1, h3, act and y_perm; the
    activation recompute drops act; the lean backward keeps y_perm only (it
    rebuilds the rest from x, which the caller holds anyway)."""
    s = 4 if cfg.dtype == "f32" else 2
    H, F = cfg.H, cfg.F
    per_row = {"plain": 2 * H + 3 * F, "recompute_act": 2 * H + 2 * F, "lean": H}
    return {k: round(v * s * P / cfg.T, 1) for k, v in per_row.items()}


class Layer:
    """One workload resident on the GPU with its buffers and the step."""

    def __init__(self, dm, cfg, dev, gather="auto", inputs=None):
        import numpy as np
        import torch
        from workloads import make_inputs
        self.dm, self.cfg, self.dev = dm, cfg, dev
        self.inp = inputs if inputs is not None else make_inputs(cfg)
        dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
        up = lambda a, d=dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(d)
        inp = self.inp
        self.x, self.dy = up(inp.x), up(inp.dy)
        self.ids = up(inp.top_experts, torch.int32)
        self.w = up(inp.weights, torch.float32)
        self.w1, self.w3, self.w2 = up(inp.w1), up(inp.w3), up(inp.w2)
        self.D = dm.Dims(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k,
                         dm.DMOE_F32 if cfg.dtype == "f32" else dm.DMOE_BF16)
        self.fused = cfg.dtype == "bf16" and (
            gather == "fused" or (gather == "auto" and dm.fused_gather_pays(self.D)))
        self.layer = dm.DMoELayer(self.D, dev, fused_gather=self.fused)
        self.fwd_kernels = [n for n in FWD_KERNELS if not (self.fused and n == "padded_gather")]
        self.bwd_kernels = list(BWD_KERNELS)
        if self.fused:   # the backward gathers x_perm right before the up dgrad
            self.bwd_kernels.insert(self.bwd_kernels.index("gemm_up_dgrad"), "padded_gather")
        self.y = torch.empty(cfg.T, cfg.H, dtype=dt, device=dev)
        self.grads = dict(dx=torch.empty(cfg.T, cfg.H, dtype=dt, device=dev),
                          dw1=torch.empty_like(self.w1), dw3=torch.empty_like(self.w3),
                          dw2=torch.empty_like(self.w2),
                          d_weights=torch.empty(cfg.T, cfg.k, dtype=torch.float32,
                                                device=dev))
        self.stream = torch.cuda.current_stream(dev)
        self.phases = (META_KERNELS, self.fwd_kernels, self.bwd_kernels)
        self.names = META_KERNELS + self.fwd_kernels + self.bwd_kernels

    def step(self, ev=None, lean=False, stream="fixed"):
        """Metadata + forward + backward.  stream=None: torch's current
        stream at call time (for graph capture)."""
        st = self.stream if stream == "fixed" else None
        L = self.layer
        L.metadata(self.ids, st, ev[0] if ev else None)
        L.forward(self.x, self.ids, self.w, self.w1, self.w3, self.w2, y=self.y, stream=st,
                  run_metadata=False, events=ev[1] if ev else None)
        L.backward(self.dy, self.w, self.w1, self.w3, self.w2, grads=self.grads, stream=st,
                   events=ev[2] if ev else None, lean=lean)

    def padded_rows(self):
        import torch
        torch.cuda.synchronize()
        assert int(self.layer.buf.meta.status.item()) == 0
        return int(self.layer.buf.meta.num_padded_rows.item())

    def per_kernel(self, n, ovh, flush=None):
        """Mean ms of every kernel over n untimed steps with an event around
        every kernel, less one record's cost; flush(): called before each
        step, outside the events (cold-cache pass)."""
        import torch
        from dropless_mixture_experts_amd.hip_events import EventArray
        raw = {k: 0.0 for k in self.names}
        evs = [tuple(EventArray(len(ks) + 1) for ks in self.phases) for _ in range(n)]
        torch.cuda.synchronize()
        for ev in evs:            # back to back, as in the timed steps
            if flush:
                flush()
            self.step(ev)
        torch.cuda.synchronize()
        for ev in evs:
            for arr, ks in zip(ev, self.phases):
                for j, k in enumerate(ks):
                    raw[k] += arr.elapsed_ms(j, j + 1) / n
                arr.close()
        return raw, {k: max(raw[k] - ovh, 0.0) for k in self.names}

    def timed(self, K, dom=None, lean=False):
        """Wall time of K back-to-back steps between two synchronizations;
        with dom, two event records around that kernel in every step.
        Returns (ms per step, the mean raw event interval of dom)."""
        import torch
        from dropless_mixture_experts_amd.hip_events import EventArray
        evs = []
        if dom is not None:
            dph = next(i for i, ks in enumerate(self.phases) if dom in ks)
            dj = self.phases[dph].index(dom)
            for _ in range(K):
                ev = [None, None, None]
                ev[dph] = EventArray(len(self.phases[dph]) + 1, only=(dj, dj + 1))
                evs.append(tuple(ev))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            self.step(evs[i] if evs else None, lean=lean)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / K
        dom_raw = None
        if evs:
            dom_raw = sum(ev[dph].elapsed_ms(dj, dj + 1) for ev in evs) / K
            for ev in evs:
                ev[dph].close()
        return ms, dom_raw

    def graph_ms(self, K, replays=3):
        """ms per step when one whole step (metadata, forward, backward) is
        captured as a HIP graph and replayed K times back to back."""
        import torch
        side = torch.cuda.Stream(self.dev)
        side.wait_stream(torch.cuda.current_stream(self.dev))
        with torch.cuda.stream(side):
            for _ in range(2):
                self.step(stream=None)
        torch.cuda.current_stream(self.dev).wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step(stream=None)
        torch.cuda.synchronize()
        best = None
        for _ in range(replays):
            t0 = time.perf_counter()
            for _ in range(K):
                g.replay()
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1e3 / K
            best = ms if best is None else min(best, ms)
        del g
        return best

    def close(self):
        import torch
        for n in ("x", "dy", "ids", "w", "w1", "w3", "w2", "y", "grads", "layer", "inp"):
            setattr(self, n, None)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def summarise(cfg, P, per, fused):
    """The per-kernel table and the step's fractions from per-kernel ms."""
    peak = PEAK_F32_TFLOPS if cfg.dtype == "f32" else PEAK_BF16_TFLOPS
    work = kernel_work(cfg, P, fused)
    names = list(per)
    table = {}
    for n in names:
        fl, by = work[n]
        t = per[n] * 1e-3
        table[n] = {"ms": round(per[n], 4),
                    "tflops": round(fl / t / 1e12, 1) if fl and t > 0 else None,
                    "gbs": round(by / t / 1e9, 1) if t > 0 else None,
                    "roofline_frac": (round(roof_time(fl, by, peak) / t, 4)
                                      if t > 0 else None)}
    gemms = [n for n in names if n.startswith("gemm")]
    gemm_ms = sum(per[n] for n in gemms)
    gemm_roof_s = sum(roof_time(*work[n], peak) for n in gemms)
    gs = [n for n in ("padded_gather", "padded_scatter", "scatter_backward",
                      "gather_backward") if n in names]
    gs_ms = sum(per[n] for n in gs)
    gs_bytes = sum(work[n][1] for n in gs)
    executed_flop = 18.0 * P * cfg.H * cfg.F
    return table, {
        "gemm_executed_frac_peak": round(executed_flop / (gemm_ms * 1e-3) / 1e12 / peak, 4),
        # the GEMMs' time at their per-kernel roofline, max(FLOP / peak,
        # bytes / HBM peak), over their measured time
        "gemm_roofline_frac": round(gemm_roof_s / (gemm_ms * 1e-3), 4),
        "gather_scatter_frac_hbm": round(gs_bytes / (gs_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "metadata_us": round(1e3 * sum(per[n] for n in META_KERNELS), 1),
        # latency-bound: a few MB in three small launches
        "metadata_frac_hbm": round(sum(work[n][1] for n in META_KERNELS)
                                   / (sum(per[n] for n in META_KERNELS) * 1e-3) / 1e9
                                   / PEAK_HBM_GBS, 5),
    }


def roofline(cfg, P, fused, dom, dom_ms):
    """The roofline object of kernel dom, run in dom_ms per launch."""
    peak = PEAK_F32_TFLOPS if cfg.dtype == "f32" else PEAK_BF16_TFLOPS
    fl, by = kernel_work(cfg, P, fused)[dom]
    # the binding roof at the kernel's arithmetic intensity (algorithmic FLOP
    # per unique byte): the matrix cores above the ridge, HBM below it
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    intensity = fl / by if fl else 0.0
    t = dom_ms * 1e-3
    if fl and intensity >= ridge:
        achieved = fl / t / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1),
                "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": None}
    else:
        achieved = by / t / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    roof["intensity_flop_per_byte"] = round(intensity, 1)
    roof["ridge_flop_per_byte"] = round(ridge, 1)
    if fl:
        roof["tflops"] = round(fl / t / 1e12, 1)
        roof["tflops_frac_of_mfma_peak"] = round(fl / t / 1e12 / peak, 4)
        # the kernel against its own roofline time, max(FLOP / peak, bytes / HBM)
        roof["frac_of_roofline_time"] = round(roof_time(fl, by, peak) / t, 4)
    roof["launch_ms"] = round(dom_ms, 4)
    roof["algorithmic_bytes_per_launch"] = by
    roof["algorithmic_flop_per_launch"] = fl
    roof["traffic"] = committed_traffic(dom, cfg.name)
    return roof


def other_workload(dm, name, dev, args, ovh):
    """Compact record of one more workload: its step, GEMM fractions and
    the roofline of its dominant kernel."""
    from workloads import CONFIGS
    cfg = CONFIGS[name]
    t0 = time.perf_counter()
    L = Layer(dm, cfg, dev, gather=args.gather)
    t_in = time.perf_counter() - t0
    print(f"bench: workload {name} (inputs {t_in:.1f} s)", file=sys.stderr, flush=True)
    K, W = 10, 3
    for _ in range(W):
        L.step()
    P = L.padded_rows()
    _, per = L.per_kernel(3, ovh)
    dom = max(L.names, key=lambda n: per[n])
    ms, dom_raw = L.timed(K, dom)
    table, fr = summarise(cfg, P, per, L.fused)
    peak = PEAK_F32_TFLOPS if cfg.dtype == "f32" else PEAK_BF16_TFLOPS
    useful = 18.0 * cfg.T * cfg.k * cfg.H * cfg.F / (ms * 1e-3) / 1e12
    rec = {"config": {"T": cfg.T, "H": cfg.H, "F": cfg.F, "E": cfg.E, "k": cfg.k,
                      "dtype": cfg.dtype, "routing": cfg.routing, "P": P,
                      "gather": "fused" if L.fused else "plain"},
           "steps": K, "warmup": W, "ms_per_step": round(ms, 4),
           "tokens_s": round(cfg.T / (ms * 1e-3), 1),
           "useful_tflops": round(useful, 1), "useful_frac_peak": round(useful / peak, 4),
           **fr,
           "roofline": roofline(cfg, P, L.fused, dom, dom_raw - ovh),
           "kernels": {n: table[n]["ms"] for n in L.names}}
    if cfg.dtype == "f32" or cfg.T * cfg.k <= 4096:
        # small layers are bound by the host's launches: the same step
        # captured once as a HIP graph and replayed
        g = L.graph_ms(K)
        rec["graph_replay"] = {"ms_per_step": round(g, 4),
                               "tokens_s": round(cfg.T / (g * 1e-3), 1)}
    L.close()
    return rec


def token_rounding(dm, name, dev, args, ovh, topk_ms):
    """The layer's step on tile-aware token-rounded routing against top-k
    on the same logits: the rounding's own time, the padded rows, and the
    step.  topk_ms: the top-k step of this workload, if measured here."""
    import dataclasses
    import numpy as np
    import torch
    from workloads import CONFIGS, make_inputs, make_logits
    cfg = CONFIGS[name]
    logits, _ = make_logits(cfg)
    D = dm.Dims(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, dm.DMOE_F32)
    l = torch.from_numpy(logits).to(dev)
    ids = torch.empty(cfg.T, cfg.k + 1, dtype=torch.int32, device=dev)
    w = torch.empty(cfg.T, cfg.k + 1, dtype=torch.float32, device=dev)
    ws = torch.empty(dm.dmoe_token_round_workspace_bytes(D), dtype=torch.uint8, device=dev)
    for _ in range(3):
        dm.dmoe_token_round(D, l, ids, w, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dm.dmoe_token_round(D, l, ids, w, ws)
    e1.record()
    torch.cuda.synchronize()
    round_us = e0.elapsed_time(e1) * 1e3 / 10
    inp = make_inputs(cfg)
    rcfg = cfg.replace(k=cfg.k + 1)
    inp = dataclasses.replace(inp, cfg=rcfg, top_experts=ids.cpu().numpy(),
                              weights=w.cpu().numpy())
    L = Layer(dm, rcfg, dev, gather=args.gather, inputs=inp)
    for _ in range(3):
        L.step()
    P = L.padded_rows()
    ms, _ = L.timed(10)
    if topk_ms is None:
        T = Layer(dm, cfg, dev, gather=args.gather, inputs=make_inputs(cfg))
        for _ in range(3):
            T.step()
        topk_P = T.padded_rows()
        topk_ms, _ = T.timed(10)
        T.close()
    else:
        topk_P = None
    occupied = int((L.ids >= 0).sum().item())
    L.close()
    rec = {"workload": name, "tile_rows": 128, "round_us": round(round_us, 1),
           "entries": occupied, "entries_topk": cfg.T * cfg.k, "P": P,
           "ms_per_step": round(ms, 4), "tokens_s": round(cfg.T / (ms * 1e-3), 1),
           "topk_ms_per_step": round(topk_ms, 4),
           "speedup_vs_topk": round(topk_ms / ms, 3),
           "note": ("metadata + forward + backward on the token-rounded slots (k + 1 per token, "
                    "empty slots -1), against the same step on top-k routing; the rounding's "
                    "own time (router top-(k+1), metadata of the k + 1 slots, selection) is "
                    "round_us, outside the step like the router's")}
    if topk_P is not None:
        rec["P_topk"] = topk_P
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="fine_e64")
    ap.add_argument("--workloads", default="zipf_e64,coarse_e8,sparse_e256,tiny_f32,moa_e16",
                    help="comma-separated other workloads reported under 'workloads' "
                         "(10 steps each; moa_e16, the dMoA map / reduce pair, under "
                         "'moa'), or 'none'")
    ap.add_argument("--rounding", default="sparse_e256",
                    help="workload on which to time the layer on tile-aware token-rounded "
                         "routing against top-k, or 'none'")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-lean", action="store_true",
                    help="skip the step with the activation-lean backward")
    ap.add_argument("--kernels", action="store_true",
                    help="also print the per-kernel table on stderr")
    ap.add_argument("--gather", choices=("auto", "plain", "fused"), default="auto",
                    help="plain: padded copy in the forward; fused: the gather "
                         "inside the up projection's operand loads (bf16); auto: "
                         "fused where the padded copy of x exceeds the last-level "
                         "cache")
    ap.add_argument("--fused-gather", action="store_true",
                    help="same as --gather fused")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB "
                         "three times (reference for hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if world != 1:
        print("bench.py is single-process: WORLD_SIZE must be 1", file=sys.stderr)
        sys.exit(2)
    if args.fused_gather:
        args.gather = "fused"

    import torch

    import dropless_mixture_experts_amd as dm
    from workloads import CONFIGS

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    dm.load_library()   # fail loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    cfg = CONFIGS[args.workload]
    L = Layer(dm, cfg, dev, gather=args.gather)
    stream = L.stream
    print(f"bench: workload {cfg.name}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        L.step()
    P = L.padded_rows()
    K = args.steps

    # Per-kernel table: a pass of its own, outside the timed region, with an
    # event around every kernel (each record puts a timestamp between two
    # kernels, ~5 us each at 15 per step).
    ovh = event_overhead_ms(stream)
    KP = max(3, min(K, 10))
    raw, per = L.per_kernel(KP, ovh)
    dom = max(L.names, key=lambda n: per[n])
    # The timed region: K steps with two event records, around the dominant
    # kernel, whose duration the roofline takes from here.
    ms, dom_raw = L.timed(K, dom)
    tokens_s = cfg.T / (ms * 1e-3)
    peak = PEAK_F32_TFLOPS if cfg.dtype == "f32" else PEAK_BF16_TFLOPS
    useful_tf = 18.0 * cfg.T * cfg.k * cfg.H * cfg.F / (ms * 1e-3) / 1e12
    table, fr = summarise(cfg, P, per, L.fused)
    for n in L.names:
        table[n]["interval_ms"] = round(raw[n], 4)
    roof = roofline(cfg, P, L.fused, dom, dom_raw - ovh)
    roof["event_interval_ms"] = round(dom_raw, 4)

    out = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; Gaussian router logits, top-k + softmax)",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "F": cfg.F,
                   "E": cfg.E, "k": cfg.k, "routing": cfg.routing, "P": P,
                   "gather": ("fused into the up projection's loads; gathered in the "
                              "backward" if L.fused else "padded copy in the forward")},
        "useful_tflops": round(useful_tf, 1),
        "useful_frac_peak": round(useful_tf / peak, 4),
        **fr,
        "roofline": roof,
        "kernels": table,
        "event_overhead_us": round(ovh * 1e3, 2),
        "kernels_note": (f"per-kernel ms from {KP} untimed steps with an event around every "
                         f"kernel; roofline.kernel timed inside the {K} timed steps; ms = "
                         f"interval_ms less event_overhead_us, the interval between two "
                         f"records with nothing between them"),
    }
    out["router_us"] = router_time(dm, cfg, dev, stream, K)
    if not args.no_lean:
        lean_ms, _ = L.timed(K, lean=True)
        out["lean_backward"] = {
            "ms_per_step": round(lean_ms, 4),
            "tokens_s": round(cfg.T / (lean_ms * 1e-3), 1),
            "saved_activation_bytes_per_token": saved_bytes_per_token(cfg, P),
            "note": ("metadata + forward + dmoe_backward_lean, which rebuilds x_perm, h1, h3 "
                     "and act from x: only y_perm is kept from forward to backward"),
        }
    # Cold cache: each step after a 512 MB write that evicts the 256 MB
    # last-level cache, timed as a whole and, in a pass of its own, per kernel.
    flush_buf = torch.empty(512 << 18, dtype=torch.float32, device=dev)
    flush = lambda: flush_buf.fill_(1.0)
    cold = cold_steps(L.step, stream, min(K, 10))
    _, cper = L.per_kernel(5, ovh, flush=flush)
    _, cfr = summarise(cfg, P, cper, L.fused)
    del flush_buf
    gs = [n for n in ("padded_gather", "padded_scatter", "scatter_backward",
                      "gather_backward") if n in L.names]
    out["cold_cache"] = {"ms_per_step_median": round(cold, 4),
                         "tokens_s": round(cfg.T / (cold * 1e-3), 1),
                         "gather_scatter_frac_hbm": cfr["gather_scatter_frac_hbm"],
                         "kernels_ms": {n: round(cper[n], 4) for n in L.names},
                         "gather_scatter_ms": {n: round(cper[n], 4) for n in gs},
                         "note": ("last-level cache flushed by a 512 MB write before each "
                                  "step; per-kernel figures from 5 such steps with an event "
                                  "around every kernel")}
    if args.kernels:
        for n in L.names:
            print(f"{n:28s} {table[n]}", file=sys.stderr)
    if args.calibrate_copy_mb:
        nbytes = args.calibrate_copy_mb << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["calibration_copy_bytes"] = nbytes
        del src, dst
    inp = L.inp
    L.close()
    others = [n for n in args.workloads.split(",") if n and n != "none" and n != cfg.name]
    if "moa_e16" in others:
        # the dMoA map / reduce pair: its own record, not a dMoE layer's
        others.remove("moa_e16")
        out["moa"] = moa_leg(dm, dev, ovh)
    if others:
        out["workloads"] = {n: other_workload(dm, n, dev, args, ovh) for n in others}
    if args.rounding != "none":
        print(f"bench: token rounding on {args.rounding}", file=sys.stderr, flush=True)
        known = (out.get("workloads", {}).get(args.rounding, {}).get("ms_per_step")
                 if args.rounding != cfg.name else ms)
        out["token_rounding"] = token_rounding(dm, args.rounding, dev, args, ovh, known)
        if known is not None:
            P_topk = (P if args.rounding == cfg.name
                      else out["workloads"][args.rounding]["config"]["P"])
            out["token_rounding"]["P_topk"] = P_topk
    if not args.no_cpu:
        print("bench: CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
