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
the CPU oracle's rate on the host.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import threading
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


def gpu_sclk_mhz():
    """The shader clock the amdgpu kernel driver reports as current (sysfs
    pp_dpm_sclk, the level marked '*'), or None where it is not readable."""
    import glob
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for line in open(f):
                if "*" in line:
                    return int(line.split(":")[1].strip().lower().split("mhz")[0])
        except (OSError, ValueError, IndexError):
            continue
    return None


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="fine_e64")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--kernels", action="store_true",
                    help="also print the per-kernel table on stderr")
    ap.add_argument("--gather", choices=("auto", "plain", "fused"), default="auto",
                    help="plain: padded copy in the forward; fused: the gather "
                         "inside the up projection's operand loads (bf16); auto: "
                         "fused where the padded copy of x exceeds the last-level "
                         "cache")
    ap.add_argument("--fused-gather", action="store_true",
                    help="same as --gather fused: time the path with the gather fused into the up "
                         "projection's operand loads (the backward gathers x_perm)")
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

    import numpy as np
    import torch

    import dropless_mixture_experts_amd as dm
    from dropless_mixture_experts_amd.hip_events import EventArray
    from workloads import CONFIGS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    dm.load_library()   # fail loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    cfg = CONFIGS[args.workload]
    t_gen = time.perf_counter()
    inp = make_inputs(cfg)
    t_gen = time.perf_counter() - t_gen
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    up = lambda a, d=dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(d)
    x, dy = up(inp.x), up(inp.dy)
    ids = up(inp.top_experts, torch.int32)
    w = up(inp.weights, torch.float32)
    w1, w3, w2 = up(inp.w1), up(inp.w3), up(inp.w2)
    D = dm.Dims(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k,
                dm.DMOE_F32 if cfg.dtype == "f32" else dm.DMOE_BF16)
    mode = "fused" if args.fused_gather else args.gather
    fused = cfg.dtype == "bf16" and (
        mode == "fused" or (mode == "auto" and dm.fused_gather_pays(D)))
    layer = dm.DMoELayer(D, dev, fused_gather=fused)
    fwd_kernels = [n for n in FWD_KERNELS if not (fused and n == "padded_gather")]
    bwd_kernels = list(BWD_KERNELS)
    if fused:   # the backward gathers x_perm right before the up dgrad
        bwd_kernels.insert(bwd_kernels.index("gemm_up_dgrad"), "padded_gather")
    y = torch.empty(cfg.T, cfg.H, dtype=dt, device=dev)
    grads = dict(dx=torch.empty(cfg.T, cfg.H, dtype=dt, device=dev),
                 dw1=torch.empty_like(w1), dw3=torch.empty_like(w3),
                 dw2=torch.empty_like(w2),
                 d_weights=torch.empty(cfg.T, cfg.k, dtype=torch.float32, device=dev))
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        layer.metadata(ids, stream, ev[0] if ev else None)
        layer.forward(x, ids, w, w1, w3, w2, y=y, stream=stream, run_metadata=False,
                      events=ev[1] if ev else None)
        layer.backward(dy, w, w1, w3, w2, grads=grads, stream=stream,
                       events=ev[2] if ev else None)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    P = int(layer.buf.meta.num_padded_rows.item())
    assert int(layer.buf.meta.status.item()) == 0

    K = args.steps
    phases = (META_KERNELS, fwd_kernels, bwd_kernels)
    names = META_KERNELS + fwd_kernels + bwd_kernels

    # Per-kernel table: a pass of its own, outside the timed region, with an
    # event around every kernel (each record puts a timestamp between two
    # kernels, ~5 us each at 15 per step).
    KP = max(3, min(K, 10))
    evs = [tuple(EventArray(len(ks) + 1) for ks in phases) for _ in range(KP)]
    for i in range(KP):
        step(evs[i])
    torch.cuda.synchronize()
    raw = {n: 0.0 for n in names}
    for ev in evs:
        for arr, ks in zip(ev, phases):
            for j, n in enumerate(ks):
                raw[n] += arr.elapsed_ms(j, j + 1) / KP
            arr.close()
    # every interval carries one record's cost; kernel durations are the
    # intervals less the interval between two records with nothing between
    ovh = event_overhead_ms(stream)
    per = {n: max(raw[n] - ovh, 0.0) for n in names}
    dom = max(names, key=lambda n: per[n])
    dph = next(i for i, ks in enumerate(phases) if dom in ks)
    dj = phases[dph].index(dom)

    # The timed region: K steps with two event records, around the dominant
    # kernel, whose duration the roofline takes from here.
    evs = []
    for _ in range(K):
        ev = [None, None, None]
        ev[dph] = EventArray(len(phases[dph]) + 1, only=(dj, dj + 1))
        evs.append(tuple(ev))
    # The shader clock is sampled every ~1 ms by a thread of its own while the
    # steps run: a sysfs read of it takes about a millisecond, so polling it
    # in the wait for the last step would notice the end late.
    sclk = []
    stop = threading.Event()

    def sample():
        while not stop.is_set() and len(sclk) < 1000:
            c = gpu_sclk_mhz()
            if c is None:
                break
            sclk.append(c)
            stop.wait(0.001)

    sampler = threading.Thread(target=sample, daemon=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(evs[i])
        if i == 0:
            sampler.start()        # while the first step runs
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stop.set()
    sampler.join()
    dom_raw_ms = sum(ev[dph].elapsed_ms(dj, dj + 1) for ev in evs) / K
    dom_ms = dom_raw_ms - ovh
    for ev in evs:
        ev[dph].close()

    ms = elapsed * 1e3 / K
    tokens_s = cfg.T / (ms * 1e-3)
    useful_flop = 18.0 * cfg.T * cfg.k * cfg.H * cfg.F
    executed_flop = 18.0 * P * cfg.H * cfg.F
    peak = PEAK_F32_TFLOPS if cfg.dtype == "f32" else PEAK_BF16_TFLOPS
    useful_tf = useful_flop / (ms * 1e-3) / 1e12
    work = kernel_work(cfg, P, fused)
    table = {}
    for n in names:
        fl, by = work[n]
        t = per[n] * 1e-3
        table[n] = {"ms": round(per[n], 4), "interval_ms": round(raw[n], 4),
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
    fl, by = work[dom]
    # the binding roof at the kernel's arithmetic intensity (algorithmic FLOP
    # per unique byte): the matrix cores above the ridge, HBM below it
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    intensity = fl / by if fl else 0.0
    t_dom = dom_ms * 1e-3
    if fl and intensity >= ridge:
        achieved = fl / t_dom / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1),
                "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": None}
    else:
        achieved = by / t_dom / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    roof["intensity_flop_per_byte"] = round(intensity, 1)
    roof["ridge_flop_per_byte"] = round(ridge, 1)
    if fl:
        roof["tflops"] = round(fl / t_dom / 1e12, 1)
        roof["tflops_frac_of_mfma_peak"] = round(fl / t_dom / 1e12 / peak, 4)
    if fl and sclk:
        # the published peak assumes the 2.4 GHz top clock; the matrix cores
        # scale with the clock the chip holds under this load
        at_clk = peak * (sorted(sclk)[len(sclk) // 2] / 2400.0)
        roof["mfma_peak_at_median_sclk"] = round(at_clk, 1)
        roof["tflops_frac_at_median_sclk"] = round(fl / t_dom / 1e12 / at_clk, 4)
    roof["launch_ms"] = round(dom_ms, 4)
    roof["event_interval_ms"] = round(dom_raw_ms, 4)
    roof["algorithmic_bytes_per_launch"] = by
    roof["algorithmic_flop_per_launch"] = fl
    roof["traffic"] = committed_traffic(dom, cfg.name)

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
                              "backward" if fused else "padded copy in the forward")},
        "useful_tflops": round(useful_tf, 1),
        "useful_frac_peak": round(useful_tf / peak, 4),
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
        "sclk_mhz_during_timing": ({"samples": len(sclk), "min": min(sclk),
                                    "median": sorted(sclk)[len(sclk) // 2],
                                    "max": max(sclk)} if sclk else None),
        "roofline": roof,
        "kernels": table,
        "event_overhead_us": round(ovh * 1e3, 2),
        "kernels_note": (f"per-kernel ms from {KP} untimed steps with an event around every "
                         f"kernel; roofline.kernel timed inside the {K} timed steps; ms = "
                         f"interval_ms less event_overhead_us, the interval between two "
                         f"records with nothing between them"),
    }
    out["router_us"] = router_time(dm, cfg, dev, stream, K)
    cold = cold_steps(step, stream, min(K, 10))
    out["cold_cache"] = {"ms_per_step_median": round(cold, 4),
                         "tokens_s": round(cfg.T / (cold * 1e-3), 1),
                         "note": "last-level cache flushed by a 512 MB write before each step"}
    if args.kernels:
        for n in names:
            print(f"{n:22s} {table[n]}", file=sys.stderr)
    if args.calibrate_copy_mb:
        nbytes = args.calibrate_copy_mb << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["calibration_copy_bytes"] = nbytes
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(inp)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
