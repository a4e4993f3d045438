"""Host-side logic of bench.py (no GPU): the per-kernel work model, the
roofline time, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

import bench
from workloads import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name", ["fine_e64", "coarse_e8", "sparse_e256", "tiny_f32"])
def test_gemm_flops_add_up_to_the_executed_work(name):
    """The five GEMM launches execute 18 P H F FLOPs in all: forward 6, down
    dgrad and dw2 4, up dgrad 4, dw1/dw3 4 (2 P H F each per product)."""
    cfg = CONFIGS[name]
    P = 128 * (cfg.T * cfg.k // 128 + cfg.E)
    w = bench.kernel_work(cfg, P)
    gemms = [n for n in w if n.startswith("gemm")]
    assert len(gemms) == 5
    assert sum(w[n][0] for n in gemms) == 18 * P * cfg.H * cfg.F
    for n in w:
        if not n.startswith("gemm"):
            assert w[n][0] == 0, n
        assert w[n][1] > 0, n


def test_fused_gather_moves_the_x_reads_only():
    """With the gather fused, the up projection reads the T token rows of x
    instead of the P padded rows; nothing else changes."""
    cfg = CONFIGS["fine_e64"]
    P = 36736
    s = 2
    a = bench.kernel_work(cfg, P)
    b = bench.kernel_work(cfg, P, fused=True)
    assert a["gemm_up_gate"][1] - b["gemm_up_gate"][1] == (P - cfg.T) * cfg.H * s
    for n in a:
        if n != "gemm_up_gate":
            assert a[n] == b[n], n


def test_permutation_bytes_are_symmetric():
    """The forward scatter and the gather's backward move the same rows (the
    scatter also reads the fp32 routing weights); the gather and its
    backward differ only by reading P padded rows against T k entry rows."""
    cfg = CONFIGS["sparse_e256"]
    P = 146304
    w = bench.kernel_work(cfg, P)
    N = cfg.T * cfg.k
    assert w["padded_scatter"][1] - w["gather_backward"][1] == 4 * N
    assert w["padded_gather"][1] - w["gather_backward"][1] == (P - N) * cfg.H * 2


def test_moa_work_model():
    """The dMoA calls execute 12 P H F FLOPs in all (map and reduce 2 each,
    their backward 4 each).  With H = F the map and the reduce move the
    same bytes but for the reduce's fp32 routing weights.  Each backward
    adds one weight-gradient product (P H + P F reads, E H F writes) to its
    forward's traffic.  In the reduce's backward the scatter's backward also
    writes the P padded rows of do_perm, and the slot unpermute moves 2 N
    rows where the forward's slot permute moves N + P (net N H with H = F);
    it reads the routing weights and writes d_weights (8 bytes per entry
    against the forward's 4)."""
    cfg = CONFIGS["moa_e16"]
    assert cfg.H == cfg.F
    P = 128 * (cfg.T * cfg.k // 128 + cfg.E)
    w = bench.moa_work(cfg, P)
    assert set(w) == set(bench.MOA_CALLS)
    assert sum(w[n][0] for n in w) == 12 * P * cfg.H * cfg.F
    T, H, F, E, k = cfg.T, cfg.H, cfg.F, cfg.E, cfg.k
    N = T * k
    assert w["moa_reduce"][1] - w["moa_map"][1] == 4 * N
    wg = (P * H + P * F + E * H * F) * 2
    assert w["moa_map_backward"][1] - w["moa_map"][1] == wg
    assert w["moa_reduce_backward"][1] - w["moa_reduce"][1] == wg + N * H * 2 + 4 * N


def test_roof_time_takes_the_binding_roof():
    # 1 GFLOP and 1 MB: MFMA-bound (0.4 us against 0.125 us)
    assert bench.roof_time(1e9, 1e6, 2500.0) == pytest.approx(1e9 / 2.5e15)
    # 1 GFLOP and 1 GB: HBM-bound (125 us)
    assert bench.roof_time(1e9, 1e9, 2500.0) == pytest.approx(1e9 / 8e12)
    # a copy kernel has no FLOPs
    assert bench.roof_time(0, 8e9, 2500.0) == pytest.approx(1e-3)
    # at the ridge (312.5 FLOP/B) both roofs agree
    assert bench.roof_time(312.5e9, 1e9, 2500.0) == pytest.approx(1e9 / 8e12)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, env=e, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single-process" in r.stderr
    assert r.stdout == ""
