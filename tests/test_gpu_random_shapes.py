"""A seeded sweep of random layer shapes on the GPU against the oracle.

Each case draws T, H, F (multiples of 128), E <= 256, k <= min(E, 8), the
dtype and the routing (Gaussian or Zipf) from one seed, so that tile
counts, ragged tails, odd multiples of 128, empty and single-block experts
and the merged and split launches all get mixed.  bf16 cases also run the
fused-gather path, which must be bitwise equal to the plain one."""
import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, make_inputs, shrink

from gpu_helpers import TOL, Run, assert_close, down

pytestmark = pytest.mark.gpu

OUTS = ("dx", "dw1", "dw3", "dw2", "d_weights")


def _case(i):
    rng = np.random.default_rng(9000 + i)
    E = int(rng.choice([1, 2, 3, 5, 8, 13, 32, 64, 100, 256]))
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.choice([1, 7, 64, 129, 300, 777, 1500, 2500]))
    H = 128 * int(rng.integers(1, 9))
    F = 128 * int(rng.integers(1, 9))
    f32 = bool(rng.random() < 0.25)
    zipf = not f32 and bool(rng.random() < 0.4)
    base = CONFIGS["tiny_f32"] if f32 else CONFIGS["zipf_e64" if zipf else "fine_e64"]
    return shrink(base, T=T, H=H, F=F, E=E, k=k)


CASES = [_case(i) for i in range(24)]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_random_shape_against_oracle(cfg):
    inp = make_inputs(cfg)
    print(f"random {cfg.name} dtype={cfg.dtype} routing={cfg.routing}", flush=True)
    r = Run(inp)
    tol = TOL[cfg.dtype]
    ref_y, sv = oracle.forward_padded(inp.x, inp.top_experts, inp.weights,
                                      inp.w1, inp.w3, inp.w2)
    ref_g = oracle.backward_padded(inp.x, inp.top_experts, inp.weights, inp.w1,
                                   inp.w3, inp.w2, inp.dy, sv)
    md = sv["md"]
    assert r.P == md["P"]
    np.testing.assert_array_equal(r.meta_np()["row_of_entry"], md["row_of_entry"])
    assert np.array_equal(down(r.saved.x_perm[:r.P]), sv["x_perm"])
    assert_close(down(r.y), ref_y, tol, "y")
    for key in OUTS:
        assert_close(down(r.g[key]), ref_g[key], tol, key)
    if cfg.dtype == "bf16" and cfg.T * cfg.H * 2 < (1 << 31):
        f = Run(inp, fused_gather=True)
        assert torch.equal(f.y, r.y)
        for key in OUTS:
            assert torch.equal(f.g[key], r.g[key]), key
