"""The gather fused into the up projection's operand loads
(dmoe_forward_fused_gather / dmoe_backward_fused_gather) on the GPU.

The fused up projection feeds the matrix cores the very values the plain
path copies into x_perm (token rows of x, zeros on pad rows), in the same
order, and the fused backward gathers x_perm itself before the products that
read it, so every output and every saved or scratch buffer must equal the
plain path's bit for bit.  The plain path itself is checked against the
oracle in test_gpu_layer.py; here the fused outputs are also compared with
the oracle directly on the small cases."""
import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, make_inputs, shrink

from gpu_helpers import TOL, Run, assert_close, down, torch_dtype, up

pytestmark = pytest.mark.gpu

OUTS = ("dx", "dw1", "dw3", "dw2", "d_weights")

SMALL = [
    shrink(CONFIGS["fine_e64"], T=512, H=256, F=256),
    shrink(CONFIGS["zipf_e64_empty"], T=1024, H=128, F=256),      # empty experts
    shrink(CONFIGS["coarse_e8"], T=1024, H=512, F=1024),
    shrink(CONFIGS["sparse_e256"], T=2048, H=384, F=256),         # odd H/128
    shrink(CONFIGS["fine_e64"], T=5, H=128, F=128, E=1, k=1),     # one expert, ragged
    shrink(CONFIGS["fine_e64"], T=1, H=256, F=128, E=4, k=2),     # one token
    shrink(CONFIGS["fine_e64"], T=200, H=128, F=128, E=4, k=4),   # k = E
    shrink(CONFIGS["sparse_e256"], T=16, H=128, F=128),           # most experts empty
    # the up-dgrad launch without the dw1/dw3 tail fill
    shrink(CONFIGS["fine_e64"], T=3584, H=2048, F=128, E=8, k=2),
    # an expert of 17 row pairs: row groups of 6, 6 and 5
    shrink(CONFIGS["fine_e64"], T=4300, H=128, F=256, E=1, k=1),
]


def _compare_bitwise(a, b):
    P = a.P
    assert b.P == P
    assert torch.equal(a.y, b.y), "y"
    for key in OUTS:
        assert torch.equal(a.g[key], b.g[key]), key
    for key in ("x_perm", "h1", "h3", "act", "y_perm"):
        assert torch.equal(getattr(a.saved, key)[:P], getattr(b.saved, key)[:P]), key
    for key in ("dy_perm", "dh1", "dh3", "dx_perm"):
        assert torch.equal(getattr(a.scratch, key)[:P], getattr(b.scratch, key)[:P]), key


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: f"{c.name}-T{c.T}-H{c.H}-E{c.E}-k{c.k}")
def test_small_case_bitwise_and_against_oracle(cfg):
    inp = make_inputs(cfg)
    print(f"fused gather {cfg.name} T={cfg.T} H={cfg.H} F={cfg.F} E={cfg.E} k={cfg.k}",
          flush=True)
    a = Run(inp)
    b = Run(inp, fused_gather=True)
    _compare_bitwise(a, b)
    tol = TOL[cfg.dtype]
    ref_y, sv = oracle.forward_padded(inp.x, inp.top_experts, inp.weights,
                                      inp.w1, inp.w3, inp.w2)
    ref_g = oracle.backward_padded(inp.x, inp.top_experts, inp.weights, inp.w1,
                                   inp.w3, inp.w2, inp.dy, sv)
    assert_close(down(b.y), ref_y, tol, "y")
    for key in OUTS:
        assert_close(down(b.g[key]), ref_g[key], tol, key)
    P = b.P
    assert_close(down(b.saved.h1[:P]), sv["h1"], tol, "h1")
    assert_close(down(b.saved.h3[:P]), sv["h3"], tol, "h3")


@pytest.mark.parametrize("name", ["fine_e64", "zipf_e64_empty", "coarse_e8", "sparse_e256"])
def test_full_size_bitwise(name):
    """At the benchmark's sizes and launch configuration."""
    inp = make_inputs(CONFIGS[name])
    print(f"fused gather full {name}", flush=True)
    a = Run(inp)
    b = Run(inp, fused_gather=True)
    _compare_bitwise(a, b)


def test_forward_writes_no_x_perm_and_backward_gathers_it():
    """saved.x_perm is not touched by the fused forward (NaN stays NaN) and
    holds exactly the gathered rows after the fused backward."""
    cfg = shrink(CONFIGS["zipf_e64_empty"], T=600, H=256, F=256)
    inp = make_inputs(cfg)
    print(f"fused gather x_perm {cfg.name}", flush=True)
    a = Run(inp)
    b = Run(inp, fused_gather=True, backward=False)
    P = b.P
    xp = b.saved.x_perm
    xp.fill_(float("nan"))
    b.layer.forward(b.x, b.ids, b.w, b.w1, b.w3, b.w2)
    torch.cuda.synchronize()
    assert bool(torch.isnan(xp).all())
    assert torch.equal(b.y, a.y)
    g = b.layer.backward(up(inp.dy, torch_dtype(cfg), b.dev), b.w, b.w1, b.w3, b.w2)
    torch.cuda.synchronize()
    assert torch.equal(xp[:P], a.saved.x_perm[:P])
    for key in OUTS:
        assert torch.equal(g[key], a.g[key]), key


def test_fp32_is_rejected():
    from dropless_mixture_experts_amd import DMoEError
    inp = make_inputs(shrink(CONFIGS["tiny_f32"], T=64))
    with pytest.raises(DMoEError):
        Run(inp, fused_gather=True)
