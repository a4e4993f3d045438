"""padded_gather / padded_scatter on the GPU: the gather is a pure copy and
must match the oracle bit for bit; the unit-weight scatter of a gather is k*x
exactly for k a power of two; the weighted scatter matches the oracle."""
import numpy as np
import pytest
import torch

import dropless_mixture_experts_amd as dm
import oracle
from workloads import CONFIGS, make_inputs, shrink

from gpu_helpers import TOL, assert_close, device, dims_of, down, torch_dtype, up

pytestmark = pytest.mark.gpu


def _setup(cfg):
    dev = device()
    inp = make_inputs(cfg, with_weights=False, with_dy=False)
    D = dims_of(cfg)
    dt = torch_dtype(cfg)
    meta, ws = dm.allocate_meta(D, dev)
    ids = up(inp.top_experts, torch.int32, dev)
    print(f"permute {cfg.name}", flush=True)
    dm.dmoe_metadata(D, ids, meta, ws)
    pm = 128 * dm.dmoe_max_tiles(D)
    return dev, inp, D, dt, meta, pm


CASES = [shrink(CONFIGS["tiny_f32"], T=300),
         shrink(CONFIGS["fine_e64"], T=700, H=256),
         CONFIGS["zipf_e64_empty"].replace(H=128),
         shrink(CONFIGS["sparse_e256"], T=2000, H=384),
         CONFIGS["fine_e64"],
         CONFIGS["sparse_e256"]]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_gather_bit_exact_and_unit_scatter_identity(cfg):
    dev, inp, D, dt, meta, pm = _setup(cfg)
    x = up(inp.x, dt, dev)
    x_perm = torch.full((pm, cfg.H), float("nan"), dtype=dt, device=dev)
    dm.dmoe_padded_gather(D, x, meta, x_perm)
    torch.cuda.synchronize()
    P = int(meta.num_padded_rows.item())
    md = oracle.metadata(inp.top_experts, cfg.E)
    assert P == md["P"]
    got = x_perm[:P].float().cpu().numpy()
    ref = oracle.padded_gather(inp.x, md, cfg.k)
    # bit-exact: both are exact copies of the same representable values
    assert np.array_equal(got.astype(np.float64), ref)
    # rows in [P, P_max) are left untouched
    assert bool(torch.isnan(x_perm[P:].float()).all())
    # gather then unit-weight scatter = k * x (k a power of two: exact)
    if cfg.k in (1, 2, 4, 8):
        out = torch.empty(cfg.T, cfg.H, dtype=dt, device=dev)
        dm.dmoe_padded_scatter(D, x_perm, None, meta, out)
        torch.cuda.synchronize()
        assert torch.equal(out, x * cfg.k)


@pytest.mark.parametrize("cfg", CASES[:4], ids=lambda c: c.name)
def test_weighted_scatter(cfg):
    dev, inp, D, dt, meta, pm = _setup(cfg)
    rng = np.random.default_rng(3)
    md = oracle.metadata(inp.top_experts, cfg.E)
    yp = rng.standard_normal((pm, cfg.H)).astype(np.float32)
    src = up(yp, dt, dev)
    yp_seen = down(src)                 # the values the GPU actually holds
    w = up(inp.weights, torch.float32, dev)
    out = torch.empty(cfg.T, cfg.H, dtype=dt, device=dev)
    dm.dmoe_padded_scatter(D, src, w, meta, out)
    torch.cuda.synchronize()
    ref = oracle.padded_scatter(yp_seen[:md["P"]], md, inp.weights, cfg.T, cfg.k)
    assert_close(down(out), ref, TOL[cfg.dtype], "scatter")
