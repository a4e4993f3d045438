"""Router parity on the GPU: dmoe_router_forward / dmoe_router_backward
through the C ABI against oracle.router on the same seeded logits.

Ids must match bit for bit (the selection is unique: equal logits go to the
lower expert id).  Weights, z, the z-loss and d_logits are fp32 on the GPU
and fp64 in the oracle; the bar is max|err| <= 1e-5 * max|ref| per tensor
(a few fp32 ulps of the softmax's exp and sums)."""
import numpy as np
import pytest
import torch

import dropless_mixture_experts_amd as dm
import workloads as W
from oracle import router as R

from gpu_helpers import assert_close, device

pytestmark = pytest.mark.gpu

TOL = 1e-5

CASES = [
    ("fine_e64", {}, False),
    ("sparse_e256", {}, False),
    ("coarse_e8", {}, False),
    ("tiny_f32", {}, False),
    ("tiny_f32", {"T": 1}, False),                  # one token
    ("tiny_f32", {"T": 37, "k": 8}, False),         # k = E, ragged last workgroup
    ("tiny_f32", {"T": 129, "E": 1, "k": 1}, False),  # one expert
    ("sparse_e256", {"T": 61, "k": 256}, False),    # k = E = 256: four slots per lane
    ("sparse_e256", {"T": 300, "E": 100, "k": 70}, False),  # ragged E, k > 64
    ("fine_e64", {"T": 515}, True),                 # ties among the top k
    ("sparse_e256", {"T": 515}, True),
]


def _cfg(name, dims):
    c = W.CONFIGS[name]
    return W.shrink(c, **dims) if dims else c


def _dims(cfg):
    return dm.Dims(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, dm.DMOE_F32)


def _run(cfg, logits, d_weights, coef):
    dev = device()
    T, E, k = cfg.T, cfg.E, cfg.k
    D = _dims(cfg)
    l = torch.from_numpy(logits).to(dev)
    ids = torch.full((T, k), -7, dtype=torch.int32, device=dev)
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device=dev)
    z = torch.full((T,), float("nan"), dtype=torch.float32, device=dev)
    zl = torch.full((1,), float("nan"), dtype=torch.float32, device=dev)
    dm.dmoe_router_forward(D, l, ids, w, zloss_coef=coef, z=z, zloss=zl)
    g = torch.from_numpy(d_weights).to(dev)
    dl = torch.full((T, E), float("nan"), dtype=torch.float32, device=dev)
    dm.dmoe_router_backward(D, l, ids, w, g, dl, zloss_coef=coef)
    torch.cuda.synchronize()
    return (ids.cpu().numpy(), w.cpu().numpy(), z.cpu().numpy(), float(zl.item()),
            dl.cpu().numpy())


@pytest.mark.parametrize("coef", [0.0, 0.001])
@pytest.mark.parametrize("name,dims,ties", CASES,
                         ids=[f"{n}-{'_'.join(f'{a}{b}' for a, b in d.items()) or 'full'}"
                              f"{'-ties' if t else ''}" for n, d, t in CASES])
def test_router_parity(name, dims, ties, coef):
    cfg = _cfg(name, dims)
    logits, d_weights = W.make_logits(cfg, ties=ties)
    print(f"router case {cfg.name} T={cfg.T} E={cfg.E} k={cfg.k} ties={ties} coef={coef}",
          flush=True)
    ids, w, z, zl, dl = _run(cfg, logits, d_weights, coef)

    ref_ids, ref_w = R.router_forward(logits, cfg.k)
    assert np.array_equal(ids.astype(np.int64), ref_ids), "top_experts differ"
    assert_close(w, ref_w, TOL, "weights")
    if coef != 0.0:
        ref_zl, ref_z = R.zloss(logits, coef)
        assert_close(z, ref_z, TOL, "z")
        assert abs(zl - ref_zl) <= TOL * abs(ref_zl), (zl, ref_zl)
    # Backward on the GPU's own forward outputs (identical ids, fp32 weights).
    ref_dl = R.router_backward(logits, ids, w, d_weights, coef)
    assert_close(dl, ref_dl, TOL, "d_logits")
    # Unchosen experts get exactly zero without the z-loss.
    if coef == 0.0:
        mask = np.ones_like(dl, dtype=bool)
        np.put_along_axis(mask, ids.astype(np.int64), False, axis=1)
        assert np.all(dl[mask] == 0.0)


def test_router_ids_match_input_recipe():
    """The router on the Gaussian recipe's logits picks the recipe's experts."""
    cfg = W.CONFIGS["fine_e64"]
    logits, d_weights = W.make_logits(cfg)
    inp = W.make_inputs(cfg, with_weights=False, with_dy=False)
    ids, w, _, _, _ = _run(cfg, logits, d_weights, 0.0)
    assert np.array_equal(ids, inp.top_experts)
    assert_close(w, inp.weights, TOL, "weights")


def test_router_rejects_missing_zloss_buffers():
    cfg = W.CONFIGS["tiny_f32"]
    dev = device()
    D = _dims(cfg)
    l = torch.zeros(cfg.T, cfg.E, device=dev)
    ids = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device=dev)
    w = torch.empty(cfg.T, cfg.k, device=dev)
    with pytest.raises(ValueError):
        dm.dmoe_router_forward(D, l, ids, w, zloss_coef=0.5)


@pytest.mark.parametrize("E,k", [(64, 8), (256, 8), (100, 70)])
def test_router_ids_on_signed_zeros_subnormals_and_extremes(E, k):
    """Rows drawn from a handful of values, so that most of the top k are
    ties: +0 and -0 (one value), subnormals of both signs, +-FLT_MAX and
    ordinary values.  Ids must equal the oracle's stable order exactly."""
    vals = np.array([0.0, -0.0, 1e-40, -1e-40, 2e-45, 1.5, -1.5, 3.0,
                     np.finfo(np.float32).max, -np.finfo(np.float32).max],
                    dtype=np.float32)
    rng = np.random.default_rng(4242 + E)
    T = 96
    logits = vals[rng.integers(0, len(vals), size=(T, E))].astype(np.float32)
    d_weights = rng.standard_normal((T, k)).astype(np.float32)
    cfg = W.shrink(W.CONFIGS["sparse_e256"], T=T, E=E, k=k)
    print(f"router extremes E={E} k={k}", flush=True)
    ids, w, _, _, dl = _run(cfg, logits, d_weights, 0.0)
    ref_ids, ref_w = R.router_forward(logits, k)
    assert np.array_equal(ids.astype(np.int64), ref_ids), "top_experts differ"
    assert_close(w, ref_w, TOL, "weights")
    assert np.all(np.isfinite(dl))
