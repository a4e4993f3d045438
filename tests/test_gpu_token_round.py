"""Tile-aware token rounding on the GPU against the oracle (ids bit-exact,
weights within 1e-6 of the fp64 softmax), and the layer run on the rounded
slots, whose experts then need no pad rows."""
import dataclasses
import json
import os

import numpy as np
import pytest
import torch

import dropless_mixture_experts_amd as dm
import oracle
from oracle.token_round import token_round
from workloads import CONFIGS, make_inputs, make_logits, shrink

from gpu_helpers import TOL, Run, assert_close, device, down

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "token_round_hand.json")


def _gpu_round(logits, k, M):
    dev = device()
    T, E = logits.shape
    D = dm.Dims(T, 128, 128, E, k, dm.DMOE_F32)
    l = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).to(dev)
    ids = torch.full((T, k + 1), -7, dtype=torch.int32, device=dev)
    w = torch.full((T, k + 1), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(dm.dmoe_token_round_workspace_bytes(D), dtype=torch.uint8, device=dev)
    dm.dmoe_token_round(D, l, ids, w, ws, tile_rows=M)
    torch.cuda.synchronize()
    return ids.cpu().numpy().astype(np.int64), w.cpu().numpy().astype(np.float64)


def _compare(logits, k, M, name):
    print(f"token round {name} T={logits.shape[0]} E={logits.shape[1]} k={k} M={M}", flush=True)
    ids, w = _gpu_round(logits, k, M)
    ref_ids, ref_w, info = token_round(logits, k, M)
    np.testing.assert_array_equal(ids, ref_ids, err_msg=name)
    assert float(np.max(np.abs(w - ref_w))) <= 1e-6, name
    n = np.bincount(ids[ids >= 0], minlength=logits.shape[1])
    assert np.all(n % M == 0)
    return ids, w


def test_hand_worked_cases():
    with open(GOLDEN) as f:
        cases = json.load(f)
    for c in cases:
        ids, w = _gpu_round(np.asarray(c["logits"], np.float32), c["k"], c["M"])
        np.testing.assert_array_equal(ids, c["ids"], err_msg=c["name"])
        assert float(np.max(np.abs(w - np.asarray(c["weights"])))) <= 1e-6, c["name"]


@pytest.mark.parametrize("T,E,k,M,ties,seed", [
    (1, 2, 1, 128, False, 0), (300, 8, 2, 16, True, 1), (1000, 16, 4, 32, False, 2),
    (777, 5, 4, 8, True, 3), (64, 256, 255, 4, False, 4), (5000, 3, 1, 128, True, 5)])
def test_random_logits(T, E, k, M, ties, seed):
    rng = np.random.default_rng(seed)
    l = rng.standard_normal((T, E)).astype(np.float32)
    if ties:
        l = np.round(l * 2) / 2
        l[rng.random((T, E)) < 0.1] = -0.0
    _compare(l, k, M, f"random{seed}")


@pytest.mark.parametrize("name", ["fine_e64", "coarse_e8", "sparse_e256"])
def test_workload_logits(name):
    cfg = CONFIGS[name]
    logits, _ = make_logits(cfg)
    _compare(logits, cfg.k, 128, name)


def test_rejects_bad_arguments():
    dev = device()
    l = torch.zeros(4, 2, dtype=torch.float32, device=dev)
    ids = torch.empty(4, 3, dtype=torch.int32, device=dev)
    w = torch.empty(4, 3, dtype=torch.float32, device=dev)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    with pytest.raises(dm.DMoEError):        # k = E: no candidate
        dm.dmoe_token_round(dm.Dims(4, 128, 128, 2, 2, dm.DMOE_F32), l, ids, w, ws)
    with pytest.raises(dm.DMoEError):        # a tile of no rows
        dm.dmoe_token_round(dm.Dims(4, 128, 128, 2, 1, dm.DMOE_F32), l, ids, w, ws, tile_rows=0)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["sparse_e256", "fine_e64"])
def test_layer_on_rounded_slots(name):
    """The token-rounded routing (k + 1 slots, some empty) through the whole
    layer at full size: metadata bit-exact with no pad rows, every output
    and intermediate element by element against the oracle."""
    cfg = CONFIGS[name]
    logits, _ = make_logits(cfg)
    ids, w = _compare(logits, cfg.k, 128, name)
    inp = make_inputs(cfg)
    inp = dataclasses.replace(inp, cfg=cfg.replace(k=cfg.k + 1), top_experts=ids.astype(np.int32),
                              weights=w.astype(np.float32))
    print(f"layer on rounded slots {name}", flush=True)
    r = Run(inp)
    md = oracle.metadata(inp.top_experts, cfg.E, len(r.meta.tile_expert))
    got = r.meta_np()
    for key in ("tokens_per_expert", "bins", "padded_bins", "indices", "bin_ids",
                "row_of_entry", "tile_expert"):
        np.testing.assert_array_equal(got[key], md[key], err_msg=key)
    # no pad rows: P is the number of occupied slots
    assert r.P == md["P"] == int((ids >= 0).sum())
    assert np.all(md["tokens_per_expert"] % 128 == 0)
    from test_gpu_layer import _elementwise
    _elementwise(r, inp, md, TOL[cfg.dtype], name + "_rounded")
    # an empty slot's routing-weight gradient is exactly 0
    assert np.all(down(r.g["d_weights"])[ids < 0] == 0.0)


@pytest.mark.parametrize("cfg", [
    shrink(CONFIGS["zipf_e64_empty"], T=700, H=256, F=256),
    shrink(CONFIGS["tiny_f32"], T=300, H=128, F=256),
    shrink(CONFIGS["fine_e64"], T=200, H=128, F=128, E=4, k=4),
], ids=lambda c: c.name)
def test_layer_with_random_empty_slots(cfg):
    """Slots set to -1 at random (whole tokens included): metadata
    bit-exact, status 0, every output and intermediate against the oracle."""
    inp = make_inputs(cfg)
    rng = np.random.default_rng(99)
    ids = inp.top_experts.copy()
    ids[rng.random(ids.shape) < 0.3] = -1
    ids[:3] = -1                             # tokens with no expert at all
    inp = dataclasses.replace(inp, top_experts=ids)
    print(f"empty slots {cfg.name}", flush=True)
    r = Run(inp)
    md = oracle.metadata(ids, cfg.E, len(r.meta.tile_expert))
    got = r.meta_np()
    for key in ("tokens_per_expert", "bins", "padded_bins", "indices", "bin_ids",
                "row_of_entry", "tile_expert"):
        np.testing.assert_array_equal(got[key], md[key], err_msg=key)
    assert r.P == md["P"]
    from test_gpu_layer import _elementwise
    _elementwise(r, inp, md, TOL[cfg.dtype], cfg.name + "_empty_slots")
    assert np.all(down(r.g["d_weights"])[ids < 0] == 0.0)
    assert np.all(down(r.y)[:3] == 0.0) and np.all(down(r.g["dx"])[:3] == 0.0)
