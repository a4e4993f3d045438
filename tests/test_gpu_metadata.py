"""Routing metadata on the GPU vs the oracle: bit-exact (integer work with
one correct answer, the sort being stable)."""
import json
import os

import numpy as np
import pytest
import torch

import dropless_mixture_experts_amd as dm
import oracle
from workloads import CONFIGS, make_inputs

from gpu_helpers import device, dims_of, schedule_tables, up

pytestmark = pytest.mark.gpu

KEYS = ("tokens_per_expert", "bins", "padded_bins", "indices", "bin_ids",
        "row_of_entry", "tile_expert")


def _run_meta(ids_np, E, dtype=dm.DMOE_BF16, H=128, F=128):
    dev = device()
    T, k = ids_np.shape
    D = dm.Dims(T, H, F, E, k, dtype)
    meta, ws = dm.allocate_meta(D, dev)
    # poison the outputs: anything left unwritten shows up
    for name in KEYS:
        getattr(meta, name).fill_(-12345)
    meta.status.fill_(777)
    meta.row_token.fill_(-12345)
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).to(dev)
    print(f"metadata T={T} k={k} E={E}", flush=True)
    dm.dmoe_metadata(D, ids, meta, ws)
    torch.cuda.synchronize()
    out = {k: getattr(meta, k).cpu().numpy().astype(np.int64) for k in KEYS}
    out["P"] = int(meta.num_padded_rows.item())
    out["status"] = int(meta.status.item())
    sched = schedule_tables(meta, dm.dmoe_max_tiles(D))
    out["pair_first"] = sched["pair_first"]
    out["num_pairs"] = sched["num_pairs"]
    out["row_token"] = meta.row_token.cpu().numpy().astype(np.int64)
    return out, dm.dmoe_max_tiles(D)


def _check_pairs(got):
    """The row-block groups: each expert's blocks in order, two at a time
    (an odd last block alone), every block exactly once, -1 afterwards."""
    te = got["tile_expert"]
    nb = got["P"] // 128
    expect = []
    r = 0
    while r < nb:
        expect.append(r)
        r += 2 if r + 1 < nb and te[r + 1] == te[r] else 1
    S = got["num_pairs"]
    assert S == len(expect)
    np.testing.assert_array_equal(got["pair_first"][:S], expect)
    assert np.all(got["pair_first"][S:] == -1)


def _compare(ids_np, E):
    got, nt = _run_meta(ids_np, E)
    ref = oracle.metadata(ids_np, E, nt)
    assert got["status"] == 0
    for key in KEYS:
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    assert got["P"] == ref["P"]
    _check_pairs(got)
    P = ref["P"]
    np.testing.assert_array_equal(got["row_token"][:P], oracle.row_token(ref, ids_np.shape[1]),
                                  err_msg="row_token")
    assert np.all(got["row_token"][P:] == -12345)     # rows from P on untouched
    return got


def test_hand_worked_fixtures():
    path = os.path.join(os.path.dirname(__file__), "golden", "metadata_hand.json")
    for case in json.load(open(path)):
        ids = np.asarray(case["top_experts"], dtype=np.int32)
        got, nt = _run_meta(ids, case["E"])
        assert nt == case["max_tiles"]
        for key in KEYS:
            np.testing.assert_array_equal(got[key], case[key],
                                          err_msg=f"{case['name']} {key}")
        assert got["P"] == case["P"]


@pytest.mark.parametrize("name", ["tiny_f32", "fine_e64", "zipf_e64",
                                  "zipf_e64_empty", "coarse_e8", "sparse_e256"])
def test_workload_routing_full_size(name):
    cfg = CONFIGS[name]
    inp = make_inputs(cfg.replace(H=8, F=8), with_weights=False, with_dy=False)
    got = _compare(inp.top_experts, cfg.E)
    if name == "zipf_e64_empty":
        assert np.sum(got["tokens_per_expert"] == 0) == 8


@pytest.mark.parametrize("E", [1, 2, 3, 8, 64, 255, 256])
@pytest.mark.parametrize("n", [1, 63, 64, 65, 1000, 32771, 131072])
def test_fuzz_shapes(E, n):
    rng = np.random.default_rng(E * 1000003 + n)
    k = 1 if n % 2 else min(2, E)
    T = max(1, n // k)
    p = rng.dirichlet(np.full(E, 0.2))
    ids = rng.choice(E, size=(T, k), p=p).astype(np.int32)
    _compare(ids, E)


def test_many_chunks_larger_than_minimum():
    # 2^23 entries: more than 4096 chunks of 1024, so chunks grow beyond 1024
    rng = np.random.default_rng(5)
    ids = rng.integers(0, 64, size=(1 << 20, 8)).astype(np.int32)
    _compare(ids, 64)


def test_all_entries_one_expert_and_k_equals_E():
    _compare(np.full((3000, 1), 7, dtype=np.int32), 8)
    rng = np.random.default_rng(1)
    ids = np.stack([rng.permutation(8) for _ in range(700)]).astype(np.int32)
    _compare(ids, 8)


def test_invalid_expert_id_sets_status():
    ids = np.array([[0, 1], [5, 2], [1, -1], [2, 0]], dtype=np.int32)
    got, _ = _run_meta(ids, 3)
    assert got["status"] == -5
    flat = ids.reshape(-1)
    bad = (flat < 0) | (flat >= 3)
    assert np.all(got["row_of_entry"][bad] == -1)
    valid = ~bad
    assert got["tokens_per_expert"].sum() == valid.sum()


def test_deterministic():
    rng = np.random.default_rng(9)
    ids = rng.integers(0, 256, size=(16384, 8)).astype(np.int32)
    a, _ = _run_meta(ids, 256)
    b, _ = _run_meta(ids, 256)
    for key in KEYS:
        np.testing.assert_array_equal(a[key], b[key])
