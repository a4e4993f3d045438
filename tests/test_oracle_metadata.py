"""Pins of the oracle's routing metadata and permutation (CPU only).

The metadata is integer work with one correct answer (the sort is stable), so
every pin here is exact.
"""
import json
import os

import numpy as np
import pytest

import oracle
from workloads import CONFIGS, make_inputs, shrink

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "metadata_hand.json")
KEYS = ("tokens_per_expert", "bins", "padded_bins", "indices", "bin_ids",
        "row_of_entry", "tile_expert")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
@pytest.mark.parametrize("impl", ["library", "counting"])
def test_hand_worked_metadata(case, impl):
    ids = np.asarray(case["top_experts"], dtype=np.int32)
    assert ids.shape == (case["T"], case["k"])
    nt = oracle.max_tiles(case["T"], case["k"], case["E"])
    assert nt == case["max_tiles"]
    fn = oracle.metadata if impl == "library" else oracle.metadata_counting_sort
    md = fn(ids, case["E"], nt)
    for key in KEYS:
        np.testing.assert_array_equal(md[key], case[key], err_msg=key)
    assert md["P"] == case["P"]


def _check_invariants(ids, E, md):
    n = ids.size
    flat = ids.reshape(-1)
    # indices is a permutation of [0, T*k)
    assert np.array_equal(np.sort(md["indices"]), np.arange(n))
    # bin_ids non-decreasing, and consistent with the sort
    assert np.all(np.diff(md["bin_ids"]) >= 0)
    assert np.array_equal(md["bin_ids"], flat[md["indices"]])
    # stability: within a bin the flattened index increases
    same = md["bin_ids"][1:] == md["bin_ids"][:-1]
    assert np.all(np.diff(md["indices"])[same] > 0)
    # sum of the histogram is T*k; bins ends at T*k
    assert md["tokens_per_expert"].sum() == n
    assert md["bins"][-1] == n
    pc = np.diff(np.concatenate([[0], md["padded_bins"]]))
    c = md["tokens_per_expert"]
    # every padded_bins entry is a multiple of 128, waste in [0, 127]
    assert np.all(md["padded_bins"] % 128 == 0)
    assert np.all((pc - c >= 0) & (pc - c <= 127))
    assert np.all(pc[c == 0] == 0)
    # row_of_entry is injective and lies inside its expert's real rows
    rows = md["row_of_entry"]
    assert np.unique(rows).size == n
    start = md["padded_bins"] - pc
    e = flat
    assert np.all(rows >= start[e]) and np.all(rows < start[e] + c[e])
    # one expert per 128-row tile; tiles past P are -1
    P = md["P"]
    te = md["tile_expert"]
    for r, owner in enumerate(te):
        if 128 * r < P:
            assert start[owner] <= 128 * r and 128 * r + 127 < md["padded_bins"][owner]
        else:
            assert owner == -1
    assert P <= 128 * oracle.max_tiles(ids.shape[0], ids.shape[1], E)


@pytest.mark.parametrize("T,k,E,seed", [
    (1, 1, 1, 0), (3, 2, 5, 1), (64, 4, 8, 2), (200, 2, 3, 3),
    (333, 8, 64, 4), (129, 1, 2, 5), (500, 3, 256, 6), (1000, 8, 16, 7)])
def test_library_matches_counting_sort_and_invariants(T, k, E, seed):
    rng = np.random.default_rng(seed)
    # skewed ids so that some experts are empty and some span several tiles
    p = rng.dirichlet(np.full(E, 0.3))
    ids = rng.choice(E, size=(T, k), p=p).astype(np.int32)
    nt = oracle.max_tiles(T, k, E)
    a = oracle.metadata(ids, E, nt)
    b = oracle.metadata_counting_sort(ids, E, nt)
    for key in KEYS:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    assert a["P"] == b["P"]
    _check_invariants(ids, E, a)


@pytest.mark.parametrize("name", ["tiny_f32", "fine_e64", "zipf_e64",
                                  "zipf_e64_empty", "sparse_e256"])
def test_invariants_on_workload_routing(name):
    cfg = CONFIGS[name]
    inp = make_inputs(shrink(cfg, H=8, F=8) if cfg.T * cfg.k > 40000 else
                      cfg.replace(H=8, F=8), with_weights=False, with_dy=False)
    md = oracle.metadata(inp.top_experts, cfg.E,
                         oracle.max_tiles(cfg.T, cfg.k, cfg.E))
    _check_invariants(inp.top_experts, cfg.E, md)
    if name == "zipf_e64_empty":
        assert np.sum(md["tokens_per_expert"] == 0) == 8


def test_duplicate_ids_in_one_token_are_separate_entries():
    ids = np.array([[1, 1], [0, 1]], dtype=np.int32)
    md = oracle.metadata(ids, 2, oracle.max_tiles(2, 2, 2))
    np.testing.assert_array_equal(md["tokens_per_expert"], [1, 3])
    np.testing.assert_array_equal(md["indices"], [2, 0, 1, 3])
    np.testing.assert_array_equal(md["row_of_entry"], [128, 129, 0, 130])


def test_out_of_range_id_rejected():
    with pytest.raises(ValueError):
        oracle.metadata(np.array([[3]]), 3)
    with pytest.raises(ValueError):
        oracle.metadata(np.array([[-2]]), 3)


@pytest.mark.parametrize("T,k,E,seed", [(1, 1, 1, 0), (50, 3, 4, 1), (300, 8, 16, 2),
                                        (129, 2, 3, 3)])
def test_empty_slots(T, k, E, seed):
    """Slots holding -1 are routed nowhere: the routed entries alone give
    the same metadata as a layer without those slots, the sorted arrays end
    in -1, and the counting sort agrees."""
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    ids[rng.random((T, k)) < 0.3] = -1
    if seed == 0:
        ids[:] = -1                          # nothing routed at all
    nt = oracle.max_tiles(T, k, E)
    a = oracle.metadata(ids, E, nt)
    b = oracle.metadata_counting_sort(ids, E, nt)
    for key in KEYS:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    flat = ids.reshape(-1)
    routed = np.nonzero(flat >= 0)[0]
    nv = routed.size
    assert a["bins"][-1] == nv
    np.testing.assert_array_equal(np.sort(a["indices"][:nv]), routed)
    assert np.all(a["indices"][nv:] == -1) and np.all(a["bin_ids"][nv:] == -1)
    assert np.array_equal(a["row_of_entry"] < 0, flat < 0)
    # the routed entries alone, as a one-slot layer of nv "tokens" in order
    c = oracle.metadata(flat[routed].reshape(nv, 1), E, nt)
    for key in ("tokens_per_expert", "bins", "padded_bins", "tile_expert"):
        np.testing.assert_array_equal(a[key], c[key], err_msg=key)
    np.testing.assert_array_equal(a["row_of_entry"][routed], c["row_of_entry"])
    np.testing.assert_array_equal(a["indices"][:nv], routed[c["indices"][:nv]])
    assert a["P"] == c["P"]


@pytest.mark.parametrize("k", [1, 2, 3, 8])
def test_gather_then_unit_scatter_is_k_times_x(k):
    rng = np.random.default_rng(k)
    T, H, E = 77, 5, 6
    ids = np.stack([rng.permutation(E)[:k] if k <= E else rng.integers(0, E, k)
                    for _ in range(T)]).astype(np.int32)
    x = rng.standard_normal((T, H)).astype(np.float32)
    md = oracle.metadata(ids, E)
    xp = oracle.padded_gather(x, md, k)
    # pad rows are exactly zero; real rows are copies
    real = np.zeros(md["P"], dtype=bool)
    real[md["row_of_entry"]] = True
    assert np.all(xp[~real] == 0.0)
    a = np.arange(T * k)
    np.testing.assert_array_equal(xp[md["row_of_entry"]], x[a // k])
    y = oracle.padded_scatter(xp, md, np.ones((T, k), np.float32), T, k)
    np.testing.assert_array_equal(y, k * x.astype(np.float64))


def test_scatter_reads_only_real_rows():
    """Garbage in pad rows must not reach the output ([MB] §5)."""
    rng = np.random.default_rng(11)
    T, k, E, H = 40, 2, 3, 4
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    md = oracle.metadata(ids, E)
    yp = rng.standard_normal((md["P"], H))
    w = rng.random((T, k))
    y1 = oracle.padded_scatter(yp, md, w, T, k)
    real = np.zeros(md["P"], dtype=bool)
    real[md["row_of_entry"]] = True
    yp2 = yp.copy()
    yp2[~real] = 1e30
    np.testing.assert_array_equal(oracle.padded_scatter(yp2, md, w, T, k), y1)


@pytest.mark.parametrize("T,k,E,seed", [
    (1, 1, 1, 0), (3, 2, 5, 1), (77, 3, 6, 2), (200, 8, 16, 3), (129, 1, 2, 4)])
def test_row_token_agrees_with_the_gather_and_padding(T, k, E, seed):
    """row_token read against the separately pinned gather and §2's padding:
    a real row holds the token the gather copies there, every token appears
    k times, and the -1 rows are exactly each expert's tail past its count."""
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    md = oracle.metadata(ids, E)
    rt = oracle.row_token(md, k)
    assert rt.shape == (md["P"],)
    # rows of x that are all distinct and non-zero: x[t] = t + 1
    x = np.repeat(np.arange(1, T + 1, dtype=np.float32)[:, None], 3, axis=1)
    xp = oracle.padded_gather(x, md, k)
    real = rt >= 0
    np.testing.assert_array_equal(xp[real, 0], rt[real] + 1)
    assert np.all(xp[~real] == 0.0)
    assert np.array_equal(np.bincount(rt[real], minlength=T), np.full(T, k))
    c = md["tokens_per_expert"]
    pc = np.diff(np.concatenate([[0], md["padded_bins"]]))
    pad = np.zeros(md["P"], dtype=bool)
    for e in range(E):
        pad[md["padded_bins"][e] - pc[e] + c[e]:md["padded_bins"][e]] = True
    np.testing.assert_array_equal(~real, pad)
    assert (~real).sum() == md["P"] - T * k
