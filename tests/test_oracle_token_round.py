"""Pins of the token-rounding oracle (CPU only): hand-worked cases and the
properties the rounding rule fixes on random logits."""
import json
import os

import numpy as np
import pytest

from oracle.token_round import token_round

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "token_round_hand.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_worked_cases(case):
    ids, w, info = token_round(np.asarray(case["logits"], np.float32), case["k"], case["M"])
    np.testing.assert_array_equal(ids, case["ids"])
    np.testing.assert_allclose(w, case["weights"], rtol=1e-12, atol=1e-15)
    assert info["decision"] == case["decision"]


def _check(l, k, M, ids, w, info):
    T, E = l.shape
    order = np.argsort(-l, axis=1, kind="stable")
    top, cand = order[:, :k], order[:, k]
    c = np.bincount(top.reshape(-1), minlength=E)
    np.testing.assert_array_equal(info["c"], c)
    n = np.bincount(ids[ids >= 0], minlength=E)
    np.testing.assert_array_equal(info["n"], n)
    # every expert receives a multiple of M tokens, within M - 1 of top-k
    assert np.all(n % M == 0)
    assert np.all(np.abs(n - c) <= M - 1)
    # slots: j < k hold the top-k id or -1; slot k the candidate or -1
    assert np.all((ids[:, :k] == top) | (ids[:, :k] == -1))
    assert np.all((ids[:, k] == cand) | (ids[:, k] == -1))
    for e in range(E):
        r = c[e] % M
        kept = [float(l[t, e]) for t in range(T) for j in range(k) if ids[t, j] == e]
        dropped = [(float(l[t, e]), -t) for t in range(T) for j in range(k)
                   if top[t, j] == e and ids[t, j] == -1]
        added = [(-float(l[t, e]), t) for t in range(T) if ids[t, k] == e]
        left = [(-float(l[t, e]), t) for t in range(T) if cand[t] == e and ids[t, k] != e]
        d = info["decision"][e]
        if r == 0:
            assert d == "keep" and not dropped and not added
        elif d == "up":
            assert M - r < r and len(added) == M - r and not dropped
            # the added candidates are the best ones
            assert not left or max(added) < min(left)
        else:
            assert d == "down" and len(dropped) == r and not added
            assert (M - r >= r) or sum(cand == e) < M - r
            # the dropped entries are the worst ones
            routed = [(float(l[t, e]), -t) for t in range(T) for j in range(k)
                      if top[t, j] == e and ids[t, j] == e]
            assert not routed or max(dropped) < min(routed)
        assert len(kept) == c[e] - len(dropped)
    # weights: softmax over the occupied slots
    occ = ids >= 0
    assert np.all(w[~occ] == 0.0)
    has = occ.any(axis=1)
    np.testing.assert_allclose(w[has].sum(axis=1), 1.0, rtol=1e-12)
    for t in np.nonzero(has)[0][:50]:
        z = np.array([l[t, e] for e in ids[t][occ[t]]], dtype=np.float64)
        p = np.exp(z - z.max())
        np.testing.assert_allclose(w[t][occ[t]], p / p.sum(), rtol=1e-12)


@pytest.mark.parametrize("T,E,k,M,ties,seed", [
    (64, 4, 1, 4, False, 0), (300, 8, 2, 16, False, 1), (300, 8, 2, 16, True, 2),
    (1000, 16, 4, 32, False, 3), (2048, 64, 8, 128, False, 4), (777, 5, 4, 8, True, 5),
    (4096, 256, 8, 128, False, 6)])
def test_rounding_properties(T, E, k, M, ties, seed):
    rng = np.random.default_rng(seed)
    l = rng.standard_normal((T, E)).astype(np.float32)
    if ties:
        l = np.round(l * 2) / 2
        l[rng.random((T, E)) < 0.1] = -0.0
    ids, w, info = token_round(l, k, M)
    _check(l, k, M, ids, w, info)


def test_rejects_k_not_below_E():
    with pytest.raises(ValueError):
        token_round(np.zeros((4, 2), np.float32), 2, 4)
