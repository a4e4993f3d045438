"""Pins of the dMoA map/reduce oracle (CPU only): a hand-worked fixture, a
per-slot scalar brute force, map-then-reduce with inverse experts giving x
back, expert relabelling, and central finite differences."""
import json
import os

import numpy as np
import pytest

from oracle import moa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "moa_hand.json")


def _case(seed, T=7, k=3, E=5, H=4, F=6, empty=True):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    if empty:
        ids[rng.random(ids.shape) < 0.2] = -1
    w = rng.random((T, k))
    w[ids < 0] = 0.0
    return (rng.standard_normal((T, H)), ids, w, rng.standard_normal((E, H, F)),
            rng.standard_normal((E, F, H)), rng.standard_normal((T, k, F)))


def test_hand_worked_fixture():
    g = json.load(open(GOLDEN))
    q = moa.map_forward(g["x"], g["top_experts"], g["w1"])
    np.testing.assert_array_equal(q, g["q"])
    out = moa.reduce_forward(q, g["top_experts"], g["weights"], g["w2"])
    np.testing.assert_array_equal(out, g["out_of_q"])
    dy, dw2, dwt = moa.reduce_backward(q, g["top_experts"], g["weights"], g["w2"], g["dout"])
    np.testing.assert_array_equal(dy, g["dy"])
    np.testing.assert_array_equal(dw2, g["dw2"])
    np.testing.assert_array_equal(dwt, g["d_weights"])
    dx, dw1 = moa.map_backward(g["x"], g["top_experts"], g["w1"], dy)
    np.testing.assert_array_equal(dx, g["dx_of_dy"])
    np.testing.assert_array_equal(dw1, g["dw1_of_dy"])


def test_scalar_brute_force():
    """Every output element as an explicit sum over the hidden index."""
    x, ids, w, w1, w2, y = _case(1, T=3, k=2, E=3, H=3, F=2)
    q = moa.map_forward(x, ids, w1)
    out = moa.reduce_forward(y, ids, w, w2)
    T, k = ids.shape
    H, F = w1.shape[1], w1.shape[2]
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            for f in range(F):
                ref = 0.0 if e < 0 else sum(x[t, h] * w1[e, h, f] for h in range(H))
                assert abs(q[t, j, f] - ref) < 1e-12
        for h in range(H):
            ref = 0.0
            for j in range(k):
                e = ids[t, j]
                if e >= 0:
                    ref += w[t, j] * sum(y[t, j, f] * w2[e, f, h] for f in range(F))
            assert abs(out[t, h] - ref) < 1e-12


def test_inverse_experts_give_x_back():
    """With w2[e] = w1[e]^-1 and weights summing to one per token, reduce
    applied to map's output returns x (attention as the identity)."""
    rng = np.random.default_rng(3)
    T, k, E, H = 9, 3, 4, 5
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    w = rng.random((T, k))
    w /= w.sum(axis=1, keepdims=True)
    w1 = rng.standard_normal((E, H, H)) + 3 * np.eye(H)
    w2 = np.linalg.inv(w1)
    x = rng.standard_normal((T, H))
    out = moa.reduce_forward(moa.map_forward(x, ids, w1), ids, w, w2)
    np.testing.assert_allclose(out, x, rtol=1e-10, atol=1e-10)


def test_relabelling_experts():
    x, ids, w, w1, w2, y = _case(4)
    E = w1.shape[0]
    perm = np.random.default_rng(5).permutation(E)      # expert e becomes perm[e]
    ids2 = np.where(ids >= 0, perm[np.maximum(ids, 0)], -1)
    w1b = np.empty_like(w1)
    w2b = np.empty_like(w2)
    w1b[perm], w2b[perm] = w1, w2
    np.testing.assert_allclose(moa.map_forward(x, ids2, w1b), moa.map_forward(x, ids, w1))
    np.testing.assert_allclose(moa.reduce_forward(y, ids2, w, w2b),
                               moa.reduce_forward(y, ids, w, w2))


def _fd(f, a, eps=1e-6):
    g = np.zeros_like(a)
    it = np.nditer(a, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = a[i]
        a[i] = old + eps
        hi = f()
        a[i] = old - eps
        lo = f()
        a[i] = old
        g[i] = (hi - lo) / (2 * eps)
    return g


@pytest.mark.parametrize("seed", [7, 8])
def test_gradients_by_finite_differences(seed):
    x, ids, w, w1, w2, y = _case(seed, T=4, k=2, E=3, H=3, F=4)
    rng = np.random.default_rng(seed + 100)
    dq = rng.standard_normal((4, 2, 4))
    dout = rng.standard_normal((4, 3))
    live = (ids >= 0)[:, :, None]
    Lmap = lambda: float(np.sum(dq * moa.map_forward(x, ids, w1)))
    Lred = lambda: float(np.sum(dout * moa.reduce_forward(y, ids, w, w2)))
    dx, dw1 = moa.map_backward(x, ids, w1, dq)
    np.testing.assert_allclose(dx, _fd(Lmap, x), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dw1, _fd(Lmap, w1), rtol=1e-6, atol=1e-8)
    dy, dw2, dwt = moa.reduce_backward(y, ids, w, w2, dout)
    np.testing.assert_allclose(dy, _fd(Lred, y) * live, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dw2, _fd(Lred, w2), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dwt, _fd(Lred, w) * live[:, :, 0], rtol=1e-6, atol=1e-8)
    assert np.all(dy[ids < 0] == 0) and np.all(dwt[ids < 0] == 0)
