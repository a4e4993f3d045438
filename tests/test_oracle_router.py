"""Pins of the router oracle (oracle/router.py) against facts that do not
depend on it: a hand-sorted fixture with ties, closed forms, the full softmax
at k = E, invariances, and central finite differences of both losses."""
import math

import numpy as np
import pytest

from oracle import router

RNG = np.random.default_rng(7)


def test_hand_fixture_with_ties():
    l = np.array([[0.5, 2.0, 2.0, -1.0, 2.0],
                  [-3.0, -3.0, -3.0, -3.0, -3.0]], dtype=np.float32)
    # equal logits go to the lower id first
    assert router.topk(l, 3).tolist() == [[1, 2, 4], [0, 1, 2]]
    assert router.topk(l, 4).tolist() == [[1, 2, 4, 0], [0, 1, 2, 3]]
    ids, w = router.router_forward(l, 3)
    np.testing.assert_allclose(w, np.full((2, 3), 1.0 / 3.0), rtol=0, atol=1e-15)


def test_nan_logits_rejected():
    with pytest.raises(ValueError):
        router.topk(np.array([[0.0, np.nan]]), 1)


def test_k1_weight_one_and_no_gradient():
    l = RNG.standard_normal((6, 5)).astype(np.float32)
    ids, w = router.router_forward(l, 1)
    assert ids[:, 0].tolist() == [int(np.argmax(r)) for r in l]
    np.testing.assert_array_equal(w, np.ones((6, 1)))
    g = RNG.standard_normal((6, 1))
    np.testing.assert_array_equal(router.router_backward(l, ids, w, g), np.zeros((6, 5)))


def test_k2_closed_form():
    l = RNG.standard_normal((5, 4)).astype(np.float32)
    ids, w = router.router_forward(l, 2)
    for t in range(5):
        a, b = float(l[t, ids[t, 0]]), float(l[t, ids[t, 1]])
        w0 = 1.0 / (1.0 + math.exp(b - a))
        assert abs(w[t, 0] - w0) < 1e-15 and abs(w[t, 1] - (1.0 - w0)) < 1e-15


def test_k_equals_e_is_the_full_softmax():
    l = RNG.standard_normal((3, 6)).astype(np.float32)
    ids, w = router.router_forward(l, 6)
    for t in range(3):
        row = [float(v) for v in l[t]]
        den = sum(math.exp(v) for v in row)
        assert ids[t].tolist() == sorted(range(6), key=lambda e: (-row[e], e))
        for j, e in enumerate(ids[t]):
            assert abs(w[t, j] - math.exp(row[e]) / den) < 1e-14


def test_shift_invariance():
    # logits above 0 keep log-sum-exp positive, so sqrt(z) is log-sum-exp itself
    l = RNG.standard_normal((4, 8)) + 2.0
    ids, w = router.router_forward(l, 3)
    ids2, w2 = router.router_forward(l + 5.0, 3)
    np.testing.assert_array_equal(ids, ids2)
    np.testing.assert_allclose(w, w2, rtol=1e-12)
    # the selection and its weights ignore a common shift; log-sum-exp moves with it
    _, z = router.zloss(l, 1.0)
    _, z2 = router.zloss(l + 5.0, 1.0)
    np.testing.assert_allclose(np.sqrt(z2), np.sqrt(z) + 5.0, rtol=1e-12)


def test_zloss_uniform_closed_form():
    c, E, T = 0.3, 7, 4
    l = np.full((T, E), c)
    loss, z = router.zloss(l, 0.001)
    assert abs(loss - 0.001 * (c + math.log(E)) ** 2) < 1e-15
    # the gradient of a uniform row is the same for every expert
    g = router.zloss_grad(l, 0.001)
    np.testing.assert_allclose(g, np.full((T, E), 0.001 * 2 / T * (c + math.log(E)) / E), rtol=1e-12)


def test_selection_gradient_sums_to_zero():
    l = RNG.standard_normal((5, 9))
    ids, w = router.router_forward(l, 4)
    d = router.router_backward(l, ids, w, RNG.standard_normal((5, 4)))
    np.testing.assert_allclose(d.sum(axis=1), 0.0, atol=1e-14)


def _fd(f, x, h=1e-6):
    g = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        g[idx] = (f(xp) - f(xm)) / (2 * h)
    return g


def test_backward_matches_finite_differences():
    # distinct, well-separated logits so a small step never changes the choice
    T, E, k = 3, 6, 3
    l = np.stack([RNG.permutation(E) * 0.37 + RNG.standard_normal(E) * 0.01 for _ in range(T)])
    g = RNG.standard_normal((T, k))
    ids, w = router.router_forward(l, k)
    coef = 0.05

    def loss(x):
        ii, ww = router.router_forward(x, k)
        assert (ii == ids).all()
        return float((ww * g).sum()) + router.zloss(x, coef)[0]

    np.testing.assert_allclose(router.router_backward(l, ids, w, g, coef), _fd(loss, l),
                               rtol=1e-6, atol=1e-9)
