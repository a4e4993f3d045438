"""Pins of the oracle's forward and backward (CPU only).

Each test checks the oracle against something other than itself: a closed
form evaluated with ``math.exp``, a dense gated-SiLU MLP built from torch's
``silu``, symmetries of the layer, agreement of the per-entry definition with
the pages' padded pipeline, and central finite differences for every
gradient.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand_layer(rng, T, H, F, E, k, distinct=True):
    if distinct and k <= E:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    else:
        ids = rng.integers(0, E, (T, k))
    return dict(
        x=rng.standard_normal((T, H)),
        top_experts=ids.astype(np.int32),
        weights=rng.random((T, k)) + 0.1,
        w1=rng.standard_normal((E, H, F)) * 0.5,
        w3=rng.standard_normal((E, H, F)) * 0.5,
        w2=rng.standard_normal((E, F, H)) * 0.5,
    )


def test_closed_form_one_number():
    """T=H=F=E=k=1: y = w * silu(x a1) * (x a3) * a2."""
    x, a1, a3, a2, wt = 2.0, 1.0, 3.0, 0.5, 0.75
    u1 = x * a1
    expect = wt * (u1 / (1.0 + math.exp(-u1))) * (x * a3) * a2
    y, _ = oracle.forward_loop(np.array([[x]]), np.array([[0]]),
                               np.array([[wt]]), np.array([[[a1]]]),
                               np.array([[[a3]]]), np.array([[[a2]]]))
    assert abs(y[0, 0] - expect) <= 1e-15 * abs(expect)


def test_closed_form_identity_weights():
    """w1 = w3 = w2 = I: each expert maps x to silu(x) * x elementwise."""
    rng = np.random.default_rng(0)
    T, H, E, k = 6, 3, 2, 2
    x = rng.standard_normal((T, H))
    eye = np.stack([np.eye(H)] * E)
    ids = np.array([[0, 1]] * T, dtype=np.int32)
    w = rng.random((T, k))
    y, _ = oracle.forward_loop(x, ids, w, eye, eye, eye)
    for t in range(T):
        for h in range(H):
            v = x[t, h]
            expect = (w[t, 0] + w[t, 1]) * v / (1.0 + math.exp(-v)) * v
            assert abs(y[t, h] - expect) <= 1e-14 * max(1.0, abs(expect))


def _dense_mlp_torch(x, w1, w3, w2):
    x, w1, w3, w2 = (torch.from_numpy(np.asarray(a, np.float64))
                     for a in (x, w1, w3, w2))
    return (torch.nn.functional.silu(x @ w1) * (x @ w3) @ w2).numpy()


def test_single_expert_top1_is_dense_gated_silu_mlp():
    rng = np.random.default_rng(1)
    L = _rand_layer(rng, 9, 6, 4, 1, 1)
    L["weights"] = np.ones((9, 1))
    ref = _dense_mlp_torch(L["x"], L["w1"][0], L["w3"][0], L["w2"][0])
    y, _ = oracle.forward_loop(**L)
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)
    yp, _ = oracle.forward_padded(**L)
    np.testing.assert_allclose(yp, ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("impl", ["loop", "padded"])
def test_identical_experts_any_routing(impl):
    """All experts equal and each token's weights summing to 1: the layer
    is the dense MLP whatever the routing (checks the permutation apart from
    the sort)."""
    rng = np.random.default_rng(2)
    T, H, F, E, k = 150, 5, 7, 4, 3
    L = _rand_layer(rng, T, H, F, E, k)
    for name in ("w1", "w3", "w2"):
        L[name] = np.stack([L[name][0]] * E)
    L["weights"] = L["weights"] / L["weights"].sum(axis=1, keepdims=True)
    ref = _dense_mlp_torch(L["x"], L["w1"][0], L["w3"][0], L["w2"][0])
    fn = oracle.forward_loop if impl == "loop" else oracle.forward_padded
    y, _ = fn(**L)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_linear_in_routing_weights():
    rng = np.random.default_rng(3)
    L = _rand_layer(rng, 20, 4, 3, 3, 2)
    wa, wb = rng.random((20, 2)), rng.random((20, 2))
    ya, _ = oracle.forward_padded(**{**L, "weights": wa})
    yb, _ = oracle.forward_padded(**{**L, "weights": wb})
    yab, _ = oracle.forward_padded(**{**L, "weights": wa + 2 * wb})
    np.testing.assert_allclose(yab, ya + 2 * yb, rtol=1e-12, atol=1e-12)


def test_token_and_expert_relabelling_equivariance():
    rng = np.random.default_rng(4)
    T, H, F, E, k = 30, 4, 5, 5, 2
    L = _rand_layer(rng, T, H, F, E, k)
    y, _ = oracle.forward_padded(**L)
    perm_t = rng.permutation(T)
    perm_e = rng.permutation(E)          # new id of old expert e is perm_e[e]
    inv_e = np.argsort(perm_e)
    L2 = dict(x=L["x"][perm_t], top_experts=perm_e[L["top_experts"][perm_t]],
              weights=L["weights"][perm_t], w1=L["w1"][inv_e],
              w3=L["w3"][inv_e], w2=L["w2"][inv_e])
    y2, _ = oracle.forward_padded(**L2)
    np.testing.assert_allclose(y2, y[perm_t], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("T,H,F,E,k,distinct", [
    (5, 3, 4, 2, 1, True), (40, 6, 5, 3, 2, True), (300, 4, 3, 3, 2, True),
    (64, 5, 6, 8, 3, False), (17, 2, 2, 1, 1, True)])
def test_loop_equals_padded_pipeline(T, H, F, E, k, distinct):
    rng = np.random.default_rng(T + H)
    L = _rand_layer(rng, T, H, F, E, k, distinct)
    y_loop, ent = oracle.forward_loop(**L)
    y_pad, sv = oracle.forward_padded(**L)
    np.testing.assert_allclose(y_pad, y_loop, rtol=1e-12, atol=1e-12)
    rows = sv["md"]["row_of_entry"]
    np.testing.assert_allclose(sv["h1"][rows], ent["u1"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sv["act"][rows], ent["act"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sv["y_perm"][rows], ent["o"], rtol=1e-12, atol=1e-12)
    pad = np.ones(sv["md"]["P"], bool)
    pad[rows] = False
    for key in ("x_perm", "h1", "h3", "act", "y_perm"):
        assert np.all(sv[key][pad] == 0.0), key
    dy = rng.standard_normal((T, H))
    g_loop = oracle.backward_loop(**L, dy=dy)
    g_pad = oracle.backward_padded(**L, dy=dy, saved=sv)
    for key in ("dx", "dw1", "dw3", "dw2", "d_weights"):
        np.testing.assert_allclose(g_pad[key], g_loop[key], rtol=1e-11,
                                   atol=1e-11, err_msg=key)
    for key in ("dy_perm", "dh1", "dh3", "dx_perm"):
        assert np.all(g_pad[key][pad] == 0.0), key


def _loss(L, dy):
    y, _ = oracle.forward_loop(**L)
    return float(np.sum(y * dy))


@pytest.mark.parametrize("seed", [0, 1])
def test_gradients_by_central_differences(seed):
    rng = np.random.default_rng(100 + seed)
    T, H, F, E, k = 5, 4, 3, 3, 2
    L = _rand_layer(rng, T, H, F, E, k)
    dy = rng.standard_normal((T, H))
    g = oracle.backward_loop(**L, dy=dy)
    g_pad = oracle.backward_padded(**L, dy=dy)
    eps = 1e-6
    names = {"x": "dx", "w1": "dw1", "w3": "dw3", "w2": "dw2",
             "weights": "d_weights"}
    for pname, gname in names.items():
        p = L[pname]
        num = np.zeros_like(p)
        for idx in np.ndindex(p.shape):
            old = p[idx]
            p[idx] = old + eps
            lp = _loss(L, dy)
            p[idx] = old - eps
            lm = _loss(L, dy)
            p[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        scale = np.max(np.abs(num))
        assert scale > 0
        assert np.max(np.abs(g[gname] - num)) <= 1e-7 * scale, pname
        assert np.max(np.abs(g_pad[gname] - num)) <= 1e-7 * scale, pname


def test_empty_expert_has_zero_weight_gradient():
    rng = np.random.default_rng(5)
    L = _rand_layer(rng, 12, 3, 4, 4, 2)
    L["top_experts"] = np.where(L["top_experts"] == 2, 3, L["top_experts"])
    L["top_experts"][:, 1] = np.where(L["top_experts"][:, 0] == 3, 0, 3)
    assert not np.any(L["top_experts"] == 2)
    g = oracle.backward_padded(**L, dy=rng.standard_normal((12, 3)))
    for key in ("dw1", "dw3", "dw2"):
        assert np.all(g[key][2] == 0.0)
        assert np.any(g[key][3] != 0.0)


def test_sampled_outputs_match_full_backward():
    rng = np.random.default_rng(6)
    T, H, F, E, k = 50, 6, 5, 4, 2
    L = _rand_layer(rng, T, H, F, E, k)
    dy = rng.standard_normal((T, H))
    y, _ = oracle.forward_loop(**L)
    g = oracle.backward_loop(**L, dy=dy)
    rows = oracle.sampled_rows(**L, dy=dy, tokens=[0, 7, 49])
    for t, r in rows.items():
        np.testing.assert_allclose(r["y"], y[t], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(r["dx"], g["dx"][t], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(r["d_weights"], g["d_weights"][t],
                                   rtol=1e-12, atol=1e-12)
    picks = [("dw1", 0, 1, 2), ("dw3", 3, 5, 4), ("dw2", 2, 4, 5),
             ("dw2", 1, 0, 0), ("dw1", 2, 0, 3)]
    vals = oracle.sampled_dw(**L, dy=dy, picks=picks)
    for (name, e, i, j), v in zip(picks, vals):
        assert abs(v - g[name][e][i, j]) <= 1e-12 * max(1.0, abs(v))


@pytest.mark.parametrize("T,H,F,E,k,distinct", [
    (40, 8, 6, 5, 2, True),      # most experts under one 128-row block
    (300, 4, 3, 3, 2, True),     # experts of several blocks
    (30, 5, 4, 7, 1, True),      # some experts empty
    (200, 3, 5, 2, 3, False),    # duplicate ids in a token's row
])
def test_layer_by_expert_equals_padded_pipeline(T, H, F, E, k, distinct):
    """The expert-at-a-time form gives every padded intermediate, every
    weight gradient and y, dx, d_weights of the whole-layer padded form."""
    rng = np.random.default_rng(T + 7 * E)
    L = _rand_layer(rng, T, H, F, E, k, distinct)
    dy = rng.standard_normal((T, H))
    y, sv = oracle.forward_padded(**L)
    g = oracle.backward_padded(**L, dy=dy, saved=sv)
    out = dict(y=np.zeros((T, H)), dx=np.zeros((T, H)), d_weights=np.zeros((T, k)))
    seen = []
    for r in oracle.layer_by_expert(**L, dy=dy, out=out):
        e, (r0, r1) = r["e"], r["rows"]
        seen.append(e)
        for key in ("dw1", "dw3", "dw2"):
            np.testing.assert_allclose(r[key], g[key][e], rtol=1e-12, atol=1e-12)
        if r1 == r0:
            continue
        for key, ref in (("x_perm", sv["x_perm"]), ("h1", sv["h1"]), ("h3", sv["h3"]),
                         ("act", sv["act"]), ("y_perm", sv["y_perm"]),
                         ("dy_perm", g["dy_perm"]), ("dh1", g["dh1"]),
                         ("dh3", g["dh3"]), ("dx_perm", g["dx_perm"])):
            np.testing.assert_allclose(r[key], ref[r0:r1], rtol=1e-12, atol=1e-12,
                                       err_msg=key)
    assert seen == list(range(E))
    np.testing.assert_allclose(out["y"], y, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["dx"], g["dx"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["d_weights"], g["d_weights"], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("impl", ["loop", "padded", "by_expert"])
def test_empty_slot_is_a_zero_weight_entry(impl):
    """An empty slot (expert id -1) adds to y, dx, dw1, dw3 and dw2 exactly
    what an entry of routing weight 0 adds, i.e. nothing, and its
    routing-weight gradient is 0; the other slots' gradients are unchanged."""
    rng = np.random.default_rng(21)
    T, H, F, E, k = 40, 6, 5, 4, 3
    L = _rand_layer(rng, T, H, F, E, k)
    dy = rng.standard_normal((T, H))
    empty = rng.random((T, k)) < 0.35
    Lz = dict(L, weights=np.where(empty, 0.0, L["weights"]))
    Le = dict(L, top_experts=np.where(empty, -1, L["top_experts"]).astype(np.int32))

    def run(layer):
        if impl == "loop":
            y, _ = oracle.forward_loop(**layer)
            return y, oracle.backward_loop(**layer, dy=dy)
        if impl == "padded":
            y, sv = oracle.forward_padded(**layer)
            return y, oracle.backward_padded(**layer, dy=dy, saved=sv)
        out = dict(y=np.zeros((T, H)), dx=np.zeros((T, H)), d_weights=np.zeros((T, k)))
        g = {key: np.zeros(np.shape(layer[w])) for key, w in
             (("dw1", "w1"), ("dw3", "w3"), ("dw2", "w2"))}
        for r in oracle.layer_by_expert(**layer, dy=dy, out=out):
            for key in g:
                g[key][r["e"]] = r[key]
        g.update(dx=out["dx"], d_weights=out["d_weights"])
        return out["y"], g

    yz, gz = run(Lz)
    ye, ge = run(Le)
    np.testing.assert_allclose(ye, yz, rtol=1e-12, atol=1e-13)
    for key in ("dx", "dw1", "dw3", "dw2"):
        np.testing.assert_allclose(ge[key], gz[key], rtol=1e-12, atol=1e-13, err_msg=key)
    assert np.all(ge["d_weights"][empty] == 0.0)
    np.testing.assert_allclose(ge["d_weights"][~empty], gz["d_weights"][~empty],
                               rtol=1e-12, atol=1e-13)
