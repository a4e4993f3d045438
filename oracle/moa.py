"""CPU oracle of the dMoA map / reduce pair -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module; the HIP path never calls it and the two share no code.
Plain numpy in float64: bf16 and fp32 inputs convert exactly, and nothing
here rounds.

Source: the "yikangshen/megablocks" README, which adds mixture of attention
heads (dMoA) to the library and shows a causal self-attention whose query
projection is a dMoA layer.  Its expert is the library's plain MLP with no
activation and no bias, with ffn_hidden_size equal to hidden_size.  The
forward calls ``map`` on x, reads the result as k * n_head query heads per
token, runs attention (an external kernel) against shared keys and values,
and calls ``reduce`` on the attention output reshaped to (tokens, k,
hidden).

Reading R27 (the README prints no formula for map and reduce):
* an expert e is the two matrices of that MLP, w1[e] of shape [H, F] and
  w2[e] of shape [F, H] (an MLP without activation computes x w1 w2);
* ``map`` applies the first half to each routed slot, without the routing
  weight: q[t, j] = x[t] w1[e(t, j)];
* ``reduce`` applies the second half to each slot and sums the slots with
  the routing weights, as the dMoE layer's scatter does:
  out[t] = sum_j w[t, j] * (y[t, j] w2[e(t, j)]);
* the routing (top_experts, weights) is the router's and is shared by map
  and reduce; an empty slot (id -1, as in the dMoE layer) maps to a zero row
  and adds nothing to the reduction, and its gradients are zero.

Pins (tests/test_oracle_moa.py): a hand-worked fixture
(tests/golden/moa_hand.json), a per-slot scalar brute force on tiny inputs,
map followed by reduce with w2[e] the inverse of w1[e] and weights summing
to one giving x back, invariance under relabelling the experts, and central
finite differences for every gradient.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

__all__ = ["map_forward", "reduce_forward", "map_backward", "reduce_backward"]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _slots(top_experts, e):
    """(tokens, slots) of the entries routed to expert e, in entry order."""
    ids = np.asarray(top_experts)
    t, j = np.nonzero(ids == e)
    return t, j


def map_forward(x, top_experts, w1) -> np.ndarray:
    """q[t, j] = x[t] @ w1[e(t, j)]; zero rows for empty slots.  [T, k, F]."""
    x, w1 = _f64(x), _f64(w1)
    T, k = np.asarray(top_experts).shape
    q = np.zeros((T, k, w1.shape[2]))
    for e in range(w1.shape[0]):
        t, j = _slots(top_experts, e)
        if len(t):
            q[t, j] = x[t] @ w1[e]
    return q


def reduce_forward(y, top_experts, weights, w2) -> np.ndarray:
    """out[t] = sum_j weights[t, j] * (y[t, j] @ w2[e(t, j)]).  [T, H]."""
    y, weights, w2 = _f64(y), _f64(weights), _f64(w2)
    T, k = np.asarray(top_experts).shape
    out = np.zeros((T, w2.shape[2]))
    for e in range(w2.shape[0]):
        t, j = _slots(top_experts, e)
        if len(t):
            # np.add.at: a token may reach one expert in two slots only if
            # the routing repeats an id, which a top-k never does; it keeps
            # the sum right regardless
            np.add.at(out, t, weights[t, j][:, None] * (y[t, j] @ w2[e]))
    return out


def map_backward(x, top_experts, w1, dq) -> Tuple[np.ndarray, np.ndarray]:
    """Gradients of map for the upstream gradient dq [T, k, F]:
    dx[t] = sum_j dq[t, j] @ w1[e]^T and dw1[e] = sum over e's slots of
    x[t]^T dq[t, j]."""
    x, w1, dq = _f64(x), _f64(w1), _f64(dq)
    dx = np.zeros_like(x)
    dw1 = np.zeros_like(w1)
    for e in range(w1.shape[0]):
        t, j = _slots(top_experts, e)
        if len(t):
            np.add.at(dx, t, dq[t, j] @ w1[e].T)
            dw1[e] = x[t].T @ dq[t, j]
    return dx, dw1


def reduce_backward(y, top_experts, weights, w2, dout
                    ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of reduce for the upstream gradient dout [T, H]:
    dy[t, j] = weights[t, j] * dout[t] @ w2[e]^T,
    dw2[e] = sum over e's slots of weights[t, j] * y[t, j]^T dout[t],
    d_weights[t, j] = <dout[t], y[t, j] @ w2[e]> (0 for an empty slot)."""
    y, weights, w2, dout = _f64(y), _f64(weights), _f64(w2), _f64(dout)
    dy = np.zeros_like(y)
    dw2 = np.zeros_like(w2)
    dwt = np.zeros_like(weights)
    for e in range(w2.shape[0]):
        t, j = _slots(top_experts, e)
        if len(t):
            g = weights[t, j][:, None] * dout[t]          # the slot's share of dout
            dy[t, j] = g @ w2[e].T
            dw2[e] = y[t, j].T @ g
            dwt[t, j] = np.sum(dout[t] * (y[t, j] @ w2[e]), axis=1)
    return dy, dw2, dwt
