"""CPU oracle for the router in front of the dMoE layer -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module; the HIP router shares no code with it.

Plain numpy in float64 on the exact fp32 logits.

Sources:

* [FL] Fast-LLM issue "[feat] Support sparse copy for a large number of
  experts": the model config routes each token to ``num_experts_per_token``
  of ``num_experts`` experts and sets ``expert_z_loss_coefficient: 0.001``.
* [MR] the "yikangshen/megablocks" README: the router z-loss "introduced in
  ST-MoE" is supported.
* The layer's input recipe: the top-k logits of each token, and weights that
  are the softmax over those k logits.

Readings (the pages print no router code or formula):

* R19: top-k by descending logit; equal logits go to the lower expert id, so
  the selection is unique.  The routing weights are the softmax over the k
  chosen logits.  Logits must not be NaN.
* R20: the z-loss is ST-MoE's router z-loss, ``coef * mean_t (log sum_e
  exp(l[t, e]))**2``, over all E logits of each token.
* R21: the selection is piecewise constant, so no gradient flows through it:
  ``d l[t, e_j] = w_j (g_j - sum_i w_i g_i)`` for the chosen ``e_j`` (the
  softmax Jacobian), 0 for the others; the z-loss adds
  ``coef * 2 / T * lse_t * softmax(l[t])_e`` to every logit.

Pins (tests/test_oracle_router.py): a hand-sorted fixture with ties, k = 1,
k = E against the full softmax, closed forms, shift invariance, the zero sum
of the selection gradient, central finite differences of both losses.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

__all__ = ["topk", "router_forward", "router_backward", "zloss", "zloss_grad"]


def topk(logits, k: int) -> np.ndarray:
    """Ids of the k largest logits per row, descending; ties to the lower id.

    A stable sort of the negated values keeps equal values in ascending id
    order (R19)."""
    l = np.asarray(logits)
    if np.isnan(l).any():
        raise ValueError("NaN logits")
    order = np.argsort(-l.astype(np.float64), axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def _softmax(z: np.ndarray) -> np.ndarray:
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


def router_forward(logits, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """(ids [T,k], weights [T,k]): top-k and the softmax over the chosen logits."""
    l = np.asarray(logits, dtype=np.float64)
    ids = topk(logits, k)
    chosen = np.take_along_axis(l, ids, axis=1)
    return ids, _softmax(chosen)


def _lse(l: np.ndarray) -> np.ndarray:
    """log sum_e exp(l[t, e]) per row."""
    m = l.max(axis=1)
    return m + np.log(np.exp(l - m[:, None]).sum(axis=1))


def zloss(logits, coef: float) -> Tuple[float, np.ndarray]:
    """(coef * mean_t lse_t**2, per-token lse_t**2) with lse_t = log sum_e exp."""
    z = _lse(np.asarray(logits, dtype=np.float64)) ** 2
    return float(coef * z.mean()), z


def zloss_grad(logits, coef: float) -> np.ndarray:
    """d(coef * mean_t lse_t**2) / d logits = coef * 2 / T * lse_t * softmax(l_t)."""
    l = np.asarray(logits, dtype=np.float64)
    return coef * 2.0 / l.shape[0] * _lse(l)[:, None] * _softmax(l)


def router_backward(logits, ids, weights, d_weights, coef: float = 0.0) -> np.ndarray:
    """d logits [T,E] for upstream d_weights [T,k] (R21), plus the z-loss's."""
    l = np.asarray(logits, dtype=np.float64)
    w = np.asarray(weights, dtype=np.float64)
    g = np.asarray(d_weights, dtype=np.float64)
    T, E = l.shape
    out = np.zeros((T, E))
    dot = (w * g).sum(axis=1, keepdims=True)
    np.put_along_axis(out, np.asarray(ids, dtype=np.int64), w * (g - dot), axis=1)
    if coef != 0.0:
        out += zloss_grad(l, coef)
    return out
