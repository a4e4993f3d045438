"""CPU oracle for tile-aware token rounding -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module; the HIP path never calls it and shares no code with it.

Source: "SonicMoE: Accelerating MoE with IO and Tile-aware Optimizations"
(abstract): under high MoE sparsity, padding each expert's rows up to the
grouped GEMM's tile wastes compute; a tile-aware "token rounding" of the
routing instead rounds the number of tokens each expert receives so that
little padding is left, keeping the quality of top-K routing.  The page
gives no rule, so this module fixes one (reading R25):

* Route each token to its k largest logits (descending, equal logits to the
  lower expert id, as the router does); its (k+1)-th largest is its
  candidate expert.  c_e is the number of tokens routed to e.
* For every expert with r = c_e mod M != 0 (M = 128, the row block of the
  padded layout): when M - r < r (the next multiple of M is nearer) and at
  least M - r tokens have e as their candidate, e takes the M - r of them
  with the largest logit for e (equal logits: lower token id first); those
  tokens gain e in their extra slot.  Otherwise e drops the r of its routed
  tokens with the smallest logit for e (equal logits: higher token id
  first); those slots become empty.  Every expert then receives a multiple
  of M tokens, and the padded layout of the layer has no pad rows.
* The result is laid out as k+1 slots per token: slot j < k holds the j-th
  routed expert or -1 if it was dropped, slot k the candidate if it was
  added or -1.  Routing weights are the softmax over the logits of a
  token's occupied slots, 0 in empty slots; a token left with no expert
  gets all zeros (its output is zero).

Everything is plain numpy and Python loops (fp64 for the weights).
"""
from __future__ import annotations

import numpy as np

__all__ = ["BLOCK", "token_round"]

BLOCK = 128


def token_round(logits, k: int, M: int = BLOCK):
    """(ids [T,k+1] int64 with -1 for empty slots, weights [T,k+1] fp64,
    info) for fp32 logits [T,E]; requires 1 <= k < E.  info holds the
    routed counts c, the final counts n, and per expert "up", "down" or
    "keep"."""
    l = np.asarray(logits, dtype=np.float32)
    T, E = l.shape
    if not 1 <= k < E:
        raise ValueError("token rounding needs 1 <= k < E")
    # descending logit, equal logits to the lower id (a stable sort of the
    # negation keeps ascending ids among equal values; -0 equals +0)
    order = np.argsort(-l, axis=1, kind="stable")
    top, cand = order[:, :k], order[:, k]
    c = np.bincount(top.reshape(-1), minlength=E)
    ids = np.full((T, k + 1), -1, dtype=np.int64)
    ids[:, :k] = top
    decision = []
    for e in range(E):
        r = int(c[e]) % M
        if r == 0:
            decision.append("keep")
            continue
        up = M - r
        cands = [int(t) for t in np.nonzero(cand == e)[0]]       # tokens whose next choice is e
        if up < r and len(cands) >= up:
            cands.sort(key=lambda t: (-float(l[t, e]), t))
            for t in cands[:up]:
                ids[t, k] = e
            decision.append("up")
        else:
            routed = [(int(t), int(j)) for t, j in zip(*np.nonzero(top == e))]
            routed.sort(key=lambda tj: (float(l[tj[0], e]), -tj[0]))
            for t, j in routed[:r]:
                ids[t, j] = -1
            decision.append("down")
    weights = np.zeros((T, k + 1))
    for t in range(T):
        occ = [j for j in range(k + 1) if ids[t, j] >= 0]
        if not occ:
            continue
        z = np.array([float(l[t, ids[t, j]]) for j in occ])
        p = np.exp(z - z.max())
        p /= p.sum()
        for j, v in zip(occ, p):
            weights[t, j] = v
    n = np.bincount(ids[ids >= 0].reshape(-1), minlength=E)
    return ids, weights, dict(c=c, n=n, decision=decision)
