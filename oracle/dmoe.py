"""CPU oracle for the dropless-MoE (dMoE) expert layer -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path (the HIP library and its Python
binding) never calls it; the two share no code.

Everything here is plain numpy in float64.  Inputs are converted to float64
exactly (bf16 and fp32 values are exact in fp64), so the oracle sees the very
values the GPU sees and rounds nowhere.

Sources (the pages are the authority on what the layer computes):

* [MB] "02 · dropless MoE 与 block-sparse 重构", the MegaBlocks chapter on
  ai-reference-codex: §2 (round each expert's count up to 128, one expert
  per 128-row block, at most 127 pad rows per expert), §3 (the sdd/dsd
  pair), §4.1 (sort / histogram / cumsum, round_up, bins and padded_bins),
  §4.2 (padded_gather / padded_scatter index arithmetic, the A_TO_B switch,
  the routing-weight gradient, the gather <-> scatter backward pairing),
  §4.3 (row block -> expert column blocks), §4.5 (the forward sketch),
  §5 (GLU variant shares the topology, ffn % 128, pad rows are zero and
  dropped on scatter).
* [FL] Fast-LLM issue "[feat] Support sparse copy for a large number of
  experts": the layer is gated with activation SiLU, no biases.

Readings where the pages are silent or garbled (each is used below):

* R1/R2: ``bins[e-1]`` and ``padded_bins[e-1]`` at e = 0 mean 0 (the
  exclusive start), not Python's wrap-around to the last element.
* R3: the sketch's ``rows`` are flattened (token, slot) entries
  ``a = t*k + j``; the source token is ``a // k`` (the kernel of §4.2
  divides by TOP_K) and the weight is ``weights.flat[a]``.
* R4/R5: the activation is gated SiLU, ``silu(x@w1) * (x@w3)`` then ``@w2``
  (the sketch's ungated gelu is replaced by [FL]'s gated silu).
* R6: the sort is stable: ties keep ascending ``a``.
* R7: ``round_up(0) = 0``: an empty expert gets no rows and no tile.
* R9: the top-k reduction is a plain sum over j (the oracle does not round).
* R26: an expert id of -1 is an empty slot: the entry is routed nowhere,
  gets no padded row (row_of_entry = -1), adds nothing to y or dx and has a
  routing-weight gradient of 0.  The sorted arrays list the routed entries
  only and hold -1 past them.  Token rounding leaves such slots.
* w1, w3 are stored ``[E,H,F]`` and w2 ``[E,F,H]``.

Pins (tests/test_oracle_*.py): hand-derived metadata fixtures, a pure-Python
counting sort against the library sort, the padding invariants of §2, the
gather-then-unit-scatter identity, a dense gated-SiLU MLP (E=1, k=1) and
identical experts, closed forms, loop vs. padded-pipeline agreement, and
central finite differences for every gradient.
"""
from __future__ import annotations

from typing import Dict, Iterable, Optional, Sequence, Tuple

import numpy as np

BLOCK = 128

__all__ = [
    "BLOCK", "round_up", "max_tiles", "metadata", "metadata_counting_sort",
    "padded_gather", "row_token", "padded_scatter", "silu", "sigmoid", "forward_loop",
    "backward_loop", "forward_padded", "backward_padded", "layer_by_expert",
    "sampled_rows", "sampled_dw",
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# Metadata  ([MB] §4.1, §4.2, §4.3)
# --------------------------------------------------------------------------

def round_up(c, block: int = BLOCK):
    """Round a count up to a multiple of ``block`` ([MB] §4.1).  round_up(0)=0."""
    c = np.asarray(c, dtype=np.int64)
    return ((c + block - 1) // block) * block


def max_tiles(T: int, k: int, E: int) -> int:
    """Host bound on the number of 128-row tiles.

    Every non-empty expert wastes at most 127 rows ([MB] §2), so
    ``P <= T*k + 127*min(E, T*k)``; P is a multiple of 128.
    """
    n = T * k
    return (n + 127 * min(E, n)) // BLOCK


def metadata(top_experts, num_experts: int, n_tiles: Optional[int] = None
             ) -> Dict[str, np.ndarray]:
    """Routing metadata from top-k expert ids, with library primitives.

    [MB] §4.1: a stable sort of the flattened entries by expert, a histogram
    (tokens per expert), its inclusive cumsum ``bins``, the per-expert counts
    rounded up to 128, and their inclusive cumsum ``padded_bins``.
    [MB] §4.2: entry ``indices[s]`` lands on padded row
    ``(s - bins[e-1]) + padded_bins[e-1]`` with e its expert (R1: the start of
    expert 0 is 0).  [MB] §2/§4.3: each 128-row block belongs to one expert;
    ``tile_expert[r]`` names it, -1 past the last padded row.
    """
    ids = np.asarray(top_experts).reshape(-1).astype(np.int64)
    E = int(num_experts)
    if ids.size and (ids.min() < -1 or ids.max() >= E):
        raise ValueError("expert id out of range")
    n = ids.size
    routed = np.nonzero(ids >= 0)[0]        # R26: -1 is an empty slot
    nv = routed.size
    counts = np.bincount(ids[routed], minlength=E).astype(np.int64)
    order = routed[np.argsort(ids[routed], kind="stable")]      # R6
    indices = np.full(n, -1, dtype=np.int64)
    indices[:nv] = order
    bin_ids = np.full(n, -1, dtype=np.int64)
    bin_ids[:nv] = ids[order]
    bins = np.cumsum(counts)
    padded = round_up(counts)
    padded_bins = np.cumsum(padded)
    bins_start = bins - counts              # R1: exclusive starts
    padded_start = padded_bins - padded
    s = np.arange(nv, dtype=np.int64)
    row_of_entry = np.full(n, -1, dtype=np.int64)
    row_of_entry[order] = padded_start[ids[order]] + (s - bins_start[ids[order]])
    P = int(padded_bins[-1]) if E else 0
    if n_tiles is None:
        n_tiles = P // BLOCK
    tile_expert = np.full(n_tiles, -1, dtype=np.int64)
    live = np.arange(min(n_tiles, P // BLOCK))
    tile_expert[live] = np.searchsorted(padded_bins, live * BLOCK, side="right")
    return dict(tokens_per_expert=counts, bins=bins, padded_bins=padded_bins,
                indices=indices, bin_ids=bin_ids, row_of_entry=row_of_entry,
                tile_expert=tile_expert, P=P)


def metadata_counting_sort(top_experts, num_experts: int,
                           n_tiles: Optional[int] = None):
    """The same metadata with nothing but Python loops (small inputs only).

    A counting sort: count, take running starts, then place the entries in
    ascending flattened order, which is what makes it stable.
    """
    ids = [int(v) for v in np.asarray(top_experts).reshape(-1)]
    E = int(num_experts)
    counts = [0] * E
    for e in ids:
        if e >= 0:
            counts[e] += 1
    bins, padded_bins = [], []
    run = prun = 0
    for e in range(E):
        run += counts[e]
        prun += ((counts[e] + BLOCK - 1) // BLOCK) * BLOCK
        bins.append(run)
        padded_bins.append(prun)
    start = [bins[e] - counts[e] for e in range(E)]
    pstart = [padded_bins[e] - ((counts[e] + BLOCK - 1) // BLOCK) * BLOCK
              for e in range(E)]
    fill = [0] * E
    indices = [-1] * len(ids)
    bin_ids = [-1] * len(ids)
    row_of_entry = [-1] * len(ids)
    for a, e in enumerate(ids):
        if e == -1:                          # R26: an empty slot
            continue
        s = start[e] + fill[e]
        indices[s] = a
        bin_ids[s] = e
        row_of_entry[a] = pstart[e] + fill[e]
        fill[e] += 1
    P = padded_bins[-1] if E else 0
    if n_tiles is None:
        n_tiles = P // BLOCK
    tile_expert = []
    for r in range(n_tiles):
        owner = -1
        for e in range(E):
            if pstart[e] <= r * BLOCK < padded_bins[e]:
                owner = e
        tile_expert.append(owner)
    as_arr = lambda v: np.asarray(v, dtype=np.int64)
    return dict(tokens_per_expert=as_arr(counts), bins=as_arr(bins),
                padded_bins=as_arr(padded_bins), indices=as_arr(indices),
                bin_ids=as_arr(bin_ids), row_of_entry=as_arr(row_of_entry),
                tile_expert=as_arr(tile_expert), P=P)


# --------------------------------------------------------------------------
# Permutation  ([MB] §4.2, §4.5, §5)
# --------------------------------------------------------------------------

def padded_gather(x, md, k: int) -> np.ndarray:
    """Copy token rows into the expert-sorted, 128-padded layout.

    [MB] §4.2 gather direction: ``out[index_b] = x[index_a // TOP_K]``; every
    other row of the ``padded_bins[-1]``-row output is zero ([MB] §4.5, §5).
    """
    x = _f64(x)
    out = np.zeros((md["P"], x.shape[1]), dtype=np.float64)
    a = np.nonzero(md["row_of_entry"] >= 0)[0]          # routed entries (R26)
    out[md["row_of_entry"][a]] = x[a // k]
    return out


def row_token(md, k: int) -> np.ndarray:
    """The token each padded row holds, -1 for a pad row.

    [MB] §4.2: the gather copies token ``a // k`` (R3) onto padded row
    ``row_of_entry[a]``; [MB] §2: the rows of an expert's padded range past
    its count receive no entry.  This is the same index rule read from the
    row side: the table a kernel needs to fetch a padded row's token row
    straight from x.  Length P.
    """
    out = np.full(md["P"], -1, dtype=np.int64)
    a = np.nonzero(md["row_of_entry"] >= 0)[0]          # routed entries (R26)
    out[md["row_of_entry"][a]] = a // k
    return out


def padded_scatter(y_perm, md, weights, T: int, k: int) -> np.ndarray:
    """Weighted un-permute with top-k reduction ([MB] §4.2 scatter direction,
    §4.5 last loop).  Only real rows are read back ([MB] §5); R9: plain sum
    over the k slots of a token."""
    y_perm = _f64(y_perm)
    w = _f64(weights).reshape(-1)
    roe = md["row_of_entry"]
    rows = np.zeros((roe.size, y_perm.shape[1]))
    a = np.nonzero(roe >= 0)[0]                          # an empty slot adds 0 (R26)
    rows[a] = y_perm[roe[a]] * w[a, None]                 # entry a's term
    return rows.reshape(T, k, -1).sum(axis=1)


# --------------------------------------------------------------------------
# Expert FFN: gated SiLU  ([FL] gated + silu; [MB] §3, §5 GLU variant)
# --------------------------------------------------------------------------

def sigmoid(z):
    z = _f64(z)
    return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    z = _f64(z)
    return z / (1.0 + np.exp(-z))


def forward_loop(x, top_experts, weights, w1, w3, w2):
    """The layer's definition, one (token, slot) entry at a time.

    For token t and slot j with e = top_experts[t, j]:
    u1 = x[t] w1[e], u3 = x[t] w3[e], act = silu(u1) * u3, o = act w2[e],
    y[t] = sum_j weights[t, j] * o.  No token is dropped ([MB] §1, §4.5).
    Returns y and the per-entry (u1, u3, act, o), entry a = t*k + j.
    """
    x, w = _f64(x), _f64(weights)
    ids = np.asarray(top_experts)
    T, k = ids.shape
    F, H = np.shape(w2)[1], x.shape[1]
    y = np.zeros((T, H))
    u1s, u3s, acts, outs = (np.zeros((T * k, F)), np.zeros((T * k, F)),
                            np.zeros((T * k, F)), np.zeros((T * k, H)))
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if e < 0:                        # R26: an empty slot
                continue
            u1 = x[t] @ _f64(w1[e])
            u3 = x[t] @ _f64(w3[e])
            act = silu(u1) * u3
            o = act @ _f64(w2[e])
            y[t] += w[t, j] * o
            a = t * k + j
            u1s[a], u3s[a], acts[a], outs[a] = u1, u3, act, o
    return y, dict(u1=u1s, u3=u3s, act=acts, o=outs)


def backward_loop(x, top_experts, weights, w1, w3, w2, dy):
    """Gradients of sum(y * dy), one entry at a time (chain rule of
    ``forward_loop``; the routing-weight gradient is the dot product of dy
    with the expert output, [MB] §4.2 wgrad kernel).

    With s = sigmoid(u1): d silu(u1)/du1 = s * (1 + u1 * (1 - s)).
    """
    x, w, dy = _f64(x), _f64(weights), _f64(dy)
    ids = np.asarray(top_experts)
    T, k = ids.shape
    E = np.shape(w1)[0]
    dx = np.zeros_like(x)
    dw1 = np.zeros(np.shape(w1))
    dw3 = np.zeros(np.shape(w3))
    dw2 = np.zeros(np.shape(w2))
    dwts = np.zeros((T, k))
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if e < 0:                        # R26: an empty slot
                continue
            W1, W3, W2 = _f64(w1[e]), _f64(w3[e]), _f64(w2[e])
            u1 = x[t] @ W1
            u3 = x[t] @ W3
            s = sigmoid(u1)
            g = u1 * s
            act = g * u3
            o = act @ W2
            dwts[t, j] = dy[t] @ o
            do = w[t, j] * dy[t]
            dw2[e] += np.outer(act, do)
            da = W2 @ do
            du3 = da * g
            du1 = da * u3 * s * (1.0 + u1 * (1.0 - s))
            dw1[e] += np.outer(x[t], du1)
            dw3[e] += np.outer(x[t], du3)
            dx[t] += W1 @ du1 + W3 @ du3
    assert dw1.shape[0] == E
    return dict(dx=dx, dw1=dw1, dw3=dw3, dw2=dw2, d_weights=dwts)


# --------------------------------------------------------------------------
# The pages' pipeline in the padded layout  ([MB] §3, §4.5)
# --------------------------------------------------------------------------

def _expert_rows(md, e):
    """Padded row range [start, end) of expert e (R1)."""
    end = int(md["padded_bins"][e])
    start = end - int(round_up(md["tokens_per_expert"][e]))
    return start, end


def _expert_forward(xp, W1, W3, W2):
    """One expert's padded rows through its FFN ([MB] §3: the row blocks of
    an expert touch only that expert's weights; [FL] gated SiLU)."""
    h1 = xp @ W1
    h3 = xp @ W3
    act = silu(h1) * h3
    return h1, h3, act, act @ W2


def _expert_backward(xp, h1, h3, act, dyp, W1, W3, W2):
    """The backward of ``_expert_forward`` for upstream dyp (the expert's
    rows of dY_perm): dA = dY w2^T, the gated-SiLU derivative
    (d silu(u)/du = s (1 + u (1 - s)), s = sigmoid(u)), dw2 = A^T dY,
    dw1 = X^T dH1, dw3 = X^T dH3, dX = dH1 w1^T + dH3 w3^T."""
    da = dyp @ W2.T
    s = sigmoid(h1)
    dh3 = da * h1 * s
    dh1 = da * h3 * s * (1.0 + h1 * (1.0 - s))
    return dict(dh1=dh1, dh3=dh3, dx_perm=dh1 @ W1.T + dh3 @ W3.T,
                dw1=xp.T @ dh1, dw3=xp.T @ dh3, dw2=act.T @ dyp)


def forward_padded(x, top_experts, weights, w1, w3, w2, md=None):
    """Forward through the padded layout, as in [MB] §4.5.

    metadata -> padded gather -> for each expert, the products over its
    padded row range (the row blocks of one expert touch only that expert's
    weight columns, [MB] §3) -> gated SiLU -> down projection -> weighted
    scatter.  Returns y and the padded intermediates.
    """
    ids = np.asarray(top_experts)
    T, k = ids.shape
    E = np.shape(w1)[0]
    if md is None:
        md = metadata(ids, E)
    xp = padded_gather(x, md, k)
    P, F, H = md["P"], np.shape(w1)[2], np.shape(x)[1]
    h1, h3, act, yp = (np.zeros((P, F)), np.zeros((P, F)), np.zeros((P, F)),
                       np.zeros((P, H)))
    for e in range(E):
        r0, r1 = _expert_rows(md, e)
        if r1 == r0:
            continue
        h1[r0:r1], h3[r0:r1], act[r0:r1], yp[r0:r1] = _expert_forward(
            xp[r0:r1], _f64(w1[e]), _f64(w3[e]), _f64(w2[e]))
    y = padded_scatter(yp, md, weights, T, k)
    return y, dict(md=md, x_perm=xp, h1=h1, h3=h3, act=act, y_perm=yp)


def backward_padded(x, top_experts, weights, w1, w3, w2, dy, saved=None):
    """Backward through the padded layout.

    [MB] §4.2: the scatter's backward is a gather of dy times the routing
    weight plus the routing-weight gradient; the gather's backward is a
    scatter (unit weights, summed over the k slots).  In between, per expert:
    dA = dY w2^T, the gated-SiLU derivative, dw2 = A^T dY, dw1 = X^T dH1,
    dw3 = X^T dH3, dX = dH1 w1^T + dH3 w3^T.  An expert with no rows gets
    zero weight gradients.
    """
    ids = np.asarray(top_experts)
    T, k = ids.shape
    E = np.shape(w1)[0]
    if saved is None:
        _, saved = forward_padded(x, ids, weights, w1, w3, w2)
    md = saved["md"]
    w = _f64(weights).reshape(-1)
    dy = _f64(dy)
    P, H = md["P"], dy.shape[1]
    F = np.shape(w1)[2]
    rows = md["row_of_entry"]
    a = np.nonzero(rows >= 0)[0]             # routed entries (R26)
    dyp = np.zeros((P, H))
    dyp[rows[a]] = dy[a // k] * w[a, None]
    d_weights = np.zeros(T * k)
    d_weights[a] = np.einsum("ah,ah->a", dy[a // k], saved["y_perm"][rows[a]])
    d_weights = d_weights.reshape(T, k)
    dh1, dh3, dxp = np.zeros((P, F)), np.zeros((P, F)), np.zeros((P, H))
    dw1 = np.zeros(np.shape(w1))
    dw3 = np.zeros(np.shape(w3))
    dw2 = np.zeros(np.shape(w2))
    xp, h1, h3, act = saved["x_perm"], saved["h1"], saved["h3"], saved["act"]
    for e in range(E):
        r0, r1 = _expert_rows(md, e)
        if r1 == r0:
            continue
        g = _expert_backward(xp[r0:r1], h1[r0:r1], h3[r0:r1], act[r0:r1], dyp[r0:r1],
                             _f64(w1[e]), _f64(w3[e]), _f64(w2[e]))
        dh1[r0:r1], dh3[r0:r1], dxp[r0:r1] = g["dh1"], g["dh3"], g["dx_perm"]
        dw1[e], dw3[e], dw2[e] = g["dw1"], g["dw3"], g["dw2"]
    terms = np.zeros((T * k, H))
    terms[a] = dxp[rows[a]]
    dx = terms.reshape(T, k, H).sum(axis=1)
    return dict(dx=dx, dw1=dw1, dw3=dw3, dw2=dw2, d_weights=d_weights,
                dy_perm=dyp, dh1=dh1, dh3=dh3, dx_perm=dxp)


def layer_by_expert(x, top_experts, weights, w1, w3, w2, dy, out, md=None):
    """The forward and backward of ``forward_padded`` / ``backward_padded``,
    one expert at a time, for layers too large to hold every fp64
    intermediate at once.

    Yields, per expert e in order, a dict with its padded row range
    ``rows`` = (r0, r1), its rows of x_perm, h1, h3, act, y_perm, dy_perm,
    dh1, dh3, dx_perm (pad rows zero, as in the padded layout) and dw1[e],
    dw3[e], dw2[e] (zeros for an empty expert).  Meanwhile it adds each
    real row's share into ``out["y"]`` [T,H] and ``out["dx"]`` [T,H] and
    writes ``out["d_weights"]`` [T,k] (fp64 arrays the caller provides,
    zero-filled): the weighted scatter with the top-k sum and the gather's
    backward of [MB] §4.2, and the routing-weight gradient
    <dy[a // k], y_perm[row_of_entry[a]]>.  When the generator is exhausted,
    those three arrays hold y, dx and d_weights.
    """
    ids = np.asarray(top_experts)
    T, k = ids.shape
    E, H, F = np.shape(w1)
    if md is None:
        md = metadata(ids, E)
    wflat = _f64(weights).reshape(-1)
    rows = md["row_of_entry"]
    for e in range(E):
        r0, r1 = _expert_rows(md, e)
        n = r1 - r0
        if n == 0:
            yield dict(e=e, rows=(r0, r1), dw1=np.zeros((H, F)), dw3=np.zeros((H, F)),
                       dw2=np.zeros((F, H)))
            continue
        ent = md["indices"][md["bins"][e] - md["tokens_per_expert"][e]:md["bins"][e]]
        loc = rows[ent] - r0                 # the entries' rows within the expert
        tok = ent // k
        xp = np.zeros((n, H))
        xp[loc] = _f64(x[tok])
        W1, W3, W2 = _f64(w1[e]), _f64(w3[e]), _f64(w2[e])
        h1, h3, act, yp = _expert_forward(xp, W1, W3, W2)
        dyt = _f64(dy[tok])
        dyp = np.zeros((n, H))
        dyp[loc] = dyt * wflat[ent][:, None]
        g = _expert_backward(xp, h1, h3, act, dyp, W1, W3, W2)
        np.add.at(out["y"], tok, yp[loc] * wflat[ent][:, None])
        np.add.at(out["dx"], tok, g["dx_perm"][loc])
        out["d_weights"].reshape(-1)[ent] = np.einsum("ah,ah->a", dyt, yp[loc])
        yield dict(e=e, rows=(r0, r1), x_perm=xp, h1=h1, h3=h3, act=act, y_perm=yp,
                   dy_perm=dyp, **g)


# --------------------------------------------------------------------------
# Sampled outputs at full size, each from the per-entry definition
# --------------------------------------------------------------------------

def sampled_rows(x, top_experts, weights, w1, w3, w2, dy,
                 tokens: Iterable[int]):
    """y[t], dx[t] and d_weights[t, :] for a few tokens, by the per-entry
    definition of ``forward_loop``/``backward_loop`` (no other token is
    needed for these rows).  Entries are visited expert by expert so that
    each expert's weights are converted to fp64 once."""
    ids = np.asarray(top_experts)
    k = ids.shape[1]
    tokens = [int(t) for t in tokens]
    H = np.shape(x)[1]
    out = {t: dict(y=np.zeros(H), dx=np.zeros(H), d_weights=np.zeros(k))
           for t in tokens}
    by_expert: Dict[int, list] = {}
    for t in tokens:
        for j in range(k):
            if int(ids[t, j]) >= 0:          # R26: an empty slot adds nothing
                by_expert.setdefault(int(ids[t, j]), []).append((t, j))
    for e, ents in sorted(by_expert.items()):
        W1, W3, W2 = _f64(w1[e]), _f64(w3[e]), _f64(w2[e])
        for t, j in ents:
            xt, dyt = _f64(x[t]), _f64(dy[t])
            u1, u3 = xt @ W1, xt @ W3
            s = sigmoid(u1)
            g = u1 * s
            o = (g * u3) @ W2
            wt = float(weights[t, j])
            out[t]["y"] += wt * o
            out[t]["d_weights"][j] = dyt @ o
            da = W2 @ (wt * dyt)
            du1 = da * u3 * s * (1.0 + u1 * (1.0 - s))
            du3 = da * g
            out[t]["dx"] += W1 @ du1 + W3 @ du3
    return out


def sampled_dw(x, top_experts, weights, w1, w3, w2, dy,
               picks: Sequence[Tuple[str, int, int, int]]):
    """Single elements of dw1/dw3/dw2, each summed over the entries routed to
    its expert, by the per-entry definition of ``backward_loop``.

    ``picks`` holds (name, e, i, j) with name in {"dw1","dw3","dw2"}:
    dw1[e][h, f] and dw3[e][h, f] (i = h, j = f), dw2[e][f, h] (i = f, j = h).
    """
    ids = np.asarray(top_experts)
    T, k = ids.shape
    flat = ids.reshape(-1)
    wflat = _f64(weights).reshape(-1)
    res = []
    cache = {}
    for name, e, i, j in picks:
        if e not in cache:
            ent = np.nonzero(flat == e)[0]           # entries of expert e
            if ent.size:
                xe = _f64(x[ent // k])                         # [n_e, H]
                do = _f64(dy[ent // k]) * wflat[ent][:, None]  # [n_e, H]
            else:
                xe = do = None
            cache[e] = (ent, xe, do)
        ent, xe, do = cache[e]
        if ent.size == 0:
            res.append(0.0)
            continue
        if name == "dw2":
            f, h = i, j
            u1 = xe @ _f64(w1[e][:, f])
            u3 = xe @ _f64(w3[e][:, f])
            act = silu(u1) * u3
            res.append(float(act @ do[:, h]))
        else:
            h, f = i, j
            u1 = xe @ _f64(w1[e][:, f])
            u3 = xe @ _f64(w3[e][:, f])
            s = sigmoid(u1)
            da = do @ _f64(w2[e][f, :])
            if name == "dw1":
                du = da * u3 * s * (1.0 + u1 * (1.0 - s))
            elif name == "dw3":
                du = da * u1 * s
            else:
                raise ValueError(name)
            res.append(float(xe[:, h] @ du))
    return np.asarray(res)
