"""Seeded synthetic inputs for the dropless-MoE expert layer.

This module only draws inputs.  It holds none of the layer's arithmetic: no
sort, no padding, no expert FFN.  Both the CPU oracle and the HIP path read
their inputs from here, so the two sides see identical values.

Recipe (one numpy stream per tensor, spawned from ``SeedSequence(1000+id)``):

* ``x ~ N(0,1)[T,H]``, ``dy ~ N(0,1)[T,H]``.
* ``w1, w3 ~ N(0, std1)[E,H,F]``, ``w2 ~ N(0, std2)[E,F,H]``.  The
  fine-grained shapes use std1 = 0.02 and std2 = 0.0035355 (= 0.02/sqrt(32)),
  the initialisation of the training config on the Fast-LLM issue
  "[feat] Support sparse copy for a large number of experts".
* Router: logits ``~ N(0,1)[T,E]`` in fp32; ``top_experts`` are the k largest
  logits per token in descending order (ties to the lower id); ``weights`` are
  the softmax over those k logits, computed in fp64 and stored as fp32.
* Zipf routing: expert popularity ``p_e ~ (e+1)^-s``; each token draws k
  distinct experts without replacement from ``p`` (draw order is the j order)
  and its weights are the softmax of its N(0,1) logits at the drawn ids.
  ``zero_ranks`` removes the least popular experts from the draw, which
  forces empty experts.
* Router inputs (``make_logits``): the same fp32 N(0,1) logits the Gaussian
  routing draws from, and upstream gradients ``d_weights ~ N(0,1)[T,k]``.
  ``ties=True`` rounds the logits to multiples of 0.5 in [-2, 2], so that
  most tokens have equal logits among their top k.
* bf16 configs round every floating tensor except the routing weights to
  bf16 on the host (round to nearest even) before either side sees it;
  values are kept as fp32 arrays that hold bf16-representable numbers.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Config", "CONFIGS", "Inputs", "make_inputs", "round_to_bf16",
    "bf16_bits", "bf16_bits_to_f32", "shrink", "make_logits",
]


@dataclasses.dataclass(frozen=True)
class Config:
    """Shape and routing recipe of one synthetic dMoE layer."""
    name: str
    T: int
    H: int
    F: int
    E: int
    k: int
    dtype: str               # "f32" or "bf16"
    routing: str = "gauss"   # "gauss" or "zipf"
    std1: float = 0.02       # std of w1 and w3
    std2: float = 0.02       # std of w2
    zipf_s: float = 1.2
    zero_ranks: int = 0      # least-popular experts removed from the Zipf draw
    seed_id: int = 0

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


_W2_FINE = 0.0035355339059327372

CONFIGS: Dict[str, Config] = {
    # Tiny fp32 layer: T=512, H=128, F=256, E=8, top-2.
    "tiny_f32": Config("tiny_f32", 512, 128, 256, 8, 2, "f32", seed_id=1),
    # Fine-grained bf16 layer: 2x2048 tokens, H=2048, F=1024, E=64, top-8.
    "fine_e64": Config("fine_e64", 4096, 2048, 1024, 64, 8, "bf16",
                       std2=_W2_FINE, seed_id=2),
    # Same shapes, Zipf(1.2) expert popularity.
    "zipf_e64": Config("zipf_e64", 4096, 2048, 1024, 64, 8, "bf16",
                       routing="zipf", std2=_W2_FINE, seed_id=3),
    # Zipf routing with the 8 least popular experts removed: 8 empty experts.
    "zipf_e64_empty": Config("zipf_e64_empty", 4096, 2048, 1024, 64, 8, "bf16",
                             routing="zipf", std2=_W2_FINE, zero_ranks=8,
                             seed_id=33),
    # Coarse-grained bf16 layer: T=8192, H=4096, F=14336, E=8, top-2.
    "coarse_e8": Config("coarse_e8", 8192, 4096, 14336, 8, 2, "bf16", seed_id=4),
    # High-sparsity bf16 layer: T=16384, H=1536, F=256, E=256, top-8.
    "sparse_e256": Config("sparse_e256", 16384, 1536, 256, 256, 8, "bf16",
                          seed_id=5),
    # Mixture of attention heads, the map / reduce pair: 2x2048 tokens, hidden
    # 2048 for both halves (the "yikangshen/megablocks" README example sets
    # ffn_hidden_size to hidden_size), 16 attention experts, top-4.  The pages
    # give no sizes for it; w1 [E,H,F] and w2 [E,F,H] are the two halves, w3
    # is drawn and not used.
    "moa_e16": Config("moa_e16", 4096, 2048, 2048, 16, 4, "bf16", seed_id=6),
}


def shrink(cfg: Config, **dims) -> Config:
    """The same recipe at other sizes (used for small parity cases)."""
    return cfg.replace(name=cfg.name + "_" + "_".join(
        f"{k}{v}" for k, v in sorted(dims.items())), **dims)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 values."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return bf16_bits_to_f32(bf16_bits(a))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Inputs:
    cfg: Config
    x: np.ndarray            # [T,H] fp32 (bf16-representable for bf16 configs)
    top_experts: np.ndarray  # [T,k] int32
    weights: np.ndarray      # [T,k] fp32
    w1: np.ndarray           # [E,H,F]
    w3: np.ndarray           # [E,H,F]
    w2: np.ndarray           # [E,F,H]
    dy: np.ndarray           # [T,H]


def _normal(rng, shape, std, dtype):
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return round_to_bf16(a) if dtype == "bf16" else a


def _softmax64(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.float64)
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


def _route_gauss(rng, T, E, k):
    logits = rng.standard_normal((T, E), dtype=np.float32)
    # descending by value, ties to the lower id: stable sort of the negation
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    chosen = np.take_along_axis(logits, order, axis=1)
    return order.astype(np.int32), _softmax64(chosen).astype(np.float32)


def _route_zipf(rng_logits, rng_zipf, T, E, k, s, zero_ranks):
    p = (np.arange(E, dtype=np.float64) + 1.0) ** (-s)
    if zero_ranks:
        p[E - zero_ranks:] = 0.0
    p /= p.sum()
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        ids[t] = rng_zipf.choice(E, size=k, replace=False, p=p)
    logits = rng_logits.standard_normal((T, E), dtype=np.float32)
    chosen = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    return ids, _softmax64(chosen).astype(np.float32)


def make_inputs(cfg: Config, seed: Optional[int] = None,
                with_weights: bool = True, with_dy: bool = True) -> Inputs:
    """Draw one seeded synthetic layer.  ``seed`` overrides the config's."""
    sid = cfg.seed_id if seed is None else seed
    rl, rx, r1, r3, r2, rdy, rz = (
        np.random.default_rng(s)
        for s in np.random.SeedSequence(1000 + sid).spawn(7))
    T, H, F, E, k = cfg.T, cfg.H, cfg.F, cfg.E, cfg.k
    if cfg.routing == "zipf":
        ids, w = _route_zipf(rl, rz, T, E, k, cfg.zipf_s, cfg.zero_ranks)
    else:
        ids, w = _route_gauss(rl, T, E, k)
    # one stream per tensor: the draws are independent, so they run side by
    # side (numpy releases the GIL while it fills and rounds large arrays)
    jobs = {"x": (rx, (T, H), 1.0)}
    if with_weights:
        jobs.update(w1=(r1, (E, H, F), cfg.std1), w3=(r3, (E, H, F), cfg.std1),
                    w2=(r2, (E, F, H), cfg.std2))
    if with_dy:
        jobs["dy"] = (rdy, (T, H), 1.0)
    with ThreadPoolExecutor(len(jobs)) as ex:
        futs = {n: ex.submit(_normal, r, shape, std, cfg.dtype)
                for n, (r, shape, std) in jobs.items()}
        out = {n: f.result() for n, f in futs.items()}
    return Inputs(cfg, out["x"], ids, w, out.get("w1"), out.get("w3"), out.get("w2"),
                  out.get("dy"))


def make_logits(cfg: Config, seed: Optional[int] = None, ties: bool = False):
    """(logits [T,E] fp32, d_weights [T,k] fp32) for the router.

    The logits are the very values the Gaussian routing of ``make_inputs``
    draws for the same config and seed."""
    sid = cfg.seed_id if seed is None else seed
    rl, rg = (np.random.default_rng(s)
              for s in np.random.SeedSequence(1000 + sid).spawn(8)[0::7])
    logits = rl.standard_normal((cfg.T, cfg.E), dtype=np.float32)
    if ties:
        logits = np.clip(np.round(logits * 2.0) / 2.0, -2.0, 2.0).astype(np.float32)
    d_weights = rg.standard_normal((cfg.T, cfg.k), dtype=np.float32)
    return logits, d_weights
