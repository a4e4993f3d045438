"""Forward + backward of the whole layer on the GPU vs the fp64 oracle.

Small cases (several 128-row tiles, ragged tails, empty experts) and every
workload at full size compare every output and every intermediate element by
element; at full size the oracle runs one expert at a time
(oracle.layer_by_expert), and sampled outputs that it computes one by one
from the per-entry definition give a second opinion."""
import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, make_inputs, shrink

from gpu_helpers import TOL, Run, assert_close, down, torch_dtype, up

pytestmark = pytest.mark.gpu

OUTS = ("dx", "dw1", "dw3", "dw2", "d_weights")

SMALL = [
    CONFIGS["tiny_f32"],
    shrink(CONFIGS["fine_e64"], T=512, H=256, F=256),
    shrink(CONFIGS["zipf_e64"], T=1024, H=256, F=256),
    shrink(CONFIGS["zipf_e64_empty"], T=1024, H=128, F=256),
    shrink(CONFIGS["coarse_e8"], T=1024, H=512, F=1024),
    shrink(CONFIGS["sparse_e256"], T=2048, H=384, F=256),
    # edge cases
    shrink(CONFIGS["fine_e64"], T=5, H=128, F=128, E=1, k=1),      # one expert, ragged
    shrink(CONFIGS["fine_e64"], T=1, H=256, F=128, E=4, k=2),      # one token
    shrink(CONFIGS["fine_e64"], T=200, H=128, F=128, E=4, k=4),    # k = E
    shrink(CONFIGS["fine_e64"], T=128, H=256, F=384, E=1, k=1),    # exactly one tile
    shrink(CONFIGS["sparse_e256"], T=16, H=128, F=128),            # most experts empty
    shrink(CONFIGS["tiny_f32"], T=129, H=384, F=384, E=3, k=1),    # fp32, 2 tiles + tail
    # 256 expected up-dgrad row tiles (one whole round of 256 CUs): the plain
    # up-dgrad launch, not the one that fills its last round with dw1/dw3 tiles
    shrink(CONFIGS["fine_e64"], T=3584, H=2048, F=128, E=8, k=2),
    # experts with more than 8 row pairs, whose row tiles are split into
    # groups of near-equal size: 17 pairs (6, 6, 5; the last pair half
    # empty), two experts of 12 (6, 6), and skewed experts of 16, 13 and 11
    shrink(CONFIGS["fine_e64"], T=4300, H=128, F=256, E=1, k=1),
    shrink(CONFIGS["fine_e64"], T=3000, H=256, F=256, E=2, k=2),
    shrink(CONFIGS["zipf_e64"], T=4096, H=128, F=128),
]


def _check_small(cfg, lean=False):
    inp = make_inputs(cfg)
    print(f"layer {cfg.name} lean={lean}", flush=True)
    r = Run(inp, lean=lean)
    tol = TOL[cfg.dtype]
    ref_y, sv = oracle.forward_padded(inp.x, inp.top_experts, inp.weights,
                                      inp.w1, inp.w3, inp.w2)
    ref_g = oracle.backward_padded(inp.x, inp.top_experts, inp.weights, inp.w1,
                                   inp.w3, inp.w2, inp.dy, sv)
    md = sv["md"]
    got_md = r.meta_np()
    np.testing.assert_array_equal(got_md["row_of_entry"], md["row_of_entry"])
    P = md["P"]
    assert r.P == P
    # the gather is a copy: bit-exact, pad rows exactly zero
    assert np.array_equal(down(r.saved.x_perm[:P]), sv["x_perm"])
    pad = np.ones(P, dtype=bool)
    pad[md["row_of_entry"]] = False
    assert_close(down(r.y), ref_y, tol, "y")
    for key in OUTS:
        assert_close(down(r.g[key]), ref_g[key], tol, key)
    inter = {"act": (r.saved.act, sv["act"]), "y_perm": (r.saved.y_perm, sv["y_perm"]),
             "dh1": (r.scratch.dh1, ref_g["dh1"]), "dh3": (r.scratch.dh3, ref_g["dh3"]),
             "dx_perm": (r.scratch.dx_perm, ref_g["dx_perm"])}
    if not lean:
        # in lean mode h1/h3 hold dh1/dh3 and dy_perm holds dx_perm afterwards
        inter.update({"h1": (r.saved.h1, sv["h1"]), "h3": (r.saved.h3, sv["h3"]),
                      "dy_perm": (r.scratch.dy_perm, ref_g["dy_perm"])})
    for key, (t, ref) in inter.items():
        got = down(t[:P])
        assert_close(got, ref, tol, key)
        assert np.all(got[pad] == 0.0), f"{key}: pad rows not zero"
    return r


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_small_case_against_oracle(cfg):
    _check_small(cfg)


def test_lean_buffers_match_and_runs_are_bitwise_identical():
    cfg = shrink(CONFIGS["zipf_e64_empty"], T=600, H=256, F=256)
    a = _check_small(cfg, lean=False)
    b = _check_small(cfg, lean=True)
    assert torch.equal(a.y, b.y)
    for key in OUTS:
        assert torch.equal(a.g[key], b.g[key]), key
    c = Run(make_inputs(cfg))
    assert torch.equal(a.y, c.y)
    for key in OUTS:
        assert torch.equal(a.g[key], c.g[key]), key


@pytest.mark.parametrize("name,dims,lean", [
    ("zipf_e64_empty", dict(T=600, H=256, F=256), False),
    ("zipf_e64_empty", dict(T=600, H=256, F=256), True),
    ("coarse_e8", dict(T=1024, H=512, F=1024), True),
    ("tiny_f32", {}, False),
], ids=["zipf_empty", "zipf_empty_lean", "coarse_lean", "tiny_f32"])
def test_backward_recompute_is_bitwise_identical(name, dims, lean):
    """dmoe_backward_recompute with saved.act overwritten by NaN after the
    forward gives the plain backward's results bit for bit, and rebuilds act
    as the forward wrote it."""
    cfg = shrink(CONFIGS[name], **dims) if dims else CONFIGS[name]
    inp = make_inputs(cfg)
    print(f"recompute {cfg.name} lean={lean}", flush=True)
    a = Run(inp, lean=lean)
    b = Run(inp, lean=lean, backward=False)
    P = b.P
    act_fwd = b.saved.act[:P].clone()
    b.saved.act.fill_(float("nan"))
    dy = up(inp.dy, torch_dtype(cfg), b.dev)
    g = b.layer.backward(dy, b.w, b.w1, b.w3, b.w2, recompute=True)
    torch.cuda.synchronize()
    assert torch.equal(b.saved.act[:P], act_fwd)
    for key in OUTS:
        assert torch.equal(g[key], a.g[key]), key


@pytest.mark.parametrize("name,dims,aliased,fused", [
    ("zipf_e64_empty", dict(T=600, H=256, F=256), False, False),
    ("zipf_e64_empty", dict(T=600, H=256, F=256), True, False),
    ("coarse_e8", dict(T=1024, H=512, F=1024), True, True),
    ("tiny_f32", {}, False, False),
    ("fine_e64", {}, False, False),
    ("sparse_e256", {}, True, True),
], ids=["zipf_empty", "zipf_empty_aliased", "coarse_aliased_fused", "tiny_f32",
        "fine_e64_full", "sparse_e256_full_aliased_fused"])
def test_backward_lean_is_bitwise_identical(name, dims, aliased, fused):
    """dmoe_backward_lean with x_perm, h1, h3 and act overwritten by NaN
    after the forward (only y_perm kept) gives the plain backward's results
    bit for bit, and rebuilds the four buffers as the forward wrote them."""
    cfg = shrink(CONFIGS[name], **dims) if dims else CONFIGS[name]
    inp = make_inputs(cfg)
    print(f"lean {cfg.name} aliased={aliased} fused={fused}", flush=True)
    a = Run(inp, lean=aliased)
    b = Run(inp, lean=aliased, backward=False, fused_gather=fused)
    P = b.P
    fwd = {n: getattr(b.saved, n)[:P].clone() for n in ("h1", "h3", "act")}
    for n in ("x_perm", "h1", "h3", "act"):
        getattr(b.saved, n).fill_(float("nan"))
    dy = up(inp.dy, torch_dtype(cfg), b.dev)
    g = b.layer.backward(dy, b.w, b.w1, b.w3, b.w2, lean=True)
    torch.cuda.synchronize()
    assert torch.equal(b.y, a.y)
    for key in OUTS:
        assert torch.equal(g[key], a.g[key]), key
    # the rebuilt x_perm, and (where the backward does not overwrite them
    # with dh1/dh3) h1 and h3; act is never overwritten
    assert torch.equal(b.saved.x_perm[:P], a.saved.x_perm[:P])
    assert torch.equal(b.saved.act[:P], fwd["act"])
    if not aliased:
        assert torch.equal(b.saved.h1[:P], fwd["h1"])
        assert torch.equal(b.saved.h3[:P], fwd["h3"])
    for n in ("dy_perm", "dh1", "dh3", "dx_perm"):
        assert torch.equal(getattr(b.scratch, n)[:P], getattr(a.scratch, n)[:P]), n


def _picks(inp, md, rng, n=24):
    cfg = inp.cfg
    counts = md["tokens_per_expert"]
    big = int(np.argmax(counts))
    experts = [big] + list(rng.integers(0, cfg.E, n - 1))
    empty = np.nonzero(counts == 0)[0]
    if empty.size:
        experts[1] = int(empty[0])
    picks = []
    for i, e in enumerate(experts):
        e = int(e)
        picks.append(("dw1", e, int(rng.integers(cfg.H)), int(rng.integers(cfg.F))))
        picks.append(("dw3", e, int(rng.integers(cfg.H)), int(rng.integers(cfg.F))))
        picks.append(("dw2", e, int(rng.integers(cfg.F)), int(rng.integers(cfg.H))))
    return picks


# Padded buffers of 4.4 GB each (P x H x 2 > 2^32 bytes): every offset past
# 32 bits, at the largest row counts the tests reach.
LARGE = shrink(CONFIGS["fine_e64"], T=32768, H=8192, F=128)


def _elementwise(r, inp, md, tol, name):
    """Every output and every intermediate below P, element by element,
    against the oracle taken one expert at a time: metadata bit-exact, x_perm
    bit-exact, the rest within tol * max|ref| of each whole tensor."""
    cfg = inp.cfg
    out = dict(y=np.zeros((cfg.T, cfg.H)), dx=np.zeros((cfg.T, cfg.H)),
               d_weights=np.zeros((cfg.T, cfg.k)))
    worst = {}

    def note(key, got, ref):
        err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
        scale = float(np.max(np.abs(ref))) if ref.size else 0.0
        assert np.all(np.isfinite(got)), f"{name} {key}: non-finite values"
        e0, s0 = worst.get(key, (0.0, 0.0))
        worst[key] = (max(e0, err), max(s0, scale))

    bufs = {"h1": r.saved.h1, "h3": r.saved.h3, "act": r.saved.act,
            "y_perm": r.saved.y_perm, "dy_perm": r.scratch.dy_perm,
            "dh1": r.scratch.dh1, "dh3": r.scratch.dh3, "dx_perm": r.scratch.dx_perm}
    for res in oracle.layer_by_expert(inp.x, inp.top_experts, inp.weights, inp.w1,
                                      inp.w3, inp.w2, inp.dy, out, md=md):
        e, (r0, r1) = res["e"], res["rows"]
        for key in ("dw1", "dw3", "dw2"):
            got = down(r.g[key][e])
            if r1 == r0:
                assert np.all(got == 0.0), f"{name} {key}[{e}]: empty expert not zero"
            note(key, got, res[key])
        if r1 == r0:
            continue
        assert np.array_equal(down(r.saved.x_perm[r0:r1]), res["x_perm"]), \
            f"{name} x_perm rows of expert {e}"
        for key, t in bufs.items():
            note(key, down(t[r0:r1]), res[key])
    note("y", down(r.y), out["y"])
    note("dx", down(r.g["dx"]), out["dx"])
    note("d_weights", down(r.g["d_weights"]), out["d_weights"])
    for key, (err, scale) in sorted(worst.items()):
        print(f"  {name} {key}: max err {err:.3e}, max|ref| {scale:.3e}", flush=True)
        assert err <= tol * scale, f"{name} {key}: max err {err:.3e} > {tol} * {scale:.3e}"
    assert set(worst) == {"dw1", "dw3", "dw2", "y", "dx", "d_weights", *bufs}


def _sampled(r, inp, md, tol, name):
    """A second opinion from the per-entry definition: rows of y and dx,
    d_weights of a few tokens, and single weight-gradient elements, each
    computed on its own by the oracle."""
    cfg = inp.cfg
    rng = np.random.default_rng(17)
    toks = sorted(set([0, cfg.T - 1] + list(rng.integers(0, cfg.T, 22))))
    ref = oracle.sampled_rows(inp.x, inp.top_experts, inp.weights, inp.w1, inp.w3,
                              inp.w2, inp.dy, toks)
    idx = torch.tensor(toks, device=r.dev)
    for key, got in (("y", r.y), ("dx", r.g["dx"]), ("d_weights", r.g["d_weights"])):
        g = down(got[idx])
        want = np.stack([ref[t][key] for t in toks])
        assert_close(g, want, tol, f"{name} {key}")
    picks = _picks(inp, md, rng)
    want = oracle.sampled_dw(inp.x, inp.top_experts, inp.weights, inp.w1, inp.w3,
                             inp.w2, inp.dy, picks)
    for nm in ("dw1", "dw3", "dw2"):
        sel = [i for i, p in enumerate(picks) if p[0] == nm]
        got = np.array([float(r.g[nm][p[1], p[2], p[3]]) for p in
                        (picks[i] for i in sel)])
        scale = float(np.max(np.abs(want[sel])))
        err = float(np.max(np.abs(got - want[sel])))
        assert err <= tol * scale, f"{name} {nm}: {err:.3e} > {tol}*{scale:.3e}"


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny_f32", "fine_e64", "zipf_e64",
                                  "zipf_e64_empty", "coarse_e8", "sparse_e256",
                                  "large_over_4gb"])
def test_full_size(name):
    """The launch sequence the benchmark times, at the workload's full size:
    every output and intermediate element by element against the oracle,
    plus sampled per-entry values as a second opinion."""
    cfg = LARGE if name == "large_over_4gb" else CONFIGS[name]
    inp = make_inputs(cfg)
    print(f"full {name}", flush=True)
    r = Run(inp)
    if name == "large_over_4gb":
        assert r.P * cfg.H * 2 > (1 << 32)
        f = Run(inp, fused_gather=True)
        assert torch.equal(f.y, r.y)
        for key in OUTS:
            assert torch.equal(f.g[key], r.g[key]), key
        del f
    tol = TOL[cfg.dtype]
    md = oracle.metadata(inp.top_experts, cfg.E, len(r.meta.tile_expert))
    got_md = r.meta_np()
    for key in ("tokens_per_expert", "bins", "padded_bins", "indices", "bin_ids",
                "row_of_entry", "tile_expert"):
        np.testing.assert_array_equal(got_md[key], md[key], err_msg=key)
    P = md["P"]
    assert r.P == P
    # pad rows of every padded buffer are exact zeros
    rows = torch.from_numpy(md["row_of_entry"]).to(r.dev)
    pad = torch.ones(P, dtype=torch.bool, device=r.dev)
    pad[rows] = False
    for t in (r.saved.x_perm, r.saved.h1, r.saved.h3, r.saved.act, r.saved.y_perm,
              r.scratch.dy_perm, r.scratch.dh1, r.scratch.dh3, r.scratch.dx_perm):
        assert int(torch.count_nonzero(t[:P][pad])) == 0
    _sampled(r, inp, md, tol, name)
    _elementwise(r, inp, md, tol, name)


def test_full_size_runs_are_bitwise_identical():
    """Two runs of the whole layer at the headline size agree bit for bit in
    every output, every saved activation and every backward intermediate (no
    reduction uses atomics)."""
    inp = make_inputs(CONFIGS["fine_e64"])
    print("bitwise fine_e64", flush=True)
    a = Run(inp)
    b = Run(inp)
    assert torch.equal(a.y, b.y)
    for key in OUTS:
        assert torch.equal(a.g[key], b.g[key]), key
    P = a.P
    for name in ("x_perm", "h1", "h3", "act", "y_perm"):
        assert torch.equal(getattr(a.saved, name)[:P], getattr(b.saved, name)[:P]), name
    for name in ("dy_perm", "dh1", "dh3", "dx_perm"):
        assert torch.equal(getattr(a.scratch, name)[:P], getattr(b.scratch, name)[:P]), name
