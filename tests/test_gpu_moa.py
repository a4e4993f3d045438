"""dMoA map / reduce on the GPU against the fp64 oracle (oracle/moa.py):
every output and gradient element by element, on small edge shapes, on a
shape with H != F, on a mid-size layer, and composed with a causal
attention the way the "yikangshen/megablocks" README composes them."""
import dataclasses

import numpy as np
import pytest
import torch

import dropless_mixture_experts_amd as dm
from oracle import moa
from workloads import CONFIGS, make_inputs, round_to_bf16, shrink

from gpu_helpers import TOL, assert_close, device, down, up

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _run(cfg, ids=None, seed=0):
    """map, reduce and both backward passes on seeded bf16 inputs; returns
    the GPU results and the oracle's."""
    dev = device()
    inp = make_inputs(cfg)
    T, H, F, E, k = cfg.T, cfg.H, cfg.F, cfg.E, cfg.k
    top = inp.top_experts if ids is None else ids
    w = inp.weights.copy()
    w[top < 0] = 0.0
    rng = np.random.default_rng(1000 + seed)
    y = round_to_bf16(rng.standard_normal((T * k, F)).astype(np.float32))
    dq = round_to_bf16(rng.standard_normal((T * k, F)).astype(np.float32))
    dout = inp.dy
    print(f"moa T={T} H={H} F={F} E={E} k={k}", flush=True)
    D = dm.Dims(T, H, F, E, k, dm.DMOE_BF16)
    L = dm.DMoALayer(D, dev)
    L.metadata(up(top, torch.int32, dev))
    x_g, w1_g, w2_g = up(inp.x, BF, dev), up(inp.w1, BF, dev), up(inp.w2, BF, dev)
    w_g = up(w, torch.float32, dev)
    q = L.map(x_g, w1_g)
    out = L.reduce(up(y, BF, dev), w_g, w2_g)
    dy, dw2, dwt = L.reduce_backward(up(dout, BF, dev), w_g, w2_g)
    dx, dw1 = L.map_backward(up(dq, BF, dev), w1_g)
    torch.cuda.synchronize()
    assert int(L.meta.status.item()) == 0
    got = dict(q=down(q).reshape(T, k, F), out=down(out), dy=down(dy).reshape(T, k, F),
               dw2=down(dw2), d_weights=down(dwt), dx=down(dx), dw1=down(dw1))
    ref = dict(q=moa.map_forward(inp.x, top, inp.w1),
               out=moa.reduce_forward(y.reshape(T, k, F), top, w, inp.w2))
    ref["dy"], ref["dw2"], ref["d_weights"] = moa.reduce_backward(
        y.reshape(T, k, F), top, w, inp.w2, dout)
    ref["dx"], ref["dw1"] = moa.map_backward(inp.x, top, inp.w1, dq.reshape(T, k, F))
    return got, ref, top


def _check(got, ref, top, name):
    for key in ref:
        assert_close(got[key], ref[key], TOL["bf16"], f"{name}:{key}")
    # empty slots: zero query rows, zero dy rows, zero routing-weight gradient
    assert np.all(got["q"][top < 0] == 0) and np.all(got["dy"][top < 0] == 0)
    assert np.all(got["d_weights"][top < 0] == 0)


@pytest.mark.parametrize("cfg", [
    shrink(CONFIGS["fine_e64"], T=300, H=256, F=384, E=8, k=2),
    shrink(CONFIGS["fine_e64"], T=257, H=512, F=128, E=5, k=3),     # H > F, ragged T
    shrink(CONFIGS["zipf_e64_empty"], T=700, H=256, F=256),          # skew, empty experts
    shrink(CONFIGS["fine_e64"], T=1, H=128, F=128, E=1, k=1),
    shrink(CONFIGS["fine_e64"], T=90, H=128, F=256, E=4, k=4),       # k = E
], ids=lambda c: f"{c.name}_T{c.T}_H{c.H}_F{c.F}_E{c.E}_k{c.k}")
def test_small_shapes(cfg):
    got, ref, top = _run(cfg)
    _check(got, ref, top, cfg.name)


def test_empty_slots():
    cfg = shrink(CONFIGS["fine_e64"], T=400, H=256, F=256, E=8, k=3)
    inp = make_inputs(cfg)
    ids = inp.top_experts.copy()
    ids[np.random.default_rng(5).random(ids.shape) < 0.3] = -1
    ids[:4] = -1                      # tokens routed nowhere
    got, ref, top = _run(cfg, ids=ids)
    _check(got, ref, top, "empty_slots")
    np.testing.assert_array_equal(got["out"][:4], 0.0)
    np.testing.assert_array_equal(got["dx"][:4], 0.0)


@pytest.mark.timeout(600)
def test_mid_size_layer():
    """A mixture-of-attention-heads projection of width 1024 with 16 experts,
    top-4, 2048 tokens: several row-tile rounds and full dw tiles."""
    cfg = shrink(CONFIGS["fine_e64"], T=2048, H=1024, F=1024, E=16, k=4)
    got, ref, top = _run(cfg, seed=1)
    _check(got, ref, top, "mid")


@pytest.mark.timeout(900)
def test_full_size_bench_workload():
    """The moa_e16 layer that bench.py times (4096 tokens, H = F = 2048, 16
    experts, top-4), every output and gradient element by element."""
    cfg = CONFIGS["moa_e16"]
    got, ref, top = _run(cfg, seed=3)
    _check(got, ref, top, cfg.name)


def test_run_to_run_bitwise():
    cfg = shrink(CONFIGS["fine_e64"], T=600, H=256, F=256, E=8, k=2)
    a, _, _ = _run(cfg, seed=2)
    b, _, _ = _run(cfg, seed=2)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)


def _attention64(q, kk, v):
    """Causal softmax attention in fp64: q [T, nh, hs], kk, v [T, nh, hs]."""
    T, nh, hs = q.shape
    s = np.einsum("thd,uhd->htu", q, kk) / np.sqrt(hs)
    s = np.where(np.tril(np.ones((T, T), dtype=bool))[None], s, -np.inf)
    s = np.exp(s - s.max(axis=2, keepdims=True))
    p = s / s.sum(axis=2, keepdims=True)
    return np.einsum("htu,uhd->thd", p, v)


def test_composed_with_attention():
    """The README's layout: map(x) viewed as k * n_head query heads, keys and
    values shared by the k slots, causal attention, then reduce.  Attention
    runs in fp32 on the GPU between the two calls and in fp64 beside the
    oracle."""
    dev = device()
    cfg = shrink(CONFIGS["fine_e64"], T=256, H=256, F=256, E=4, k=2)
    inp = make_inputs(cfg)
    T, C, E, k, nh = cfg.T, cfg.H, cfg.E, cfg.k, 4
    hs = C // nh
    rng = np.random.default_rng(11)
    kk = round_to_bf16(rng.standard_normal((T, C)).astype(np.float32))
    vv = round_to_bf16(rng.standard_normal((T, C)).astype(np.float32))
    D = dm.Dims(T, C, C, E, k, dm.DMOE_BF16)
    L = dm.DMoALayer(D, dev)
    L.metadata(up(inp.top_experts, torch.int32, dev))
    q = L.map(up(inp.x, BF, dev), up(inp.w1, BF, dev))
    # q [T*k, C] -> [T, k*nh, hs]; keys and values repeated for the k slots
    qh = q.float().reshape(T, k * nh, hs)
    kh = up(kk, torch.float32, dev).reshape(T, nh, hs).repeat(1, k, 1)
    vh = up(vv, torch.float32, dev).reshape(T, nh, hs).repeat(1, k, 1)
    s = torch.matmul(qh.permute(1, 0, 2).contiguous(),
                     kh.permute(1, 2, 0).contiguous()) / float(np.sqrt(hs))
    s = s.masked_fill(~torch.ones(T, T, dtype=torch.bool, device=dev).tril(), float("-inf"))
    att = torch.matmul(torch.softmax(s, dim=2), vh.permute(1, 0, 2).contiguous())
    y = att.permute(1, 0, 2).reshape(T * k, C).to(BF).contiguous()
    out = L.reduce(y, up(inp.weights, torch.float32, dev), up(inp.w2, BF, dev))
    torch.cuda.synchronize()
    # the same on the CPU in fp64, from the oracle's map
    q64 = moa.map_forward(inp.x, inp.top_experts, inp.w1).reshape(T, k * nh, hs)
    k64 = np.tile(kk.astype(np.float64).reshape(T, nh, hs), (1, k, 1))
    v64 = np.tile(vv.astype(np.float64).reshape(T, nh, hs), (1, k, 1))
    y64 = _attention64(q64, k64, v64).reshape(T, k, C)
    ref = moa.reduce_forward(y64, inp.top_experts, inp.weights, inp.w2)
    # bf16 q and y round twice on the GPU side
    assert_close(down(out), ref, 3e-2, "composed")


def test_rejects_bad_arguments():
    dev = device()
    D32 = dm.Dims(64, 128, 128, 4, 2, dm.DMOE_F32)
    with pytest.raises(dm.DMoEError):
        dm.DMoALayer(D32, dev)
    D = dm.Dims(64, 128, 128, 4, 2, dm.DMOE_BF16)
    L = dm.DMoALayer(D, dev)
    lib = dm.load_library()
    p = L.x_perm
    import ctypes
    # fp32 dims through the C ABI: unsupported, before any launch
    c = ctypes.c_void_p(p.data_ptr())
    assert lib.dmoe_moa_map(ctypes.byref(D32._c()), c, c, ctypes.byref(L.meta._c()), c, c, c,
                            None) == -3
    assert lib.dmoe_moa_map(ctypes.byref(D._c()), None, c, ctypes.byref(L.meta._c()), c, c, c,
                            None) == -1
