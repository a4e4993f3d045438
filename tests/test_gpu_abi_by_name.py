"""The three calls of the boundary, dmoe_metadata, dmoe_forward and
dmoe_backward, called by name through ctypes with raw device pointers and
the raw stream handle (no binding helper in between), against the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import dropless_mixture_experts_amd as dm
import oracle
from workloads import CONFIGS, make_inputs, shrink

from gpu_helpers import TOL, assert_close, device, down, torch_dtype, up

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [
    shrink(CONFIGS["zipf_e64_empty"], T=700, H=256, F=384),   # empty experts, odd blocks
    shrink(CONFIGS["tiny_f32"], T=300, H=128, F=256),
], ids=lambda c: c.name)
def test_metadata_forward_backward_by_name(cfg):
    dev = device()
    lib = dm.load_library()
    inp = make_inputs(cfg)
    print(f"by name {cfg.name}", flush=True)
    dt = torch_dtype(cfg)
    T, H, F, E, k = cfg.T, cfg.H, cfg.F, cfg.E, cfg.k
    dims = dm._Dims(T, H, F, E, k, dm.DMOE_F32 if cfg.dtype == "f32" else dm.DMOE_BF16)
    nt = lib.dmoe_max_tiles(ctypes.byref(dims))
    ws_bytes = lib.dmoe_workspace_bytes(ctypes.byref(dims))
    sched_bytes = lib.dmoe_schedule_bytes(ctypes.byref(dims))
    assert nt > 0 and ws_bytes > 0 and sched_bytes > 0
    pm = 128 * nt
    i32 = dict(dtype=torch.int32, device=dev)
    arrays = [torch.empty(E, **i32), torch.empty(E, **i32), torch.empty(E, **i32),
              torch.empty(T * k, **i32), torch.empty(T * k, **i32), torch.empty(T * k, **i32),
              torch.empty(nt, **i32), torch.empty(1, **i32), torch.empty(1, **i32),
              torch.empty(pm, **i32), torch.empty(sched_bytes, dtype=torch.uint8, device=dev)]
    meta = dm._Meta(*[ctypes.c_void_p(a.data_ptr()) for a in arrays])
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    fl = dict(dtype=dt, device=dev)
    saved_t = [torch.empty(pm, H, **fl), torch.empty(pm, F, **fl), torch.empty(pm, F, **fl),
               torch.empty(pm, F, **fl), torch.empty(pm, H, **fl)]
    scratch_t = [torch.empty(pm, H, **fl), torch.empty(pm, F, **fl), torch.empty(pm, F, **fl),
                 torch.empty(pm, H, **fl)]
    saved = dm._Saved(*[ctypes.c_void_p(a.data_ptr()) for a in saved_t])
    scratch = dm._Scratch(*[ctypes.c_void_p(a.data_ptr()) for a in scratch_t])
    x, ids = up(inp.x, dt, dev), up(inp.top_experts, torch.int32, dev)
    w = up(inp.weights, torch.float32, dev)
    w1, w3, w2, dy = (up(a, dt, dev) for a in (inp.w1, inp.w3, inp.w2, inp.dy))
    y, dx = torch.empty(T, H, **fl), torch.empty(T, H, **fl)
    dw1, dw3 = torch.empty(E, H, F, **fl), torch.empty(E, H, F, **fl)
    dw2 = torch.empty(E, F, H, **fl)
    dwts = torch.empty(T, k, dtype=torch.float32, device=dev)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    assert lib.dmoe_metadata(ctypes.byref(dims), p(ids), ctypes.byref(meta), p(ws), stream) == 0
    assert lib.dmoe_forward(ctypes.byref(dims), p(x), p(w), p(w1), p(w3), p(w2),
                            ctypes.byref(meta), ctypes.byref(saved), p(y), stream) == 0
    assert lib.dmoe_backward(ctypes.byref(dims), p(dy), p(w), p(w1), p(w3), p(w2),
                             ctypes.byref(meta), ctypes.byref(saved), ctypes.byref(scratch),
                             p(dx), p(dw1), p(dw3), p(dw2), p(dwts), stream) == 0
    torch.cuda.synchronize()
    assert int(arrays[8].item()) == 0
    md = oracle.metadata(inp.top_experts, E, nt)
    for i, key in enumerate(("tokens_per_expert", "bins", "padded_bins", "indices",
                             "bin_ids", "row_of_entry", "tile_expert")):
        np.testing.assert_array_equal(arrays[i].cpu().numpy(), md[key], err_msg=key)
    assert int(arrays[7].item()) == md["P"]
    ref_y, sv = oracle.forward_padded(inp.x, inp.top_experts, inp.weights, inp.w1, inp.w3,
                                      inp.w2)
    ref = oracle.backward_padded(inp.x, inp.top_experts, inp.weights, inp.w1, inp.w3,
                                 inp.w2, inp.dy, sv)
    tol = TOL[cfg.dtype]
    assert np.array_equal(down(saved_t[0][:md["P"]]), sv["x_perm"])
    assert_close(down(y), ref_y, tol, "y")
    for key, got in (("dx", dx), ("dw1", dw1), ("dw3", dw3), ("dw2", dw2),
                     ("d_weights", dwts)):
        assert_close(down(got), ref[key], tol, key)
