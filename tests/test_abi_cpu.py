"""The C-ABI library loads and exports every entry point include/dmoe.h
declares; host-side argument checks return their status codes before any
launch (no GPU needed: nothing is enqueued when a check fails)."""
import ctypes
import os
import re

import pytest

import dropless_mixture_experts_amd as dm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dmoe.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dmoe_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dm.library_path()):
        pytest.fail("libdmoe.so is not built: run __graft_entry__.build()")
    return dm.load_library()


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("dmoe_metadata", "dmoe_forward", "dmoe_backward", "dmoe_max_tiles",
              "dmoe_workspace_bytes", "dmoe_schedule_bytes", "dmoe_padded_gather",
              "dmoe_padded_scatter",
              "dmoe_status_string", "dmoe_router_forward", "dmoe_router_backward",
              "dmoe_backward_recompute", "dmoe_backward_recompute_timed",
              "dmoe_forward_fused_gather", "dmoe_backward_fused_gather"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def _dims(**kw):
    d = dict(T=512, H=128, F=256, E=8, k=2, dtype=dm.DMOE_F32)
    d.update(kw)
    return dm._Dims(d["T"], d["H"], d["F"], d["E"], d["k"], d["dtype"])


def test_max_tiles_and_workspace(lib):
    d = _dims()
    # floor((1024 + 127*8)/128) = floor(2040/128) = 15
    assert lib.dmoe_max_tiles(ctypes.byref(d)) == 15
    assert lib.dmoe_workspace_bytes(ctypes.byref(d)) > 0
    # the schedule: 15 + 1 int32, rounded up to 256 bytes
    assert lib.dmoe_schedule_bytes(ctypes.byref(d)) == 256
    d = _dims(T=16384, H=1536, F=256, E=256, k=8)
    assert lib.dmoe_max_tiles(ctypes.byref(d)) == (131072 + 127 * 256) // 128
    assert lib.dmoe_schedule_bytes(ctypes.byref(d)) == (4 * ((131072 + 127 * 256) // 128 + 1)
                                                        + 255) // 256 * 256
    # the largest workspace: 4096 chunks of E = 256 counts and a flag each
    big = _dims(T=268_000_000, k=8, E=256)
    assert 0 < lib.dmoe_workspace_bytes(ctypes.byref(big)) <= 4096 * 257 * 4
    d = _dims(T=1, k=1, E=256)           # min(E, T*k) = 1
    assert lib.dmoe_max_tiles(ctypes.byref(d)) == 1


@pytest.mark.parametrize("kw,code", [
    (dict(F=200), -2), (dict(H=100), -2), (dict(E=257, k=2), -3),
    (dict(k=9, E=8), -1), (dict(T=0), -1), (dict(E=0), -1), (dict(k=0), -1),
    (dict(dtype=7), -3), (dict(T=1 << 29, k=8, E=8), -1)])
def test_bad_dims_rejected(lib, kw, code):
    d = _dims(**kw)
    assert lib.dmoe_max_tiles(ctypes.byref(d)) == code
    assert lib.dmoe_workspace_bytes(ctypes.byref(d)) == code
    assert lib.dmoe_schedule_bytes(ctypes.byref(d)) == code
    meta = dm._Meta(*([ctypes.c_void_p(0x1000)] * 11))
    assert lib.dmoe_metadata(ctypes.byref(d), ctypes.c_void_p(0x1000),
                             ctypes.byref(meta), ctypes.c_void_p(0x1000), None) == code


def test_null_pointers_rejected_before_launch(lib):
    d = _dims()
    meta = dm._Meta(*([ctypes.c_void_p(0x1000)] * 11))
    assert lib.dmoe_metadata(ctypes.byref(d), None, ctypes.byref(meta),
                             ctypes.c_void_p(0x1000), None) == -1
    assert lib.dmoe_metadata(ctypes.byref(d), ctypes.c_void_p(0x1000),
                             ctypes.byref(meta), None, None) == -1
    bad = dm._Meta(*([ctypes.c_void_p(0x1000)] * 10 + [None]))   # no schedule
    assert lib.dmoe_metadata(ctypes.byref(d), ctypes.c_void_p(0x1000),
                             ctypes.byref(bad), ctypes.c_void_p(0x1000), None) == -1
    saved = dm._Saved(*([ctypes.c_void_p(0x1000)] * 4 + [None]))
    p = ctypes.c_void_p(0x1000)
    assert lib.dmoe_forward(ctypes.byref(d), p, p, p, p, p, ctypes.byref(meta),
                            ctypes.byref(saved), p, None) == -1
    saved = dm._Saved(*([p] * 5))
    scratch = dm._Scratch(p, p, None, p)
    assert lib.dmoe_backward(ctypes.byref(d), p, p, p, p, p, ctypes.byref(meta),
                             ctypes.byref(saved), ctypes.byref(scratch), p, p, p,
                             p, p, None) == -1
    for fn in (lib.dmoe_backward_recompute, lib.dmoe_backward):
        assert fn(ctypes.byref(d), p, p, p, p, p, ctypes.byref(meta), ctypes.byref(saved),
                  ctypes.byref(scratch), p, p, p, p, p, None) == -1
    bad_saved = dm._Saved(*([p] * 4 + [None]))
    good_scratch = dm._Scratch(p, p, p, p)
    assert lib.dmoe_backward_recompute(ctypes.byref(d), p, p, p, p, p, ctypes.byref(meta),
                                       ctypes.byref(bad_saved), ctypes.byref(good_scratch),
                                       p, p, p, p, p, None) == -1
    assert lib.dmoe_padded_gather(ctypes.byref(d), None, ctypes.byref(meta), p,
                                  None) == -1
    assert lib.dmoe_padded_scatter(ctypes.byref(d), p, None, ctypes.byref(meta),
                                   None, None) == -1
    assert lib.dmoe_forward(None, p, p, p, p, p, ctypes.byref(meta),
                            ctypes.byref(saved), p, None) == -1


def test_fused_gather_checks_before_launch(lib):
    """The fused gather is bf16 only, needs x below 2 GB and, in the
    backward, the forward's x; a meta without row_token is rejected."""
    p = ctypes.c_void_p(0x1000)
    meta = dm._Meta(*([p] * 11))
    saved = dm._Saved(None, p, p, p, p)          # no x_perm: allowed here
    scratch = dm._Scratch(p, p, p, p)
    f32 = _dims()
    big = _dims(T=1 << 20, H=1024, E=8, k=1, dtype=dm.DMOE_BF16)   # T*H*2 = 2^31
    for d in (f32, big):
        assert lib.dmoe_forward_fused_gather(ctypes.byref(d), p, p, p, p, p, ctypes.byref(meta),
                                             ctypes.byref(saved), p, None) == -3
        assert lib.dmoe_backward_fused_gather(ctypes.byref(d), p, p, p, p, p, p,
                                              ctypes.byref(meta), ctypes.byref(saved),
                                              ctypes.byref(scratch), p, p, p, p, p,
                                              None) == -3
    bf = _dims(dtype=dm.DMOE_BF16)
    assert lib.dmoe_backward_fused_gather(ctypes.byref(bf), None, p, p, p, p, p,
                                          ctypes.byref(meta), ctypes.byref(saved),
                                          ctypes.byref(scratch), p, p, p, p, p, None) == -1
    no_rt = dm._Meta(*([p] * 9 + [None, p]))
    assert lib.dmoe_forward_fused_gather(ctypes.byref(bf), p, p, p, p, p, ctypes.byref(no_rt),
                                         ctypes.byref(saved), p, None) == -1
    # the plain path needs x_perm, and so does the fused backward (it
    # gathers into it)
    assert lib.dmoe_forward(ctypes.byref(bf), p, p, p, p, p, ctypes.byref(meta),
                            ctypes.byref(saved), p, None) == -1
    assert lib.dmoe_backward_fused_gather(ctypes.byref(bf), p, p, p, p, p, p,
                                          ctypes.byref(meta), ctypes.byref(saved),
                                          ctypes.byref(scratch), p, p, p, p, p, None) == -1


def test_router_checks_before_launch(lib):
    p = ctypes.c_void_p(0x1000)
    d = _dims()
    c0, c1 = ctypes.c_float(0.0), ctypes.c_float(0.001)
    fwd, bwd = lib.dmoe_router_forward, lib.dmoe_router_backward
    assert fwd(ctypes.byref(d), None, c0, p, p, None, None, None) == -1
    assert fwd(ctypes.byref(d), p, c0, None, p, None, None, None) == -1
    assert fwd(ctypes.byref(d), p, c0, p, None, None, None, None) == -1
    # a z-loss needs both z and the scalar
    assert fwd(ctypes.byref(d), p, c1, p, p, None, p, None) == -1
    assert fwd(ctypes.byref(d), p, c1, p, p, p, None, None) == -1
    assert fwd(None, p, c0, p, p, None, None, None) == -1
    for i in range(5):
        args = [p] * 5
        args[i] = None
        assert bwd(ctypes.byref(d), args[0], args[1], args[2], args[3], c0, args[4],
                   None) == -1
    for kw, code in ((dict(k=9, E=8), -1), (dict(E=257, k=2), -3), (dict(T=0), -1)):
        bad = _dims(**kw)
        assert fwd(ctypes.byref(bad), p, c0, p, p, None, None, None) == code
        assert bwd(ctypes.byref(bad), p, p, p, p, c0, p, None) == code


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, 42):
        assert len(lib.dmoe_status_string(code)) > 0


def test_binding_rejects_cpu_tensors():
    import torch
    D = dm.Dims(8, 128, 128, 2, 1, dm.DMOE_F32)
    with pytest.raises(ValueError):
        dm._ptr(torch.zeros(4), torch.float32, "x")
    assert dm.dmoe_max_tiles(D) == (8 + 127 * 2) // 128
    with pytest.raises(dm.DMoEError):
        dm.dmoe_max_tiles(dm.Dims(8, 100, 128, 2, 1, dm.DMOE_F32))


def test_fused_gather_policy(lib):
    """fused_gather="auto" fuses the gather where the padded copy of x
    (P_max rows of H bf16) would not fit the 256 MB last-level cache."""
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from workloads import CONFIGS
    want = {"tiny_f32": False, "fine_e64": False, "zipf_e64": False,
            "coarse_e8": False, "sparse_e256": True}
    for name, fused in want.items():
        c = CONFIGS[name]
        d = dm.Dims(c.T, c.H, c.F, c.E, c.k,
                    dm.DMOE_F32 if c.dtype == "f32" else dm.DMOE_BF16)
        assert dm.fused_gather_pays(d) is fused, name
    # x of 2 GB or more is beyond the fused entry points
    big = dm.Dims(1 << 19, 2048, 1024, 64, 8, dm.DMOE_BF16)
    assert dm.fused_gather_pays(big) is False


def test_moa_checks_before_launch(lib):
    """dMoA map/reduce: bf16 only, null pointers and bad dims rejected on the
    host."""
    p = ctypes.c_void_p(0x1000)
    meta = dm._Meta(*([p] * 11))
    f32 = _dims()
    bf = _dims(dtype=dm.DMOE_BF16)
    args_map = (p, p, ctypes.byref(meta), p, p, p, None)
    assert lib.dmoe_moa_map(ctypes.byref(f32), *args_map) == -3
    assert lib.dmoe_moa_map(ctypes.byref(bf), None, p, ctypes.byref(meta), p, p, p, None) == -1
    assert lib.dmoe_moa_reduce(ctypes.byref(f32), p, p, p, ctypes.byref(meta), p, p, p,
                               None) == -3
    assert lib.dmoe_moa_reduce(ctypes.byref(bf), p, None, p, ctypes.byref(meta), p, p, p,
                               None) == -1
    assert lib.dmoe_moa_reduce_backward(ctypes.byref(bf), p, p, p, ctypes.byref(meta), p, p, p,
                                        p, p, p, None, None) == -1
    assert lib.dmoe_moa_map_backward(ctypes.byref(bf), p, p, ctypes.byref(meta), p, p, p, p,
                                     None, None) == -1
    bad = _dims(F=200, dtype=dm.DMOE_BF16)
    assert lib.dmoe_moa_map(ctypes.byref(bad), *args_map) == -2
    no_sched = dm._Meta(*([p] * 10 + [None]))
    assert lib.dmoe_moa_map(ctypes.byref(bf), p, p, ctypes.byref(no_sched), p, p, p,
                            None) == -1
