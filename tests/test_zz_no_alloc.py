"""dmoe_metadata_noalloc (the metadata with its workspace in the library's
own device array) gives the same metadata as dmoe_metadata, bit for bit, on
two calls in a row, the second with a smaller input than the first."""
import ctypes

import numpy as np
import pytest
import torch

import dropless_mixture_experts_amd as dm
from workloads import CONFIGS, make_inputs, shrink

from gpu_helpers import device, dims_of, up

pytestmark = pytest.mark.gpu

FIELDS = ("tokens_per_expert", "bins", "padded_bins", "indices", "bin_ids",
          "row_of_entry", "tile_expert", "num_padded_rows", "status", "row_token")


def _poisoned_meta(D, dev):
    meta, ws = dm.allocate_meta(D, dev)
    for name in FIELDS:
        getattr(meta, name).fill_(-12345)
    meta.schedule.fill_(0xA5)
    return meta, ws


def test_noalloc_metadata_matches_workspace_call_twice():
    dev = device()
    lib = dm.load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    # the first call uses most of the array's chunks (131072 entries, E = 256);
    # the second is smaller, with empty experts, and reuses what the first left
    cases = [CONFIGS["sparse_e256"], shrink(CONFIGS["zipf_e64_empty"], T=700, H=128, F=128)]
    for cfg in cases:
        inp = make_inputs(cfg, with_weights=False, with_dy=False)
        D = dims_of(cfg)
        print(f"noalloc metadata {cfg.name} T={cfg.T} E={cfg.E} k={cfg.k}", flush=True)
        ids = up(inp.top_experts, torch.int32, dev)
        ref, ws = _poisoned_meta(D, dev)
        dm.dmoe_metadata(D, ids, ref, ws)
        got, _ = _poisoned_meta(D, dev)
        rc = lib.dmoe_metadata_noalloc(ctypes.byref(D._c()),
                                       ctypes.c_void_p(ids.data_ptr()),
                                       ctypes.byref(got._c()), stream)
        assert rc == 0, dm.dmoe_status_string(rc)
        torch.cuda.synchronize()
        assert int(ref.status.item()) == 0
        P = int(ref.num_padded_rows.item())
        for name in FIELDS:
            a, b = getattr(got, name), getattr(ref, name)
            if name == "row_token":          # rows from P on are left untouched
                a, b = a[:P], b[:P]
            assert torch.equal(a, b), name
        assert torch.equal(got.schedule, ref.schedule)


def test_noalloc_rejects_bad_arguments_before_launch():
    lib = dm.load_library()
    p = ctypes.c_void_p(0x1000)
    meta = dm._Meta(*([p] * 11))
    good = dm._Dims(512, 128, 256, 8, 2, dm.DMOE_BF16)
    bad = dm._Dims(512, 128, 256, 8, 9, dm.DMOE_BF16)          # k > E
    assert lib.dmoe_metadata_noalloc(ctypes.byref(bad), p, ctypes.byref(meta), None) == -1
    assert lib.dmoe_metadata_noalloc(ctypes.byref(good), None, ctypes.byref(meta), None) == -1
    no_sched = dm._Meta(*([p] * 10 + [None]))
    assert lib.dmoe_metadata_noalloc(ctypes.byref(good), p, ctypes.byref(no_sched), None) == -1
