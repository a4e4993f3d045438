"""Shared plumbing for the GPU parity tests: upload seeded inputs, run the
layer through the C ABI, compare with the oracle."""
import numpy as np
import pytest
import torch

import dropless_mixture_experts_amd as dm

# Tolerances on max|gpu - ref| relative to max|ref|, per output tensor.
TOL = {"bf16": 2e-2, "f32": 1e-5}


def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU test needs an MI355X: torch.cuda.is_available() is False")
    return torch.device("cuda:0")


def torch_dtype(cfg):
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def dims_of(cfg):
    return dm.Dims(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k,
                   dm.DMOE_F32 if cfg.dtype == "f32" else dm.DMOE_BF16)


def schedule_tables(meta, max_tiles):
    """The tables the library keeps in the opaque meta.schedule buffer, in
    its private layout (int32: pair_first[max_tiles], then num_pairs); for
    tests of that schedule only."""
    s = meta.schedule.view(torch.int32).cpu().numpy().astype(np.int64)
    return dict(pair_first=s[:max_tiles], num_pairs=int(s[max_tiles]))


def up(a, dt, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)


def down(t):
    return t.float().cpu().numpy().astype(np.float64)


def assert_close(got, ref, tol, name):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    assert err <= tol * scale, f"{name}: max err {err:.3e} > {tol} * {scale:.3e}"
    return err, scale


class Run:
    """Uploads one workload and runs metadata + forward + backward."""

    def __init__(self, inp, dev=None, lean=False, backward=True, fused_gather=False):
        self.inp = inp
        self.cfg = inp.cfg
        self.dev = dev or device()
        dt = torch_dtype(self.cfg)
        self.D = dims_of(self.cfg)
        self.x = up(inp.x, dt, self.dev)
        self.ids = up(inp.top_experts, torch.int32, self.dev)
        self.w = up(inp.weights, torch.float32, self.dev)
        self.w1 = up(inp.w1, dt, self.dev)
        self.w3 = up(inp.w3, dt, self.dev)
        self.w2 = up(inp.w2, dt, self.dev)
        self.dy = up(inp.dy, dt, self.dev) if backward else None
        self.layer = dm.DMoELayer(self.D, self.dev, lean=lean, fused_gather=fused_gather)
        self.y = self.layer.forward(self.x, self.ids, self.w, self.w1, self.w3, self.w2)
        self.g = (self.layer.backward(self.dy, self.w, self.w1, self.w3, self.w2)
                  if backward else None)
        torch.cuda.synchronize()
        self.meta = self.layer.buf.meta
        self.saved = self.layer.buf.saved
        self.scratch = self.layer.buf.scratch
        self.P = int(self.meta.num_padded_rows.item())
        assert int(self.meta.status.item()) == 0

    def meta_np(self):
        m = self.meta
        return {k: getattr(m, k).cpu().numpy().astype(np.int64) for k in (
            "tokens_per_expert", "bins", "padded_bins", "indices", "bin_ids",
            "row_of_entry", "tile_expert")}
