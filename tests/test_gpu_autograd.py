"""dmoe_autograd: the layer as a torch.autograd.Function.  Its outputs and
gradients must be the layer's own (DMoELayer through the C ABI), bit for
bit, and within tolerance of the fp64 oracle."""
import numpy as np
import pytest
import torch

import dropless_mixture_experts_amd as dm
import oracle
from workloads import CONFIGS, make_inputs, shrink

from gpu_helpers import TOL, Run, assert_close, down, torch_dtype, up

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [
    shrink(CONFIGS["fine_e64"], T=300, H=256, F=256, E=8),
    shrink(CONFIGS["tiny_f32"], T=129, H=128, F=256, E=4, k=2),
], ids=lambda c: c.name)
def test_autograd_matches_layer_and_oracle(cfg):
    inp = make_inputs(cfg)
    print(f"autograd {cfg.name}", flush=True)
    ref = Run(inp)
    dev, dt = ref.dev, torch_dtype(cfg)
    x = up(inp.x, dt, dev).requires_grad_()
    w = up(inp.weights, torch.float32, dev).requires_grad_()
    w1 = up(inp.w1, dt, dev).requires_grad_()
    w3 = up(inp.w3, dt, dev).requires_grad_()
    w2 = up(inp.w2, dt, dev).requires_grad_()
    ids = up(inp.top_experts, torch.int32, dev)
    y = dm.dmoe_autograd(x, ids, w, w1, w3, w2)
    y.backward(up(inp.dy, dt, dev))
    torch.cuda.synchronize()
    assert torch.equal(y.detach(), ref.y)
    for t, key in ((x, "dx"), (w, "d_weights"), (w1, "dw1"), (w3, "dw3"), (w2, "dw2")):
        assert t.grad is not None, key
        assert torch.equal(t.grad, ref.g[key]), key
    ref_y, sv = oracle.forward_padded(inp.x, inp.top_experts, inp.weights,
                                      inp.w1, inp.w3, inp.w2)
    ref_g = oracle.backward_padded(inp.x, inp.top_experts, inp.weights, inp.w1,
                                   inp.w3, inp.w2, inp.dy, sv)
    tol = TOL[cfg.dtype]
    assert_close(down(y.detach()), ref_y, tol, "y")
    assert_close(down(x.grad), ref_g["dx"], tol, "dx")
    assert_close(down(w.grad), ref_g["d_weights"], tol, "d_weights")
