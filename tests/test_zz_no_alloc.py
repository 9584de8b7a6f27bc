"""moe_forward_noalloc (the library-held scratch array) against moe_forward
(the caller's workspace): same kernels, so the outputs, per-expert counts and
device status must be identical bit for bit.  Two calls in a row on one GPU,
the second over a smaller batch of the same layer shape, then a third in
another element type; each is checked against moe_forward on the same inputs."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_token_amd as moe
from workloads import CONFIGS, make_layer

pytestmark = pytest.mark.gpu


def _run_both(layer, T=None):
    c = layer.cfg
    x, k = layer.x, layer.k
    if T is not None:
        x, k = x[:T].contiguous(), k[:T].contiguous()
    Tn = x.shape[0]
    E, I, d = layer.w_gate.shape
    Is = layer.ws_gate.shape[0] if layer.ws_gate is not None else 0
    desc = moe.make_desc(Tn, d, E, I, c.k_max, I_shared=Is, dtype=x.dtype, routed_scale=c.routed_scale)
    sh = (layer.ws_gate, layer.ws_up, layer.ws_down) if Is else (None, None, None)
    dev = x.device
    outs = []
    for noalloc in (True, False):
        out = torch.full((Tn, d), float("nan"), dtype=x.dtype, device=dev)
        stats = torch.full((E + 2,), -7, dtype=torch.int32, device=dev)
        status = torch.full((1,), -7, dtype=torch.int32, device=dev)
        if noalloc:
            moe.moe_forward_noalloc(desc, x, layer.w_router, layer.router_bias, k, layer.w_gate, layer.w_up,
                                    layer.w_down, *sh, out, stats, status)
        else:
            ws = moe.alloc_workspace(desc, moe.MOE_OP_FORWARD, dev)
            moe.moe_forward(desc, x, layer.w_router, layer.router_bias, k, layer.w_gate, layer.w_up,
                            layer.w_down, *sh, out, stats, status, ws)
        torch.cuda.synchronize()
        outs.append((out.view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32).cpu().numpy(),
                     stats.cpu().numpy(), int(status.item())))
    (o1, s1, st1), (o2, s2, st2) = outs
    assert st1 == st2 == 0
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(o1, o2)
    return s1


def test_noalloc_matches_forward_twice_then_smaller():
    dev = torch.device("cuda:0")
    layer = make_layer(CONFIGS["qwen3_30b_a3b_decode"], dev)
    s_big = _run_both(layer)
    s_small = _run_both(layer, T=100)
    assert s_big[-1] > s_small[-1] > 0   # A of the second call is smaller
    tiny = make_layer(CONFIGS["tiny_fp32"], dev)
    _run_both(tiny)
    _run_both(layer, T=7)
