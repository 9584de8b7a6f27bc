"""Blocked storage of the expert weights (moe_pack_weights and
desc.weight_layout = MOE_W_BLOCKED64) on the GPU.

The pack is a permutation of elements and must equal the blocked order
written out below element for element.  A layer run on packed weights must
match the oracle to the same tolerances as a row-major run; where both
layouts run the same kernel body in the same arithmetic order (the grouped
GEMM, the fp32 streaming kernel, the proxy weight gather) the outputs must
also equal the row-major run's bit for bit.
"""
import gc
import sys

import numpy as np
import pytest
import torch

import mixture_experts_layer_token_amd as moe
from tests.gpu_util import (check_routing, compare_out, oracle_out, oracle_routing, run_forward, sample_tokens,
                            shared_of)
from workloads import CONFIGS, make_custom_layer, make_layer, make_proxy_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe._lib.load()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _blocked_order(w: torch.Tensor) -> torch.Tensor:
    """The blocked order of a row-major [G, N, K] (or [N, K]) tensor, on the
    CPU: 64-row x 128-byte blocks, blocks of a matrix in (row block, column
    block) order, rows of a block one after another."""
    eb = 128 // w.element_size()
    G, N, K = (1, *w.shape) if w.dim() == 2 else tuple(w.shape)
    v = w.reshape(G, N // 64, 64, K // eb, eb).permute(0, 1, 3, 2, 4)
    return v.contiguous().reshape(-1)


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(3, 192, 256), (1, 64, 128), (2, 128, 2176), (320, 384)])
def test_pack_weights_is_the_blocked_order(dtype, shape):
    g = torch.Generator().manual_seed(sum(shape))
    w = torch.randn(shape, generator=g).to(dtype)
    got = moe.pack_weights(w.cuda())
    torch.cuda.synchronize()
    assert got.shape == w.shape
    assert torch.equal(_bits(got.cpu().reshape(-1)), _bits(_blocked_order(w)))


def test_pack_weights_empty_stack():
    w = torch.empty((0, 64, 128), dtype=torch.bfloat16, device="cuda")
    assert moe.pack_weights(w).shape == w.shape


def _forward_blocked(layer, path):
    pk = moe.pack_weights
    sh = shared_of(layer)
    out, stats, status = moe.forward(layer.x, layer.w_router, layer.router_bias, layer.k, pk(layer.w_gate),
                                     pk(layer.w_up), pk(layer.w_down), tuple(pk(t) for t in sh) if sh else None,
                                     k_max=layer.cfg.k_max, routed_scale=layer.cfg.routed_scale, path=path,
                                     weight_layout="blocked")
    torch.cuda.synchronize()
    return out, stats.cpu().numpy().astype(np.int64), int(status.item())


def _same_body(layer, path):
    """Whether both layouts run the same kernel body (same arithmetic order)."""
    if layer.x.dtype == torch.float32:
        return True
    desc = moe.make_desc(layer.x.shape[0], layer.x.shape[1], *layer.w_gate.shape[:2], layer.cfg.k_max,
                         I_shared=0 if layer.ws_gate is None else layer.ws_gate.shape[0], path=path)
    routed, shared = moe.resolve_path(desc)
    return routed == "gemm" and (layer.ws_gate is None or shared == "gemm")


SAMPLE = {"tiny_fp32": 16, "mixtral_decode": 32, "qwen3_30b_a3b_decode": 32, "subexpert_prefill": 12,
          "dsv3_decode": 6}


@pytest.mark.parametrize("name,path", [("tiny_fp32", "auto"), ("mixtral_decode", "auto"),
                                       ("qwen3_30b_a3b_decode", "auto"), ("qwen3_30b_a3b_decode", "gemm"),
                                       ("subexpert_prefill", "auto"), ("subexpert_prefill", "stream"),
                                       ("dsv3_decode", "auto")])
def test_blocked_workload_matches_oracle(name, path):
    cfg = CONFIGS[name]
    _say(f"[layout] {name} {path}: drawing layer")
    layer = make_layer(cfg, "cuda")
    out, stats, status = _forward_blocked(layer, path)
    assert status == 0
    _, p = oracle_routing(layer)
    np.testing.assert_array_equal(stats[:cfg.E], p["counts"])
    tokens = sample_tokens(cfg.T, SAMPLE[name])
    err = compare_out(out, oracle_out(layer, tokens), cfg.dtype, tokens)
    if _same_body(layer, path):
        ref, _, _ = run_forward(layer, path=path)
        assert torch.equal(_bits(out), _bits(ref))
    _say(f"[layout] {name} {path}: {err}")


# the grouped GEMM is a bf16 kernel (the ABI rejects fp32 on it), so fp32 runs
# the streaming path only
@pytest.mark.parametrize("dtype,path", [("bf16", "stream"), ("bf16", "gemm"), ("f32", "stream")])
@pytest.mark.parametrize("T,E,d,I,kmax,Is", [
    (700, 16, 256, 384, 8, 256),     # ragged row blocks, shared expert
    (40, 32, 384, 128, 4, 0),        # few rows per expert
    (520, 8, 256, 256, 4, 256),      # shared expert fused into the GEMM launches
    (48, 4, 2176, 2176, 2, 2176),    # K % 256 = 128 (2 x 2 stream waves), long K
    (300, 8, 128, 128, 8, 0),        # smallest d and I
    (64, 8, 256, 2048, 2, 0),        # down K = 2048: the deeper-ring streaming body
])
def test_blocked_shapes_match_oracle(dtype, path, T, E, d, I, kmax, Is):
    rng = np.random.default_rng(T * E + 1)
    k = rng.integers(1, kmax + 1, size=T)
    layer = make_custom_layer(T=T, d=d, E=E, I=I, k=k, dtype=dtype, k_max=kmax, I_shared=Is, zipf=1.0,
                              seed=E + 5, device="cuda")
    out, stats, status = _forward_blocked(layer, path)
    assert status == 0
    r, p = oracle_routing(layer)
    np.testing.assert_array_equal(stats[:E], p["counts"])
    tokens = sample_tokens(T, 40)
    err = compare_out(out, oracle_out(layer, tokens), dtype, tokens)
    if _same_body(layer, path):
        ref, _, _ = run_forward(layer, path=path)
        assert torch.equal(_bits(out), _bits(ref))
    _say(f"[layout] {dtype} {path} T={T} E={E} d={d} I={I}: {err}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_blocked_proxy_pack_is_packed_row_major(dtype):
    cfg = CONFIGS["subexpert_prefill"].with_(name=f"split_{dtype}", dtype=dtype, T=64, d=256, E=64, I=128,
                                             k_values=(4, 8), k_probs=(0.5, 0.5), k_max=8, split=4, seed=11)
    layer = make_layer(cfg, "cuda")
    N, r = 4, 24
    _, gate_idx = make_proxy_inputs(cfg, r, "cuda")
    wp_g, wp_u = moe.proxy_pack(layer.w_gate, layer.w_up, gate_idx, N)
    bp_g, bp_u = moe.proxy_pack(moe.pack_weights(layer.w_gate), moe.pack_weights(layer.w_up), gate_idx, N,
                                weight_layout="blocked")
    torch.cuda.synchronize()
    assert torch.equal(_bits(bp_g), _bits(moe.pack_weights(wp_g)))
    assert torch.equal(_bits(bp_u), _bits(moe.pack_weights(wp_u)))
