"""Compositional paths on the GPU (PCoMoE, arXiv 2609.01024) against the oracle.

Path routing takes its integer decisions on float32 scores computed the same
way on both sides from the routing contract's logits, so the selected paths,
their order and the source groups must match bit for bit; the weights to
float32 rounding; outputs to the layer's tolerance.  The diagonal-only list
must reproduce the vanilla layer (moe_route / moe_forward) bit for bit.
"""
import gc
import sys

import numpy as np
import pytest
import torch

import mixture_experts_layer_token_amd as moe
import oracle
from tests.gpu_util import compare_out, sample_tokens
from workloads import CONFIGS, ExpertView, make_custom_layer, make_layer, make_path_mask, make_target_router, to_f64

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


def _run(layer, k_max, src, tgt, bias, w_tgt, lam, path="auto", router="auto"):
    T, d = layer.x.shape
    E, I, _ = layer.w_gate.shape
    Is = layer.ws_gate.shape[0] if layer.ws_gate is not None else 0
    desc = moe.make_desc(T, d, E, I, k_max, I_shared=Is, dtype=layer.x.dtype, routed_scale=layer.cfg.routed_scale,
                         path=path, router=router)
    table = moe.moe_path_table(E, src, tgt, bias)
    pl = moe.PathLayer(desc, table, len(src), lam, layer.device)
    out = torch.empty((T, d), dtype=layer.x.dtype, device=layer.device)
    sh = (layer.ws_gate, layer.ws_up, layer.ws_down) if Is else None
    pl.run(layer.x, layer.w_router, layer.router_bias, w_tgt, layer.k, layer.w_gate, layer.w_up, layer.w_down, out,
           shared=sh)
    torch.cuda.synchronize()
    return pl, out


def _host(pl):
    A = int(pl.tok_off[-1].item())
    S = int(pl.src_off[-1].item())
    c = lambda t, n=None: to_f64(t if n is None else t[:n])
    return dict(tok_off=c(pl.tok_off), src=c(pl.src, A), tgt=c(pl.tgt, A), w=pl.w[:A].cpu().double().numpy(),
                status=int(pl.status.item()), src_off=c(pl.src_off), src_ids=c(pl.src_ids, S), p2s=c(pl.p2s, A), A=A)


@pytest.mark.parametrize("dtype,T,E,k_max,path", [("f32", 130, 8, 2, "auto"), ("bf16", 300, 8, 3, "auto"),
                                                  ("bf16", 700, 16, 4, "gemm"), ("bf16", 64, 32, 6, "stream")])
def test_diagonal_paths_reproduce_the_layer(dtype, T, E, k_max, path):
    """Diagonal paths with zero biases: routes = moe_route's, output =
    moe_forward's, bit for bit (with and without a target prior at lambda 0)."""
    rng = np.random.default_rng(T)
    k = rng.integers(0, k_max + 1, size=T)
    layer = make_custom_layer(T, 256, E, 256, k, dtype=dtype, k_max=k_max, seed=5, device="cuda")
    diag = np.arange(E, dtype=np.int32)
    want, stats, status = moe.forward(layer.x, layer.w_router, layer.router_bias, layer.k, layer.w_gate,
                                      layer.w_up, layer.w_down, k_max=k_max, path=path)
    torch.cuda.synchronize()
    r = oracle.route(to_f64(layer.x), to_f64(layer.w_router), None, to_f64(layer.k), k_max)
    for w_tgt in (None, make_target_router(layer.cfg, "cuda")):
        pl, out = _run(layer, k_max, diag, diag, np.zeros(E, np.float32), w_tgt, 0.0, path)
        g = _host(pl)
        np.testing.assert_array_equal(g["tok_off"], r["tok_off"])
        np.testing.assert_array_equal(g["src"], r["ids"])
        np.testing.assert_array_equal(g["tgt"], r["ids"])
        assert torch.equal(out, want), "diagonal paths differ from moe_forward"
    _say(f"[path] diagonal {dtype} T={T} E={E} k_max={k_max}: bit-exact with moe_forward")


@pytest.mark.parametrize("dtype,T,E,k_max,extra,lam", [("f32", 200, 8, 4, 3, 0.375), ("bf16", 300, 8, 2, 2, 0.5),
                                                       ("bf16", 513, 16, 6, 5, -0.25), ("f32", 77, 32, 8, 1, 1.0)])
def test_paths_match_oracle(dtype, T, E, k_max, extra, lam):
    rng = np.random.default_rng(E + T)
    k = rng.integers(0, k_max + 1, size=T)
    k[3], k[5] = k_max + 2, -1            # invalid budgets: flagged, nothing runs
    layer = make_custom_layer(T, 256, E, 128, k, dtype=dtype, k_max=k_max, seed=9, device="cuda")
    w_tgt = make_target_router(layer.cfg, "cuda")
    src, tgt, bias = make_path_mask(E, extra, seed=E)
    pl, out = _run(layer, k_max, src, tgt, bias, w_tgt, lam)
    g = _host(pl)
    ref = oracle.path_route(to_f64(layer.x), to_f64(layer.w_router), None, to_f64(w_tgt), np.float32(lam), src, tgt,
                            bias.astype(np.float64), to_f64(layer.k), k_max)
    assert g["status"] == ref["status"] == 1
    np.testing.assert_array_equal(g["tok_off"], ref["tok_off"])
    np.testing.assert_array_equal(g["src"], ref["src"])
    np.testing.assert_array_equal(g["tgt"], ref["tgt"])
    np.testing.assert_allclose(g["w"], ref["w"], rtol=2e-6, atol=2e-7)
    s_off, s_ids, p2s = oracle.path_sources(ref["tok_off"], ref["src"])
    np.testing.assert_array_equal(g["src_off"], s_off)
    np.testing.assert_array_equal(g["src_ids"], s_ids)
    np.testing.assert_array_equal(g["p2s"], p2s)
    assert s_off[-1] < ref["tok_off"][-1] or extra == 0    # some expansions are shared
    tokens = np.arange(T)
    want = oracle.path_forward(to_f64(layer.x), ref["tok_off"], ref["src"], ref["tgt"], ref["w"],
                               ExpertView(layer.w_gate), ExpertView(layer.w_up), ExpertView(layer.w_down))
    err = compare_out(out, want, dtype, tokens)
    assert not out[3].any() and not out[5].any()
    _say(f"[path] {dtype} T={T} E={E} paths={len(src)} routes={g['A']} expansions={int(s_off[-1])}: {err}")


def test_paths_graph_replay():
    """The whole path layer replays in a HIP graph with identical results."""
    T, E, k_max = 96, 8, 2
    rng = np.random.default_rng(4)
    layer = make_custom_layer(T, 256, E, 256, rng.integers(0, k_max + 1, size=T), dtype="bf16", k_max=k_max,
                              seed=2, device="cuda")
    w_tgt = make_target_router(layer.cfg, "cuda")
    src, tgt, bias = make_path_mask(E, 2, seed=1)
    pl, out = _run(layer, k_max, src, tgt, bias, w_tgt, 0.5)
    first = out.clone()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        pl.run(layer.x, layer.w_router, None, w_tgt, layer.k, layer.w_gate, layer.w_up, layer.w_down, out)
    for _ in range(3):
        out.fill_(7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, first)


def test_paths_mixtral_decode_full_size():
    """Mixtral-8x7B-shaped decode layer (64 tokens, top-2 paths over a mask of
    the 8 diagonal and 2 off-diagonal paths per source): every route, and
    every output row."""
    cfg = CONFIGS["mixtral_decode"]
    layer = make_layer(cfg, "cuda")
    w_tgt = make_target_router(cfg, "cuda")
    src, tgt, bias = make_path_mask(cfg.E, 2, seed=3)
    pl, out = _run(layer, cfg.k_max, src, tgt, bias, w_tgt, 0.5)
    g = _host(pl)
    ref = oracle.path_route(to_f64(layer.x), to_f64(layer.w_router), None, to_f64(w_tgt), np.float32(0.5), src, tgt,
                            bias.astype(np.float64), to_f64(layer.k), cfg.k_max)
    np.testing.assert_array_equal(g["src"], ref["src"])
    np.testing.assert_array_equal(g["tgt"], ref["tgt"])
    tokens = sample_tokens(cfg.T, 64)
    want = oracle.path_forward(to_f64(layer.x), ref["tok_off"], ref["src"], ref["tgt"], ref["w"],
                               ExpertView(layer.w_gate), ExpertView(layer.w_up), ExpertView(layer.w_down),
                               tokens=tokens)
    err = compare_out(out, want, cfg.dtype, tokens)
    _say(f"[path] mixtral_decode: routes {g['A']}, expansions {int(pl.src_off[-1].item())}, {err}")


@pytest.mark.parametrize("T,E,k_max,extra", [(0, 8, 2, 1), (1, 8, 8, 7), (257, 1024, 64, 0), (300, 64, 64, 15)])
def test_paths_edges(T, E, k_max, extra):
    """Empty batch, a single token over every pair of 8 experts, the largest
    list (1,024 paths over 1,024 experts) with k_max = 64, and 64 paths per
    token over a 16-wide list per source."""
    rng = np.random.default_rng(T + E)
    k = rng.integers(0, k_max + 1, size=T)
    if T:
        k[0] = k_max
    layer = make_custom_layer(T, 128, E, 128, k, dtype="f32", k_max=k_max, seed=13, device="cuda")
    w_tgt = make_target_router(layer.cfg, "cuda")
    src, tgt, bias = make_path_mask(E, extra, seed=7)
    pl, out = _run(layer, k_max, src, tgt, bias, w_tgt, 0.625)
    g = _host(pl)
    ref = oracle.path_route(to_f64(layer.x), to_f64(layer.w_router), None, to_f64(w_tgt), np.float32(0.625), src,
                            tgt, bias.astype(np.float64), to_f64(layer.k), k_max)
    np.testing.assert_array_equal(g["tok_off"], ref["tok_off"])
    np.testing.assert_array_equal(g["src"], ref["src"])
    np.testing.assert_array_equal(g["tgt"], ref["tgt"])
    np.testing.assert_allclose(g["w"], ref["w"], rtol=2e-6, atol=2e-7)
    s_off, s_ids, p2s = oracle.path_sources(ref["tok_off"], ref["src"])
    np.testing.assert_array_equal(g["src_off"], s_off)
    np.testing.assert_array_equal(g["src_ids"], s_ids)
    np.testing.assert_array_equal(g["p2s"], p2s)
    if T:
        tokens = sample_tokens(T, 24)
        want = oracle.path_forward(to_f64(layer.x), ref["tok_off"], ref["src"], ref["tgt"], ref["w"],
                                   ExpertView(layer.w_gate), ExpertView(layer.w_up), ExpertView(layer.w_down),
                                   tokens=tokens)
        compare_out(out, want, "f32", tokens)
    _say(f"[path] edge T={T} E={E} k_max={k_max} P={len(src)}: routes {g['A']}")


@pytest.mark.parametrize("T,E,d,k_max,extra,lam,tgt,bias", [(700, 8, 256, 2, 2, 0.5, True, False),
                                                            (513, 64, 512, 8, 3, -0.75, True, True),
                                                            (300, 256, 2304, 16, 2, 0.5, True, False),
                                                            (257, 256, 256, 32, 3, 0.0, False, True),
                                                            (96, 32, 128, 6, 31, 1.5, True, False)])
def test_screened_path_router_bit_exact(T, E, d, k_max, extra, lam, tgt, bias):
    """The screened path selection (MFMA bounds, exact logits for the
    candidates' sources and targets) gives the float64 path router's routes
    and weights bit for bit, and the oracle's routes (with a router bias, a
    negative lambda, no target prior, every pair active, d past one pass)."""
    rng = np.random.default_rng(T * E)
    k = rng.integers(0, k_max + 1, size=T)
    k[0] = k_max
    layer = make_custom_layer(T, d, E, 128, k, dtype="bf16", k_max=k_max, zipf=1.1 if bias else 0.0, seed=E,
                              device="cuda")
    w_tgt = make_target_router(layer.cfg, "cuda") if tgt else None
    src, tgt_ids, pbias = make_path_mask(E, extra, seed=E + 1)
    outs = {}
    for router in ("float64", "screened"):
        pl, out = _run(layer, k_max, src, tgt_ids, pbias, w_tgt, lam, router=router)
        outs[router] = (_host(pl), out, pl.w[:int(pl.tok_off[-1].item())].clone())
    a, b = outs["float64"][0], outs["screened"][0]
    for key in ("tok_off", "src", "tgt", "src_off", "src_ids", "p2s"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    assert torch.equal(outs["float64"][2], outs["screened"][2]), "weights differ"
    assert torch.equal(outs["float64"][1], outs["screened"][1]), "outputs differ"
    ref = oracle.path_route(to_f64(layer.x), to_f64(layer.w_router), to_f64(layer.router_bias),
                            None if w_tgt is None else to_f64(w_tgt), np.float32(lam), src, tgt_ids,
                            pbias.astype(np.float64), to_f64(layer.k), k_max)
    np.testing.assert_array_equal(b["src"], ref["src"])
    np.testing.assert_array_equal(b["tgt"], ref["tgt"])
    np.testing.assert_allclose(b["w"], ref["w"], rtol=2e-6, atol=2e-7)
    _say(f"[path] screened T={T} E={E} d={d} P={len(src)}: routes {b['A']} bit-exact")


def test_screened_path_router_full_size():
    """Sub-expert prefill batch (8,192 tokens, 256 experts, k <= 32, 768
    paths): the auto-selected screened path router equals the float64 one on
    every token."""
    cfg = CONFIGS["subexpert_prefill"]
    layer = make_layer(cfg, "cuda")
    w_tgt = make_target_router(cfg, "cuda")
    src, tgt, bias = make_path_mask(cfg.E, 2, seed=0)
    res = {}
    for router in ("float64", "auto"):
        pl, out = _run(layer, cfg.k_max, src, tgt, bias, w_tgt, 0.5, router=router)
        res[router] = (_host(pl), pl.w[:int(pl.tok_off[-1].item())].clone(), out)
        del pl
    a, b = res["float64"][0], res["auto"][0]
    for key in ("tok_off", "src", "tgt", "src_off", "src_ids", "p2s"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    assert torch.equal(res["float64"][1], res["auto"][1])
    assert torch.equal(res["float64"][2], res["auto"][2])
    tokens = sample_tokens(cfg.T, 24)
    ref = oracle.path_route(to_f64(layer.x)[tokens], to_f64(layer.w_router), None, to_f64(w_tgt), np.float32(0.5),
                            src, tgt, bias.astype(np.float64), to_f64(layer.k)[tokens], cfg.k_max)
    for i, t in enumerate(tokens):
        lo, hi = b["tok_off"][t], b["tok_off"][t + 1]
        r0, r1 = ref["tok_off"][i], ref["tok_off"][i + 1]
        np.testing.assert_array_equal(b["src"][lo:hi], ref["src"][r0:r1])
        np.testing.assert_array_equal(b["tgt"][lo:hi], ref["tgt"][r0:r1])
    _say(f"[path] screened full size: routes {b['A']} bit-exact with the float64 path router")


@pytest.mark.parametrize("T,Is,I", [(300, 256, 256), (90, 128, 256), (600, 256, 256)])
def test_paths_with_shared_expert(T, Is, I):
    """A layer with an always-on shared expert: the diagonal-only list
    reproduces moe_forward bit for bit (the shared expert fused into the
    routed GEMM launches when it is as wide as a routed expert, separate
    otherwise), and a general list matches the oracle."""
    E, k_max = 16, 4
    rng = np.random.default_rng(T + Is)
    k = rng.integers(0, k_max + 1, size=T)
    layer = make_custom_layer(T, 256, E, I, k, dtype="bf16", k_max=k_max, I_shared=Is, seed=17, device="cuda")
    diag = np.arange(E, dtype=np.int32)
    want, _, _ = moe.forward(layer.x, layer.w_router, layer.router_bias, layer.k, layer.w_gate, layer.w_up,
                             layer.w_down, (layer.ws_gate, layer.ws_up, layer.ws_down), k_max=k_max)
    pl, out = _run(layer, k_max, diag, diag, np.zeros(E, np.float32), None, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(out, want), "diagonal paths with a shared expert differ from moe_forward"
    w_tgt = make_target_router(layer.cfg, "cuda")
    src, tgt, bias = make_path_mask(E, 3, seed=2)
    pl, out = _run(layer, k_max, src, tgt, bias, w_tgt, 0.5)
    ref = oracle.path_route(to_f64(layer.x), to_f64(layer.w_router), None, to_f64(w_tgt), np.float32(0.5), src, tgt,
                            bias.astype(np.float64), to_f64(layer.k), k_max)
    tokens = sample_tokens(T, 40)
    want = oracle.path_forward(to_f64(layer.x), ref["tok_off"], ref["src"], ref["tgt"], ref["w"],
                               ExpertView(layer.w_gate), ExpertView(layer.w_up), ExpertView(layer.w_down),
                               tokens=tokens, shared=(to_f64(layer.ws_gate), to_f64(layer.ws_up),
                                                      to_f64(layer.ws_down)))
    err = compare_out(out, want, "bf16", tokens)
    _say(f"[path] shared expert T={T} I_shared={Is}: {err}")
