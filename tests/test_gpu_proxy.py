"""Proxy gating of a split layer on the GPU (MoE-Prism, arXiv 2510.19366,
§III-B2, Training-Free Proxy Gating) against the oracle.

Both sides score under one precision contract (each gate neuron's
pre-activations exact in float64 and rounded once to float32, activations and
their mean in float64), so the routes are compared bit for bit: whole-expert
routes, route offsets, every chosen sub-expert in its order, and each route's
weight.  Layer outputs are then compared on every sampled token with the
oracle's forward on those (identical) routes.
"""
import gc
import sys

import numpy as np
import pytest
import torch

import mixture_experts_layer_token_amd as moe
import oracle
from tests.gpu_util import compare_out, desc_of, sample_tokens
from workloads import CONFIGS, ExpertView, make_layer, make_proxy_inputs, to_f64

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


def _small_cfg(dtype, T=300, d=256, E=64, I=128, N=4, k_max=16, seed=3):
    ks = tuple(range(0, k_max + 1, max(1, k_max // 4)))
    return CONFIGS["subexpert_prefill"].with_(name=f"split_{dtype}_T{T}_E{E}_N{N}", dtype=dtype, T=T, d=d, E=E,
                                              I=I, k_values=ks, k_probs=(1.0 / len(ks),) * len(ks),
                                              k_max=k_max, split=N, seed=seed)


def _gpu_proxy(layer, N, r, m, kappa, w_base, gate_idx):
    desc = desc_of(layer)
    wp_g, wp_u = moe.proxy_pack(layer.w_gate, layer.w_up, gate_idx, N)
    pr = moe.ProxyRouter(desc, N, r, m, kappa, layer.device)
    pr.run(layer.x, w_base, layer.router_bias, layer.k, wp_g, wp_u)
    torch.cuda.synchronize()
    return desc, pr, wp_g, wp_u


def _layer_on_routes(layer, desc, tok_off, ids, w):
    """moe_permute -> moe_ffn -> moe_combine of the split layer on given routes."""
    dev = layer.device
    T, d, E, km = desc.T, desc.d, desc.E, desc.k_max
    i32 = dict(dtype=torch.int32, device=dev)
    counts = torch.empty(E, **i32)
    eoff = torch.empty(E + 1, **i32)
    ptok = torch.empty(max(T * km, 1), **i32)
    psrc = torch.empty_like(ptok)
    inv = torch.empty_like(ptok)
    nact = torch.empty(1, **i32)
    moe.moe_permute(desc, tok_off, ids, counts, eoff, ptok, psrc, inv, nact,
                    moe.alloc_workspace(desc, moe.MOE_OP_PERMUTE, dev))
    y = torch.empty((max(T * km, 1), d), dtype=layer.x.dtype, device=dev)
    moe.moe_ffn(desc, layer.x, layer.w_gate, layer.w_up, layer.w_down, None, None, None, eoff, ptok, y, None,
                moe.alloc_workspace(desc, moe.MOE_OP_FFN, dev))
    out = torch.empty((T, d), dtype=layer.x.dtype, device=dev)
    moe.moe_combine(desc, y, None, tok_off, w, inv, out)
    torch.cuda.synchronize()
    return out


def _selected_rows(w, gate_idx):
    """Rows gate_idx[sub] of every sub-expert, float64 [E][r][d] (plain
    indexing, so that the oracle's scores read r rows instead of I)."""
    E, r = gate_idx.shape
    idx = gate_idx.long().clamp(0, w.shape[1] - 1)
    rows = torch.gather(w, 1, idx[:, :, None].expand(E, r, w.shape[2]))
    return to_f64(rows)


def _check_selection(got_to, got_ids, got_w, ref, tokens):
    """Row i of the oracle's result `ref` is GPU token tokens[i]: the same
    routes (sub-expert ids in the same order) and the same weights.  Returns
    the number of routes compared."""
    n = 0
    for i, t in enumerate(tokens):
        g0, g1 = int(got_to[t]), int(got_to[t + 1])
        r0, r1 = int(ref["tok_off"][i]), int(ref["tok_off"][i + 1])
        assert g1 - g0 == r1 - r0, (t, g1 - g0, r1 - r0)
        np.testing.assert_array_equal(got_ids[g0:g1], ref["ids"][r0:r1], err_msg=f"token {t}")
        np.testing.assert_allclose(got_w[g0:g1], ref["w"][r0:r1], rtol=2e-6, atol=2e-7, err_msg=f"token {t}")
        n += g1 - g0
    return n


@pytest.mark.parametrize("dtype,N,r,m,E", [("f32", 4, 4, 4, 64), ("bf16", 4, 4, 4, 64), ("bf16", 4, 48, 4, 64),
                                          ("bf16", 8, 16, 2, 64), ("f32", 2, 64, 8, 32)])
def test_proxy_routes_and_layer(dtype, N, r, m, E):
    k_max = m * N
    cfg = _small_cfg(dtype, E=E, N=N, k_max=k_max)
    layer = make_layer(cfg, "cuda")
    # a few out-of-range budgets: flagged, and those tokens run nothing
    layer.k[7] = k_max + 1
    layer.k[11] = -1
    w_base, gate_idx = make_proxy_inputs(cfg, r, "cuda")
    kappa = moe.moe_proxy_kappa_balanced(k_max, m, N)
    desc, pr, wp_g, wp_u = _gpu_proxy(layer, N, r, m, kappa, w_base, gate_idx)

    # packed weights: a plain gather of the gate-neuron rows, zero padded
    Ip = moe.proxy_width(N, r)
    g_rows = layer.w_gate.gather(1, gate_idx.long()[:, :, None].expand(E, r, cfg.d))
    want = torch.zeros((E // N, Ip, cfg.d), dtype=layer.x.dtype, device="cuda")
    want[:, :N * r] = g_rows.reshape(E // N, N * r, cfg.d)
    assert torch.equal(wp_g, want)

    ref = oracle.proxy_route(to_f64(layer.x), to_f64(w_base), to_f64(layer.router_bias), to_f64(layer.k), k_max,
                             m, N, kappa.tolist(), to_f64(gate_idx), to_f64(layer.w_gate), to_f64(layer.w_up),
                             cfg.routed_scale)
    base = ref["base"]
    np.testing.assert_array_equal(to_f64(pr.b_tok_off), base["tok_off"])
    np.testing.assert_array_equal(to_f64(pr.b_ids)[:cfg.T * m], base["ids"])
    assert int(pr.status.item()) == ref["status"] == 1
    got_to = to_f64(pr.tok_off)
    np.testing.assert_array_equal(got_to, ref["tok_off"])
    A = int(got_to[-1])
    got_ids = to_f64(pr.ids)[:A]
    got_w = pr.w[:A].cpu().double().numpy()
    routes = _check_selection(got_to, got_ids, got_w, ref, range(cfg.T))
    assert routes == A
    out = _layer_on_routes(layer, desc, pr.tok_off, pr.ids, pr.w)
    tokens = np.asarray(list(sample_tokens(cfg.T, 40)) + [7, 11])
    want_out = oracle.forward_routes(to_f64(layer.x), ref["tok_off"], ref["ids"], ref["w"],
                                     ExpertView(layer.w_gate), ExpertView(layer.w_up), ExpertView(layer.w_down),
                                     tokens=tokens)
    err = compare_out(out, want_out, dtype, tokens)
    assert not out[7].any() and not out[11].any()
    _say(f"[proxy] {dtype} N={N} r={r} m={m}: routes {A} bit-exact, {err}")


def test_proxy_full_budget_reconstructs_whole_experts():
    """kappa_j = N for every pick (budget m*N): the split layer's output equals
    the unsplit layer's top-m output (its whole experts concatenated)."""
    N, r, m = 4, 8, 4
    cfg = _small_cfg("f32", T=96, E=64, N=N, k_max=m * N)
    layer = make_layer(cfg, "cuda")
    layer.k.fill_(m * N)
    w_base, gate_idx = make_proxy_inputs(cfg, r, "cuda")
    kappa = moe.moe_proxy_kappa_balanced(m * N, m, N)
    desc, pr, _, _ = _gpu_proxy(layer, N, r, m, kappa, w_base, gate_idx)
    out = _layer_on_routes(layer, desc, pr.tok_off, pr.ids, pr.w)
    # the whole-expert layer: expert e is sub-experts N*e .. N*e+N-1 stacked
    Eb, I, d = cfg.E // N, cfg.I, cfg.d
    wg = layer.w_gate.reshape(Eb, N * I, d)
    wu = layer.w_up.reshape(Eb, N * I, d)
    wd = layer.w_down.reshape(Eb, N, d, I).permute(0, 2, 1, 3).reshape(Eb, d, N * I)
    tokens = np.arange(cfg.T)
    want, _ = oracle.forward(to_f64(layer.x), to_f64(w_base), None, np.full(cfg.T, m), m, ExpertView(wg),
                             ExpertView(wu), ExpertView(wd.contiguous()), routed_scale=cfg.routed_scale,
                             tokens=tokens)
    err = compare_out(out, want, "f32", tokens)
    _say(f"[proxy] full budget reconstruction: {err}")


def test_proxy_full_size_sampled():
    """subexpert_prefill (T=8192, 64 whole experts cut in 4, m=8) with r=4
    gate neurons: whole-expert routes and route offsets on every token; the
    oracle's proxy routing of a token sample (per-token work, so a subset of
    rows is routed as on its own) for the selections and outputs."""
    cfg = CONFIGS["subexpert_prefill"]
    N, r, m = cfg.split, 4, cfg.k_max // cfg.split
    layer = make_layer(cfg, "cuda")
    w_base, gate_idx = make_proxy_inputs(cfg, r, "cuda")
    kappa = moe.moe_proxy_kappa_balanced(cfg.k_max, m, N)
    desc, pr, _, _ = _gpu_proxy(layer, N, r, m, kappa, w_base, gate_idx)
    x64, wb64, k = to_f64(layer.x), to_f64(w_base), to_f64(layer.k)
    base = oracle.route(x64, wb64, None, np.full(cfg.T, m), m, cfg.routed_scale)
    np.testing.assert_array_equal(to_f64(pr.b_tok_off), base["tok_off"])
    np.testing.assert_array_equal(to_f64(pr.b_ids), base["ids"])
    kap = kappa.tolist()
    got_to = to_f64(pr.tok_off)
    np.testing.assert_array_equal(np.diff(got_to), [sum(kap[int(kt)]) for kt in k])
    A = int(got_to[-1])
    got_ids, got_w = to_f64(pr.ids)[:A], pr.w[:A].cpu().double().numpy()
    # the gate-neuron rows only (plain indexing), so that scoring reads r rows
    local = np.tile(np.arange(r), (cfg.E, 1))
    wg_sel, wu_sel = _selected_rows(layer.w_gate, gate_idx), _selected_rows(layer.w_up, gate_idx)
    tokens = sample_tokens(cfg.T, 48)
    ref = oracle.proxy_route(x64[tokens], wb64, None, k[tokens], cfg.k_max, m, N, kap, local, wg_sel, wu_sel,
                             cfg.routed_scale)
    routes = _check_selection(got_to, got_ids, got_w, ref, tokens)
    out = _layer_on_routes(layer, desc, pr.tok_off, pr.ids, pr.w)
    rows = np.arange(16)
    want = oracle.forward_routes(x64[tokens], ref["tok_off"], ref["ids"], ref["w"], ExpertView(layer.w_gate),
                                 ExpertView(layer.w_up), ExpertView(layer.w_down), tokens=rows)
    err = compare_out(out, want, cfg.dtype, tokens[rows])
    _say(f"[proxy] subexpert_prefill r={r}: routes {A}, sampled routes {routes} bit-exact, {err}")


def test_proxy_bad_kappa_rows_and_graph_replay():
    """A kappa row off its budget (an entry above N, or a wrong sum) makes its
    tokens run nothing and sets the status, as in the oracle; the routing
    calls replay in a HIP graph with identical results."""
    N, r, m = 4, 4, 3
    cfg = _small_cfg("bf16", T=70, E=32, N=N, k_max=m * N)
    layer = make_layer(cfg, "cuda")
    w_base, gate_idx = make_proxy_inputs(cfg, r, "cuda")
    kappa = moe.moe_proxy_kappa_balanced(m * N, m, N)
    kappa[5] = torch.tensor([5, 0, 0], dtype=torch.int32)
    kappa[4] = torch.tensor([2, 1, 0], dtype=torch.int32)
    layer.k.copy_(torch.arange(cfg.T, device="cuda") % (m * N + 1))
    desc, pr, wp_g, wp_u = _gpu_proxy(layer, N, r, m, kappa, w_base, gate_idx)
    ref = oracle.proxy_route(to_f64(layer.x), to_f64(w_base), None, to_f64(layer.k), m * N, m, N, kappa.tolist(),
                             to_f64(gate_idx), to_f64(layer.w_gate), to_f64(layer.w_up), cfg.routed_scale)
    assert int(pr.status.item()) == ref["status"] == 1
    got_to = to_f64(pr.tok_off)
    np.testing.assert_array_equal(got_to, ref["tok_off"])
    k = to_f64(layer.k)
    assert all(got_to[t + 1] == got_to[t] for t in range(cfg.T) if k[t] in (4, 5))
    A = int(got_to[-1])
    first = (to_f64(pr.ids)[:A].copy(), pr.w[:A].clone())
    assert _check_selection(got_to, first[0], first[1].cpu().double().numpy(), ref, range(cfg.T)) == A
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        pr.run(layer.x, w_base, None, layer.k, wp_g, wp_u)
    for _ in range(3):
        pr.ids.fill_(-1)
        pr.tok_off.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_f64(pr.tok_off), got_to)
        np.testing.assert_array_equal(to_f64(pr.ids)[:A], first[0])
        assert torch.equal(pr.w[:A], first[1])


@pytest.mark.parametrize("T,N,m,E,r", [(0, 4, 2, 32, 4), (1, 8, 8, 128, 16), (129, 8, 8, 128, 3),
                                        (37, 64, 1, 128, 2)])
def test_proxy_edges(T, N, m, E, r):
    """Empty batch, one token, the widest pick set (m*N = 64) with a ragged
    token count and r not dividing the padded width, and the most sub-experts
    per pick (N = 64: the largest score table and ranking)."""
    k_max = m * N
    cfg = _small_cfg("f32", T=T, E=E, N=N, k_max=k_max)
    layer = make_layer(cfg, "cuda")
    w_base, gate_idx = make_proxy_inputs(cfg, r, "cuda")
    kappa = moe.moe_proxy_kappa_balanced(k_max, m, N)
    desc, pr, _, _ = _gpu_proxy(layer, N, r, m, kappa, w_base, gate_idx)
    ref = oracle.proxy_route(to_f64(layer.x), to_f64(w_base), None, to_f64(layer.k), k_max, m, N, kappa.tolist(),
                             to_f64(gate_idx), to_f64(layer.w_gate), to_f64(layer.w_up), cfg.routed_scale)
    got_to = to_f64(pr.tok_off)
    np.testing.assert_array_equal(got_to, ref["tok_off"])
    assert int(pr.status.item()) == ref["status"] == 0
    if T:
        A = int(got_to[-1])
        assert _check_selection(got_to, to_f64(pr.ids)[:A], pr.w[:A].cpu().double().numpy(), ref, range(T)) == A
