"""Parity of the HIP path (through the C ABI) with the CPU oracle on the GPU.

Routing ids, token offsets, per-expert counts, the permutation and the
activated-expert count must match bit for bit; outputs must be within
relative L2 <= 1e-2 and max |err| <= 5e-2 (bf16) or relative L2 <= 1e-5
(fp32).  Full-size workloads are checked on every token's routing and on a
spread sample of output rows (the oracle computes them one by one).
"""
import gc
import sys

import numpy as np
import pytest
import torch

import mixture_experts_layer_token_amd as moe
from tests.gpu_util import (check_routing, compare_out, compare_rows, covering_tokens, oracle_out,
                            oracle_routing, run_forward, run_stages, sample_tokens)
import oracle
from tests.gpu_util import desc_of
from workloads import CONFIGS, ExpertView, make_custom_layer, make_layer, to_f64

pytestmark = pytest.mark.gpu

# Output rows checked against the oracle per workload: all rows of the
# smaller batches; on the prefill batches a covering set, one token for every
# (expert, 64-row block) of the permutation and every 64-token block of the
# shared expert (covering_tokens), plus a spread sample.
SAMPLE = {"tiny_fp32": 16, "mixtral_decode": 64, "qwen3_30b_a3b_decode": 256,
          "subexpert_prefill": 24, "dsv3_decode": 128, "dsv3_prefill": 8}


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe._lib.load()
    yield
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", list(CONFIGS))
def test_workload_parity(name):
    cfg = CONFIGS[name]
    _say(f"[parity] {name}: drawing layer")
    layer = make_layer(cfg, "cuda")
    got = run_stages(layer)
    r, p = oracle_routing(layer)
    check_routing(got, r, p)
    fout, stats, status = run_forward(layer)
    assert status == 0
    torch.testing.assert_close(fout, got["out"], rtol=0, atol=0)   # fused == staged, bit for bit
    np.testing.assert_array_equal(stats[:cfg.E], p["counts"])
    assert stats[cfg.E] == p["n_active"] and stats[cfg.E + 1] == got["A"]
    tokens = sample_tokens(cfg.T, SAMPLE[name])
    if cfg.T > SAMPLE[name]:
        tokens = np.union1d(tokens, covering_tokens(got, cfg.T, 64, shared=cfg.I_shared > 0))
    _say(f"[parity] {name}: oracle on {len(tokens)} of {cfg.T} tokens")
    err = compare_out(fout, oracle_out(layer, tokens), cfg.dtype, tokens)
    _say(f"[parity] {name}: A={got['A']} n_active={p['n_active']} {err}")


@pytest.mark.parametrize("name", [n for n, c in CONFIGS.items() if c.dtype == "bf16"])
def test_workload_paths_agree_on_every_row(name):
    """The two FFN implementations (weight-streaming kernels, grouped GEMM),
    which share no kernel code, agree on every output row of the full-size
    batch to the output tolerance: a fault in any one row tile, column tile or
    shared-expert tile of either path would show here, while the oracle checks
    the covering rows above."""
    cfg = CONFIGS[name]
    _say(f"[paths-all-rows] {name}: drawing layer")
    layer = make_layer(cfg, "cuda")
    a, sa, st_a = run_forward(layer, path="stream")
    b, sb, st_b = run_forward(layer, path="gemm")
    assert st_a == st_b == 0
    np.testing.assert_array_equal(sa, sb)
    err = compare_rows(a, b, cfg.dtype)
    _say(f"[paths-all-rows] {name}: {err}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,E,d,I,kmax,Is", [
    (300, 8, 128, 256, 8, 0),      # ragged: two permutation blocks, k up to E (dense limit)
    (70, 257, 256, 128, 12, 128),  # E just above 256 (8 keys per lane), shared expert
    (33, 1024, 128, 128, 20, 0),   # largest E
    (1, 4, 128, 128, 4, 0),        # single token
    (129, 64, 384, 384, 64, 0),    # k_t up to E = 64
    (300, 128, 128, 128, 100, 0),  # two permutation blocks with k_t > 64 assignments per token
])
def test_shapes_and_ragged(dtype, T, E, d, I, kmax, Is):
    rng = np.random.default_rng(T + E)
    k = rng.integers(0, kmax + 1, size=T)
    k[0] = kmax
    layer = make_custom_layer(T=T, d=d, E=E, I=I, k=k, dtype=dtype, k_max=kmax, I_shared=Is,
                              zipf=0.7, seed=T, device="cuda")
    got = run_stages(layer)
    r, p = oracle_routing(layer)
    check_routing(got, r, p)
    tokens = sample_tokens(T, 40)
    compare_out(got["out"], oracle_out(layer, tokens), dtype, tokens)


@pytest.mark.parametrize("router", ["float64", "screened", "fused"])
def test_zero_tokens(router):
    layer = make_custom_layer(T=0, d=128, E=4, I=128, k=[], dtype="bf16", k_max=2, device="cuda")
    out, stats, status = run_forward(layer, router=router)
    assert out.shape == (0, 128) and status == 0
    assert stats[:4].tolist() == [0] * 4 and stats[4] == 0 and stats[5] == 0


def test_all_k_zero_gives_shared_only():
    T = 9
    layer = make_custom_layer(T=T, d=128, E=6, I=128, k=[0] * T, dtype="f32", k_max=3, I_shared=256,
                              device="cuda")
    out, stats, status = run_forward(layer)
    assert stats[7] == 0 and stats[6] == 0
    compare_out(out, oracle_out(layer, np.arange(T)), "f32", np.arange(T))


def test_invalid_k_flagged_and_dropped():
    k = [2, -1, 3, 9, 1]
    layer = make_custom_layer(T=5, d=128, E=8, I=128, k=k, dtype="bf16", k_max=3, device="cuda")
    got = run_stages(layer)
    r, p = oracle_routing(layer)
    assert r["status"] == moe.MOE_DEV_BAD_K
    check_routing(got, r, p)
    assert not got["out"][1].any() and not got["out"][3].any()


@pytest.mark.parametrize("T", [64, 300])
@pytest.mark.parametrize("router", ["float64", "screened", "fused"])
@pytest.mark.parametrize("policy,granule", [("batch_max", 1), ("round_up", 4), ("round_up", 2)])
def test_budget_policies(policy, granule, router, T):
    """Over-serving comparators (MoE-Prism §III-C1: a mixed dispatch runs the
    batch maximum; §V-D1: whole experts of N sub-experts run N ceil(k/N)):
    the same kernels run the transformed budgets.  Routing bit-exact against
    the oracle on the transformed budgets, outputs to tolerance, invalid
    budgets flagged and dropped, moe_forward equal to the staged calls."""
    E, d, I, kmax = 64, 256, 256, 8
    rng = np.random.default_rng(T + granule)
    k = rng.integers(0, kmax + 1, size=T)
    k[3], k[7] = kmax + 2, -1
    layer = make_custom_layer(T=T, d=d, E=E, I=I, k=k, dtype="bf16", k_max=kmax, zipf=0.8, seed=9,
                              device="cuda")
    got = run_stages(layer, router=router, k_policy=policy, k_granule=granule)
    r, p = oracle_routing(layer, policy, granule)
    assert r["status"] == moe.MOE_DEV_BAD_K
    check_routing(got, r, p)
    tokens = sample_tokens(T, 40)
    err = compare_out(got["out"], oracle_out(layer, tokens, policy, granule), "bf16", tokens)
    assert not got["out"][3].any() and not got["out"][7].any()
    fout, _, status = run_forward(layer, router=router, k_policy=policy, k_granule=granule)
    assert status == moe.MOE_DEV_BAD_K
    torch.testing.assert_close(fout, got["out"], rtol=0, atol=0)
    _say(f"[budgets] {policy}/{granule} {router} T={T}: A={got['A']} {err}")


@pytest.mark.parametrize("E", [16, 32])
@pytest.mark.parametrize("router", ["float64", "screened", "fused"])
def test_exact_ties_break_to_lower_index(router, E):
    """Zero hidden states make every logit equal its bias; duplicated router
    rows make exactly tied logits for any x."""
    T = 40
    layer = make_custom_layer(T=T, d=128, E=E, I=128, k=[5] * T, dtype="bf16", k_max=8, device="cuda")
    layer.x[: T // 2].zero_()
    layer.w_router[1::2].copy_(layer.w_router[0::2])           # experts 2j and 2j+1 tie
    got = run_stages(layer, router=router)
    r, p = oracle_routing(layer)
    check_routing(got, r, p)
    assert got["ids"][:5].tolist() == [0, 1, 2, 3, 4]
    for t in range(T):
        sel = got["ids"][5 * t:5 * t + 5]
        for e in sel:
            if e % 2 == 1:
                assert e - 1 in sel          # an odd copy is only taken after its even twin


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,E,d,kmax", [(1024, 256, 2048, 16), (1, 1, 128, 1), (77, 3, 384, 3),
                                        (300, 128, 4096, 8), (64, 8, 4096, 2),
                                        # Qwen3-shaped rows, T at its limit, few and non-power-of-two E,
                                        # d at its limit, k_t up to E
                                        (256, 128, 2048, 8), (1024, 128, 2048, 8), (5, 32, 128, 4),
                                        (129, 96, 2048, 8), (33, 64, 8192, 6), (70, 32, 4224, 32)])
def test_fused_router_matches_split_and_oracle(dtype, T, E, d, kmax):
    """The one-launch router of small batches: routing bit-exact against the
    oracle and equal to the split-K float64 router (ids, weights, offsets),
    at the largest batch and E x d it takes, E = 1 and non-power-of-two E, d
    at its limit (8192 with E = 64) and k_t up to E."""
    rng = np.random.default_rng(T * 7 + E)
    k = rng.integers(0, kmax + 1, size=T)
    k[0] = kmax
    layer = make_custom_layer(T=T, d=d, E=E, I=128, k=k, dtype=dtype, k_max=kmax, zipf=0.9, seed=T + E,
                              device="cuda")
    a = run_stages(layer, router="fused")
    b = run_stages(layer, router="float64")
    r, p = oracle_routing(layer)
    check_routing(a, r, p)
    for key in ("tok_off", "ids", "w", "perm_tok", "inv_perm"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    assert a["status"] == b["status"] == 0


def test_deterministic_bits():
    layer = make_layer(CONFIGS["qwen3_30b_a3b_decode"], "cuda")
    a, _, _ = run_forward(layer)
    b, _, _ = run_forward(layer)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_graph_capture_replays_any_k():
    """One captured graph of moe_forward serves every k mix."""
    cfg = CONFIGS["qwen3_30b_a3b_decode"]
    layer = make_layer(cfg, "cuda")
    desc = moe.make_desc(cfg.T, cfg.d, cfg.E, cfg.I, cfg.k_max, dtype=layer.x.dtype)
    ws = moe.alloc_workspace(desc)
    k_static = layer.k.clone()
    out = torch.empty_like(layer.x)
    stats = torch.empty(cfg.E + 2, dtype=torch.int32, device="cuda")
    status = torch.empty(1, dtype=torch.int32, device="cuda")

    def call():
        moe.moe_forward(desc, layer.x, layer.w_router, layer.router_bias, k_static, layer.w_gate,
                        layer.w_up, layer.w_down, None, None, None, out, stats, status, ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    rng = np.random.default_rng(1)
    for rep in range(4):
        kv = torch.as_tensor(rng.choice([0, 1, 2, 4, 8], size=cfg.T).astype(np.int32), device="cuda")
        k_static.copy_(kv)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        st = stats.clone()
        layer.k = kv
        ref, ref_stats, _ = run_forward(layer)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
        assert torch.equal(st.cpu(), torch.as_tensor(ref_stats, dtype=torch.int32))


@pytest.mark.parametrize("path", ["stream", "gemm"])
@pytest.mark.parametrize("T,E,d,I,kmax,Is", [
    (700, 16, 256, 384, 8, 256),     # ragged row blocks, shared expert over 700 tokens
    (300, 8, 128, 128, 8, 0),        # every expert has 100-300 rows
    (1500, 64, 512, 256, 16, 128),   # many experts, uneven rows
    (40, 32, 384, 128, 4, 0),        # few rows per expert (GEMM tail-only tiles)
    (520, 8, 256, 256, 4, 256),      # shared expert as wide as the routed ones: fused into the GEMM launches
    (48, 4, 2176, 2176, 2, 2176),    # K % 256 = 128 (2 x 2 stream waves) and long K (deep stream pipeline)
    (200, 16, 512, 256, 8, 256),     # 128-row GEMM tiles: 256-column gate/up, 512-column down, fused shared expert
    (90, 8, 768, 512, 6, 0),         # 128-row GEMM tiles: 256-column gate/up and down (d % 512 != 0)
    (8, 2, 128, 128, 1, 128),        # fused shared expert, fewer tiles than XCDs in both problems of a launch
    (130, 3, 256, 256, 2, 256),      # fused shared expert: two shared row tiles, a handful of routed ones
])
def test_ffn_paths_bf16(path, T, E, d, I, kmax, Is):
    """Both FFN paths compute the same function on the same routing."""
    rng = np.random.default_rng(T * E)
    k = rng.integers(1, kmax + 1, size=T)
    layer = make_custom_layer(T=T, d=d, E=E, I=I, k=k, dtype="bf16", k_max=kmax, I_shared=Is, zipf=1.0,
                              seed=E, device="cuda")
    got = run_stages(layer, path=path)
    r, p = oracle_routing(layer)
    check_routing(got, r, p)
    tokens = sample_tokens(T, 48)
    err = compare_out(got["out"], oracle_out(layer, tokens), "bf16", tokens)
    fout, _, _ = run_forward(layer, path=path)
    torch.testing.assert_close(fout, got["out"], rtol=0, atol=0)
    _say(f"[paths] {path} T={T} E={E}: {err}")


@pytest.mark.parametrize("name,path", [("qwen3_30b_a3b_decode", "gemm"), ("subexpert_prefill", "stream")])
def test_workload_other_path(name, path):
    """A workload on the path AUTO does not pick for it."""
    cfg = CONFIGS[name]
    layer = make_layer(cfg, "cuda")
    fout, stats, status = run_forward(layer, path=path)
    assert status == 0
    got = run_stages(layer, path=path)
    tokens = np.union1d(sample_tokens(cfg.T, 16), covering_tokens(got, cfg.T, 64, shared=cfg.I_shared > 0))
    compare_out(fout, oracle_out(layer, tokens), cfg.dtype, tokens)


@pytest.mark.parametrize("T,E,d,kmax,zipf", [
    (1000, 256, 2048, 32, 0.0),   # sub-expert-like: many candidates near the cut
    (777, 64, 1024, 8, 1.1),      # biased router, ragged T
    (300, 1024, 256, 20, 0.5),    # largest E
    (129, 8, 4096, 8, 0.0),       # k_t up to E
])
def test_screened_router_bit_exact(T, E, d, kmax, zipf):
    """The MFMA-screened router selects, orders and weights exactly like the
    float64 router and the oracle (only the cost differs)."""
    rng = np.random.default_rng(T + E)
    k = rng.integers(0, kmax + 1, size=T)
    layer = make_custom_layer(T=T, d=d, E=E, I=128, k=k, dtype="bf16", k_max=kmax, zipf=zipf, seed=E,
                              device="cuda")
    layer.x[T // 3].zero_()                                    # a token with all logits = bias
    got = run_stages(layer, router="screened")
    ref64 = run_stages(layer, router="float64")
    r, p = oracle_routing(layer)
    check_routing(got, r, p)
    np.testing.assert_array_equal(got["ids"], ref64["ids"])
    np.testing.assert_array_equal(got["w"], ref64["w"])        # same fp32 logits -> same weights


@pytest.mark.parametrize("name,path", [("qwen3_30b_a3b_decode", "stream"), ("qwen3_30b_a3b_decode", "gemm"),
                                       ("tiny_fp32", "stream")])
def test_split_ffn_calls_match_moe_ffn(name, path):
    """moe_ffn_plan + moe_ffn_gateup + moe_ffn_down give moe_ffn's routed output
    bit for bit (the Zipf-skewed batch has experts spanning several row blocks)."""
    cfg = CONFIGS[name]
    layer = make_layer(cfg, "cuda")
    got = run_stages(layer, path=path)
    dev = layer.device
    desc = moe.make_desc(cfg.T, cfg.d, cfg.E, cfg.I, cfg.k_max, dtype=layer.x.dtype, path=path)
    i32 = dict(dtype=torch.int32, device=dev)
    eoff = torch.as_tensor(got["expert_off"], **i32)
    ptok = torch.zeros(cfg.T * cfg.k_max, **i32)
    ptok[:got["A"]] = torch.as_tensor(got["perm_tok"], **i32)
    ws = moe.alloc_workspace(desc, moe.MOE_OP_FFN, dev)
    y_ref = torch.empty((cfg.T * cfg.k_max, cfg.d), dtype=layer.x.dtype, device=dev)
    moe.moe_ffn(desc, layer.x, layer.w_gate, layer.w_up, layer.w_down, None, None, None, eoff, ptok, y_ref,
                None, ws)
    h = torch.empty((cfg.T * cfg.k_max, cfg.I), dtype=layer.x.dtype, device=dev)
    y = torch.empty_like(y_ref)
    ws2 = moe.alloc_workspace(desc, moe.MOE_OP_FFN, dev)
    moe.moe_ffn_plan(desc, eoff, ws2)
    moe.moe_ffn_gateup(desc, layer.x, layer.w_gate, layer.w_up, eoff, ptok, h, ws2)
    moe.moe_ffn_down(desc, h, layer.w_down, eoff, y, ws2)
    torch.cuda.synchronize()
    A = got["A"]
    assert torch.equal(y[:A].view(torch.int16 if y.dtype == torch.bfloat16 else torch.int32),
                       y_ref[:A].view(torch.int16 if y.dtype == torch.bfloat16 else torch.int32))


# ---------------------------------------------------------------- expert folding

def _synthetic_routes(T, E, kmax, seed, dev):
    """Seeded routes (distinct experts per token, float32 weights) as both
    sides' input: the folding stage is tested on its own."""
    rng = np.random.default_rng(seed)
    k = rng.integers(0, kmax + 1, size=T)
    k[0] = kmax
    tok_off = np.concatenate([[0], np.cumsum(k)]).astype(np.int64)
    ids = np.concatenate([rng.permutation(E)[:kk] for kk in k]).astype(np.int64)
    w = rng.random(int(k.sum())).astype(np.float32)
    w[5] = w[6] = w[7]   # equal weights: ties in the token ranking
    i32 = lambda a: torch.as_tensor(a.astype(np.int32), device=dev)
    return tok_off, ids, w, i32(tok_off), i32(ids), torch.as_tensor(w, device=dev)


def _gpu_fold(desc, mode, budget, tables, to_d, ids_d, w_d, dev):
    S, L, H = (t.to(dev) for t in tables)
    T, E, km = desc.T, desc.E, desc.k_max
    i32 = dict(dtype=torch.int32, device=dev)
    eoff = psrc = None
    if mode == "pool":
        counts = torch.empty(E, **i32)
        eoff = torch.empty(E + 1, **i32)
        ptok = torch.empty(max(T * km, 1), **i32)
        psrc = torch.empty_like(ptok)
        inv = torch.empty_like(ptok)
        nact = torch.empty(1, **i32)
        moe.moe_permute(desc, to_d, ids_d, counts, eoff, ptok, psrc, inv, nact,
                        moe.alloc_workspace(desc, moe.MOE_OP_PERMUTE, dev))
    to_o = torch.full((T + 1,), -7, **i32)
    ids_o = torch.full((max(T * km, 1),), -7, **i32)
    w_o = torch.full((max(T * km, 1),), float("nan"), dtype=torch.float32, device=dev)
    pool = torch.full((E,), -7, **i32)
    moe.moe_fold(desc, mode, budget, S, L, H, to_d, ids_d, w_d, eoff, psrc, to_o, ids_o, w_o, pool,
                 moe.alloc_workspace(desc, moe.MOE_OP_FOLD, dev))
    torch.cuda.synchronize()
    n = int(to_o[T].item())
    return (to_o.cpu().numpy().astype(np.int64), ids_o[:n].cpu().numpy().astype(np.int64),
            w_o[:n].cpu().double().numpy(), pool.cpu().numpy())


@pytest.mark.parametrize("T,E,kmax,budget", [(300, 64, 16, 4), (64, 128, 8, 3), (8192, 256, 32, 8), (5, 8, 4, 1)])
def test_fold_token_matches_oracle(T, E, kmax, budget):
    """Token-level folding (ExFold, prefill): kept routes and targets
    bit-exact, folded weights to float32 rounding of the additions."""
    from workloads import make_fold_tables
    dev = "cuda"
    tok_off, ids, w, to_d, ids_d, w_d = _synthetic_routes(T, E, kmax, T + E, dev)
    tables = make_fold_tables(E, seed=E)
    desc = moe.make_desc(T, 128, E, 128, kmax)
    got_to, got_ids, got_w, _ = _gpu_fold(desc, "token", budget, tables, to_d, ids_d, w_d, dev)
    S, L, H = (t.numpy() for t in tables)
    ref_to, ref_ids, ref_w = oracle.fold_token(tok_off, ids, w.astype(np.float64), S, L, H, budget)
    np.testing.assert_array_equal(got_to, ref_to)
    np.testing.assert_array_equal(got_ids, ref_ids)
    np.testing.assert_allclose(got_w, ref_w, rtol=1e-5, atol=1e-6)
    _say(f"[fold token] T={T} E={E} K={budget}: routes {tok_off[-1]} -> {ref_to[-1]}")


@pytest.mark.parametrize("T,E,kmax,budget", [(256, 128, 8, 32), (300, 64, 16, 8), (64, 8, 2, 4), (40, 32, 6, 1)])
def test_fold_pool_matches_oracle(T, E, kmax, budget):
    """Expert-pool folding (ExFold, decode): pool, targets and merged routes
    bit-exact, weights to float32 rounding."""
    from workloads import make_fold_tables
    dev = "cuda"
    tok_off, ids, w, to_d, ids_d, w_d = _synthetic_routes(T, E, kmax, 3 * T + E, dev)
    tables = make_fold_tables(E, seed=E + 1)
    desc = moe.make_desc(T, 128, E, 128, kmax)
    got_to, got_ids, got_w, got_pool = _gpu_fold(desc, "pool", budget, tables, to_d, ids_d, w_d, dev)
    S, L, H = (t.numpy() for t in tables)
    ref_to, ref_ids, ref_w, ref_pool = oracle.fold_pool(tok_off, ids, w.astype(np.float64), S, L, H, budget, E)
    np.testing.assert_array_equal(got_pool, ref_pool.astype(np.int64))
    np.testing.assert_array_equal(got_to, ref_to)
    np.testing.assert_array_equal(got_ids, ref_ids)
    np.testing.assert_allclose(got_w, ref_w, rtol=1e-5, atol=1e-6)
    _say(f"[fold pool] T={T} E={E} D={budget}: experts {len(set(ids.tolist()))} -> {int(ref_pool.sum())}")


@pytest.mark.parametrize("name,mode,budget", [("qwen3_30b_a3b_decode", "pool", 32), ("subexpert_prefill", "token", 8)])
def test_folded_layer_matches_oracle(name, mode, budget):
    """Route -> fold -> permute -> FFN -> combine on a workload against the
    oracle's route -> fold -> explicit-route forward (sampled tokens)."""
    from workloads import make_fold_tables
    cfg = CONFIGS[name]
    layer = make_layer(cfg, "cuda")
    dev = layer.device
    desc = desc_of(layer)
    T, d, E, km = desc.T, desc.d, desc.E, desc.k_max
    i32 = dict(dtype=torch.int32, device=dev)
    tok_off = torch.empty(T + 1, **i32)
    ids = torch.empty(T * km, **i32)
    w = torch.empty(T * km, dtype=torch.float32, device=dev)
    status = torch.empty(1, **i32)
    moe.moe_route(desc, layer.x, layer.w_router, layer.router_bias, layer.k, tok_off, ids, w, status,
                  moe.alloc_workspace(desc, moe.MOE_OP_ROUTE, dev))
    tables = make_fold_tables(E, seed=1)
    to_f, ids_f, w_f, _ = _gpu_fold(desc, mode, budget, tables, tok_off, ids, w, dev)
    # the rest of the layer on the folded routes
    to_d = torch.as_tensor(to_f.astype(np.int32), device=dev)
    ids_d = torch.as_tensor(ids_f.astype(np.int32), device=dev)
    w_d = torch.as_tensor(w_f.astype(np.float32), device=dev)
    counts = torch.empty(E, **i32)
    eoff = torch.empty(E + 1, **i32)
    ptok = torch.empty(T * km, **i32)
    psrc = torch.empty_like(ptok)
    inv = torch.empty_like(ptok)
    nact = torch.empty(1, **i32)
    moe.moe_permute(desc, to_d, ids_d, counts, eoff, ptok, psrc, inv, nact,
                    moe.alloc_workspace(desc, moe.MOE_OP_PERMUTE, dev))
    y = torch.empty((T * km, d), dtype=layer.x.dtype, device=dev)
    moe.moe_ffn(desc, layer.x, layer.w_gate, layer.w_up, layer.w_down, None, None, None, eoff, ptok, y, None,
                moe.alloc_workspace(desc, moe.MOE_OP_FFN, dev))
    out = torch.empty((T, d), dtype=layer.x.dtype, device=dev)
    moe.moe_combine(desc, y, None, to_d, w_d, inv, out)
    torch.cuda.synchronize()
    # oracle: its own routing, its own folding, explicit-route forward
    r, _ = oracle_routing(layer)
    S, L, H = (t.numpy() for t in tables)
    if mode == "pool":
        rt, ri, rw, pool = oracle.fold_pool(r["tok_off"], r["ids"], r["w"], S, L, H, budget, E)
        assert int(nact.item()) == int(pool.sum()) <= budget
    else:
        rt, ri, rw = oracle.fold_token(r["tok_off"], r["ids"], r["w"], S, L, H, budget)
    np.testing.assert_array_equal(to_f, rt)
    np.testing.assert_array_equal(ids_f, ri)
    tokens = sample_tokens(T, SAMPLE[name])
    ref = oracle.forward_routes(to_f64(layer.x), rt, ri, rw, ExpertView(layer.w_gate), ExpertView(layer.w_up),
                                ExpertView(layer.w_down), tokens=tokens)
    err = compare_out(out, ref, cfg.dtype, tokens)
    _say(f"[fold layer] {name} {mode}={budget}: n_active {int(nact.item())} {err}")
