"""Pins of the CPU oracle against things other than itself (CPU only).

Each test would fail for a plausible slip in the oracle: a dropped term or
a wrong operand in the SwiGLU expert, a transposed weight, a wrong softmax
(not renormalised, not shifted, unscaled), a wrong tie order, a wrong
permutation key or an off-by-one in the offsets.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from tests import brute
from workloads import CONFIGS, make_custom_layer, make_layer, to_f64

HERE = os.path.dirname(os.path.abspath(__file__))


def _arrays(layer):
    sh = None
    if layer.ws_gate is not None:
        sh = (to_f64(layer.ws_gate), to_f64(layer.ws_up), to_f64(layer.ws_down))
    return dict(x=to_f64(layer.x), w_router=to_f64(layer.w_router),
                bias=to_f64(layer.router_bias), k=to_f64(layer.k),
                w_gate=to_f64(layer.w_gate), w_up=to_f64(layer.w_up),
                w_down=to_f64(layer.w_down), shared=sh)


def _oracle_forward(a, k_max, scale=1.0, tokens=None, k=None, invalid="raise"):
    return oracle.forward(a["x"], a["w_router"], a["bias"], a["k"] if k is None else k,
                          k_max, a["w_gate"], a["w_up"], a["w_down"], shared=a["shared"],
                          routed_scale=scale, tokens=tokens, invalid=invalid)


# ---------------------------------------------------------------- golden

def test_hand_worked_example():
    g = json.load(open(os.path.join(HERE, "golden", "hand_worked_layer.json")))
    arr = lambda v: np.array(v, dtype=np.float64)
    out, r = oracle.forward(arr(g["x"]), arr(g["w_router"]), None, np.array(g["k"]), 2,
                            arr(g["w_gate"]), arr(g["w_up"]), arr(g["w_down"]))
    assert r["ids"].tolist() == g["expected_ids"]
    exp_w = [eval(s, {"math": math}) for s in g["expected_weights_expr"]]
    exp_o = [eval(s, {"math": math}) for s in g["expected_out_expr"]]
    np.testing.assert_allclose(r["w"], exp_w, rtol=1e-7)   # from fp32 logits 2, 1
    np.testing.assert_allclose(out[0], exp_o, rtol=1e-7)


# ---------------------------------------------------------------- router

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_logits_match_exact_rational(dtype):
    """fp32(float64 sum) equals the exact rational dot product rounded to
    float64 then float32, on inputs where the two can only differ by a
    straddle of probability ~1e-9."""
    L = make_custom_layer(T=6, d=40, E=5, I=8, k=[1] * 6, dtype=dtype, zipf=1.1, seed=3)
    x, wr, b = to_f64(L.x), to_f64(L.w_router), to_f64(L.router_bias)
    got = oracle.router_logits(x, wr, b)
    for t in range(6):
        for e in range(5):
            exact = sum((Fraction(float(x[t, i])) * Fraction(float(wr[e, i]))
                         for i in range(40)), Fraction(float(b[e])))
            assert got[t, e] == np.float32(float(exact))


def test_topk_matches_rank_counting_with_ties():
    """Selection and order equal the rank-counting characterisation (fewer
    than k experts beat the picked one; a tie is won by the lower index),
    including many exact float32 ties and -0.0 vs +0.0."""
    rng = np.random.default_rng(7)
    for _ in range(200):
        E = int(rng.integers(1, 40))
        levels = rng.integers(0, 4, size=E).astype(np.float32) - 1.5
        lg = levels.copy()
        lg[rng.random(E) < 0.1] = np.float32(-0.0)
        lg[rng.random(E) < 0.1] = np.float32(0.0)
        for k in range(0, E + 1):
            got = oracle.select_experts(lg, k).tolist()
            assert got == brute.brute_select(lg.tolist(), k)


def test_weights_are_renormalised_softmax():
    L = make_custom_layer(T=20, d=64, E=16, I=8, k=list(range(1, 17)) + [3, 5, 7, 16], seed=1)
    a = _arrays(L)
    r = oracle.route(a["x"], a["w_router"], None, a["k"], 16, routed_scale=2.5)
    for t in range(20):
        s, e = r["tok_off"][t], r["tok_off"][t + 1]
        sel = r["ids"][s:e]
        ref = 2.5 * scipy.special.softmax(r["logits"][t, sel].astype(np.float64))
        np.testing.assert_allclose(r["w"][s:e], ref, rtol=1e-13)
        # equivalently: the full softmax over E, renormalised to the selected set
        full = scipy.special.softmax(r["logits"][t].astype(np.float64))
        np.testing.assert_allclose(r["w"][s:e], 2.5 * full[sel] / full[sel].sum(), rtol=1e-12)


def test_silu_matches_library():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(oracle.silu(z), z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)
    assert oracle.silu(np.array([0.0]))[0] == 0.0


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("with_shared", [False, True])
def test_forward_matches_brute_force(seed, with_shared):
    rng = np.random.default_rng(seed)
    T, d, E, I = 5, 8, 4, 6
    k = rng.integers(0, E + 1, size=T).tolist()
    L = make_custom_layer(T=T, d=d, E=E, I=I, k=k, I_shared=5 if with_shared else 0,
                          zipf=0.5, seed=seed)
    a = _arrays(L)
    out, r = _oracle_forward(a, E, scale=1.7)
    sh = None
    if with_shared:
        sh = tuple(brute.tolist64(m) for m in a["shared"])
    bout, bids, bw = brute.brute_layer(brute.tolist64(a["x"]), brute.tolist64(a["w_router"]),
                                       brute.tolist64(a["bias"]), k,
                                       brute.tolist64(a["w_gate"]), brute.tolist64(a["w_up"]),
                                       brute.tolist64(a["w_down"]), shared=sh, scale=1.7)
    for t in range(T):
        s, e = r["tok_off"][t], r["tok_off"][t + 1]
        assert r["ids"][s:e].tolist() == bids[t]
        np.testing.assert_allclose(r["w"][s:e], bw[t], rtol=1e-12)
    np.testing.assert_allclose(out, np.array(bout), rtol=1e-10, atol=1e-12)


def test_tiny_fp32_workload_matches_brute_force():
    L = make_layer(CONFIGS["tiny_fp32"].with_(T=4))
    a = _arrays(L)
    out, r = _oracle_forward(a, 2)
    bout, bids, _ = brute.brute_layer(brute.tolist64(a["x"]), brute.tolist64(a["w_router"]), None,
                                      [2] * 4, brute.tolist64(a["w_gate"]),
                                      brute.tolist64(a["w_up"]), brute.tolist64(a["w_down"]))
    assert [r["ids"][2 * t:2 * t + 2].tolist() for t in range(4)] == bids
    np.testing.assert_allclose(out, np.array(bout), rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- identities

def _dense_moe(a, scale=1.0):
    """Dense reference in torch float64: softmax over ALL experts, every
    expert evaluated on every token, weighted sum (the k_t = E limit)."""
    x = torch.tensor(a["x"])
    lg = torch.tensor(oracle.router_logits(a["x"], a["w_router"], a["bias"]).astype(np.float64))
    p = torch.softmax(lg, dim=1) * scale
    out = torch.zeros_like(x)
    for e in range(a["w_gate"].shape[0]):
        g = x @ torch.tensor(a["w_gate"][e]).T
        u = x @ torch.tensor(a["w_up"][e]).T
        y = (torch.nn.functional.silu(g) * u) @ torch.tensor(a["w_down"][e]).T
        out += p[:, e:e + 1] * y
    return out.numpy()


def test_dense_limit_k_equals_E():
    E = 6
    L = make_custom_layer(T=7, d=32, E=E, I=16, k=[E] * 7, zipf=1.1, seed=4)
    a = _arrays(L)
    out, _ = _oracle_forward(a, E, scale=1.3)
    np.testing.assert_allclose(out, _dense_moe(a, 1.3), rtol=1e-11, atol=1e-13)


def test_k1_is_the_argmax_expert():
    L = make_custom_layer(T=9, d=32, E=5, I=16, k=[1] * 9, seed=5)
    a = _arrays(L)
    out, r = _oracle_forward(a, 1, scale=0.75)
    lg = oracle.router_logits(a["x"], a["w_router"], None)
    x = torch.tensor(a["x"])
    for t in range(9):
        e = int(np.argmax(lg[t]))          # first maximum = lower index on ties
        assert r["ids"][t] == e and r["w"][t] == 0.75
        y = (torch.nn.functional.silu(x[t] @ torch.tensor(a["w_gate"][e]).T)
             * (x[t] @ torch.tensor(a["w_up"][e]).T)) @ torch.tensor(a["w_down"][e]).T
        np.testing.assert_allclose(out[t], 0.75 * y.numpy(), rtol=1e-12, atol=1e-14)


def test_neuron_additivity_eq2():
    """MoE-Prism Eq. (2): the expert output is the sum over intermediate
    neurons c of a_c(x) times row c of W_down (column c in [out, in] layout)."""
    L = make_custom_layer(T=3, d=16, E=1, I=10, k=[1] * 3, seed=6)
    a = _arrays(L)
    y = oracle.swiglu_expert(a["x"], a["w_gate"][0], a["w_up"][0], a["w_down"][0])
    acc = np.zeros_like(y)
    for c in range(10):
        ac = scipy.special.expit(a["x"] @ a["w_gate"][0][c]) * (a["x"] @ a["w_gate"][0][c]) \
            * (a["x"] @ a["w_up"][0][c])
        acc += ac[:, None] * a["w_down"][0][:, c][None, :]
    np.testing.assert_allclose(y, acc, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("N", [2, 4])
@pytest.mark.parametrize("contiguous", [True, False])
def test_split_expert_identity(N, contiguous):
    """MoE-Prism Eq. (3) plus the expanded linear gate: cut each expert into
    N equal neuron sets, repeat each router row N times, run k_sub = N*k with
    routed scaling N: the output equals the unsplit layer (each of the N tied
    copies gets w_e / N and the sub-experts sum to the expert)."""
    E, I, d, T = 4, 8, 16, 6
    k = [1, 2, 3, 4, 2, 1]
    L = make_custom_layer(T=T, d=d, E=E, I=I, k=k, zipf=0.3, seed=8)
    a = _arrays(L)
    base, _ = _oracle_forward(a, E)
    rng = np.random.default_rng(N)
    parts = [np.arange(I) if contiguous else rng.permutation(I) for _ in range(E)]
    Is = I // N
    sg = np.stack([a["w_gate"][e][parts[e][n * Is:(n + 1) * Is]] for e in range(E) for n in range(N)])
    su = np.stack([a["w_up"][e][parts[e][n * Is:(n + 1) * Is]] for e in range(E) for n in range(N)])
    sd = np.stack([a["w_down"][e][:, parts[e][n * Is:(n + 1) * Is]] for e in range(E) for n in range(N)])
    wr = np.repeat(a["w_router"], N, axis=0)
    b = np.repeat(a["bias"], N)
    out, r = oracle.forward(a["x"], wr, b, np.array(k) * N, E * N, sg, su, sd, routed_scale=N)
    np.testing.assert_allclose(out, base, rtol=1e-12, atol=1e-13)
    # every selected copy carries exactly the parent's weight / N
    rb = oracle.route(a["x"], a["w_router"], a["bias"], np.array(k), E)
    for t in range(T):
        s, e = r["tok_off"][t], r["tok_off"][t + 1]
        assert (r["ids"][s:e] // N).tolist() == np.repeat(rb["ids"][rb["tok_off"][t]:rb["tok_off"][t + 1]], N).tolist()


def test_split_identity_partial_budget_ties():
    """k_sub = N*k - 1: the tie among the last expert's N copies is broken to
    the lower index, so its first N-1 sub-experts run, each at the weight
    N*exp(l_e)/Z' with Z' the renormaliser over the selected copies."""
    E, I, d, T, N = 5, 8, 16, 4, 4
    k = [2, 3, 1, 4]
    L = make_custom_layer(T=T, d=d, E=E, I=I, k=k, seed=9)
    a = _arrays(L)
    Is = I // N
    sg = a["w_gate"].reshape(E * N, Is, d)
    su = a["w_up"].reshape(E * N, Is, d)
    sd = np.stack([a["w_down"][e][:, n * Is:(n + 1) * Is] for e in range(E) for n in range(N)])
    wr = np.repeat(a["w_router"], N, axis=0)
    ksub = np.array(k) * N - 1
    out, _ = oracle.forward(a["x"], wr, None, ksub, E * N, sg, su, sd, routed_scale=N)
    lg = oracle.router_logits(a["x"], a["w_router"], None).astype(np.float64)
    for t in range(T):
        order = oracle.select_experts(lg[t].astype(np.float32), k[t]).tolist()
        ref = np.zeros(d)
        z = sum(N * math.exp(lg[t, e]) for e in order[:-1]) + (N - 1) * math.exp(lg[t, order[-1]])
        for i, e in enumerate(order):
            nsub = N if i < len(order) - 1 else N - 1
            for n in range(nsub):
                y = oracle.swiglu_expert(a["x"][t:t + 1], sg[e * N + n], su[e * N + n], sd[e * N + n])[0]
                ref += N * math.exp(lg[t, e]) / z * y
        np.testing.assert_allclose(out[t], ref, rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------- permutation

@pytest.mark.parametrize("cfg", ["qwen3_30b_a3b_decode", "tiny_fp32"])
def test_permutation_invariants(cfg):
    c = CONFIGS[cfg]
    L = make_custom_layer(T=c.T, d=64, E=c.E, I=64, k=make_layer(c.with_(d=64, I=64, T=c.T)).k,
                          k_max=c.k_max, zipf=c.zipf_bias, seed=11)
    a = _arrays(L)
    r = oracle.route(a["x"], a["w_router"], a["bias"], a["k"], c.k_max)
    p = oracle.permute(r["tok_off"], r["ids"], c.E)
    A = int(r["tok_off"][-1])
    assert p["counts"].sum() == A == int(a["k"].sum())
    assert p["expert_off"][0] == 0 and (np.diff(p["expert_off"]) == p["counts"]).all()
    tok_of_a = np.repeat(np.arange(c.T), np.diff(r["tok_off"]))
    order = np.lexsort((tok_of_a, r["ids"]))          # library sort by (expert, token)
    assert (p["perm_src"] == order).all()
    assert (p["perm_tok"] == tok_of_a[order]).all()
    assert (p["inv_perm"][p["perm_src"]] == np.arange(A)).all()
    assert sorted(p["perm_src"].tolist()) == list(range(A))
    assert p["n_active"] == len(set(r["ids"].tolist()))
    for e in range(c.E):
        seg = p["perm_tok"][p["expert_off"][e]:p["expert_off"][e + 1]]
        assert (np.diff(seg) > 0).all()
        assert all(e in r["ids"][r["tok_off"][t]:r["tok_off"][t + 1]] for t in seg)


def test_permutation_degenerate():
    p = oracle.permute(np.zeros(1, np.int64), np.zeros(0, np.int64), 4)
    assert p["counts"].tolist() == [0] * 4 and p["n_active"] == 0
    assert p["perm_tok"].size == 0
    p = oracle.permute(np.array([0, 0, 1, 1]), np.array([3]), 4)
    assert p["perm_tok"].tolist() == [1] and p["expert_off"].tolist() == [0, 0, 0, 0, 1]


# ---------------------------------------------------------------- batch semantics

def test_batch_composition_invariance():
    """A token's output depends only on its own x and k (no batch-max k)."""
    L = make_custom_layer(T=12, d=32, E=8, I=16, k=[1, 8, 2, 0, 5, 3, 8, 1, 4, 6, 7, 2],
                          I_shared=8, seed=12)
    a = _arrays(L)
    full, _ = _oracle_forward(a, 8)
    perm = np.random.default_rng(0).permutation(12)
    sub, _ = _oracle_forward(a, 8, tokens=perm[:5])
    np.testing.assert_array_equal(sub, full[perm[:5]])
    shuffled = dict(a, x=a["x"][perm], k=a["k"][perm])
    outp, _ = _oracle_forward(shuffled, 8)
    np.testing.assert_allclose(outp, full[perm], rtol=1e-13, atol=1e-15)


def test_invalid_k():
    L = make_custom_layer(T=4, d=16, E=4, I=8, k=[1, 2, 1, 1], I_shared=4, seed=13)
    a = _arrays(L)
    bad = np.array([1, -1, 5, 2])
    with pytest.raises(ValueError):
        _oracle_forward(a, 4, k=bad)
    out, r = _oracle_forward(a, 4, k=bad, invalid="zero")
    assert r["status"] == 1 and r["k"].tolist() == [1, 0, 0, 2]
    shared_only = oracle.swiglu_expert(a["x"][1:3], *a["shared"])
    np.testing.assert_allclose(out[1:3], shared_only, rtol=1e-14)


def test_zero_input_ties_to_lowest_index():
    """x = 0 makes every logit equal the bias; equal biases tie, so the
    lowest indices win, and SiLU(0) = 0 makes the routed output exactly 0."""
    L = make_custom_layer(T=3, d=16, E=6, I=8, k=[3, 1, 6], seed=14)
    a = _arrays(L)
    a["x"][:] = 0.0
    out, r = _oracle_forward(a, 6)
    assert r["ids"].tolist() == [0, 1, 2, 0, 0, 1, 2, 3, 4, 5]
    np.testing.assert_allclose(r["w"][:3], [1 / 3] * 3, rtol=1e-15)
    assert not out.any()


# ---------------------------------------------------------------- executed budgets

def _smallest_multiple_at_least(k: int, n: int) -> int:
    m = 0
    while m < k:
        m += n
    return m


def test_execution_budgets_exact_is_identity_on_valid():
    k = np.array([0, 1, 4, 8, 3])
    ke, st = oracle.execution_budgets(k, 8)
    assert ke.tolist() == k.tolist() and st == 0


def test_execution_budgets_invalid_tokens_run_nothing():
    k = np.array([2, -1, 9, 5])
    for pol, g in (("exact", 1), ("batch_max", 1), ("round_up", 4)):
        ke, st = oracle.execution_budgets(k, 8, pol, g)
        assert st == 1 and ke[1] == 0 and ke[2] == 0, pol
    # the batch maximum is taken over the valid budgets only (9 is invalid)
    assert oracle.execution_budgets(k, 8, "batch_max")[0].tolist() == [5, 0, 0, 5]


def test_execution_budgets_batch_max_brute_force():
    """Every valid token runs the largest valid budget of the batch (MoE-Prism
    §III-C1), checked token by token against a direct maximum."""
    rng = np.random.default_rng(41)
    for _ in range(50):
        T = int(rng.integers(1, 40))
        k = rng.integers(-2, 11, size=T)
        ke, st = oracle.execution_budgets(k, 8, "batch_max")
        valid = [int(v) for v in k if 0 <= v <= 8]
        kb = max(valid) if valid else 0
        for t in range(T):
            assert ke[t] == (kb if 0 <= k[t] <= 8 else 0)
        assert st == int(len(valid) < T)
        assert all(ke[t] >= k[t] for t in range(T) if 0 <= k[t] <= 8)


def test_execution_budgets_round_up_formula():
    """k_exec = N ceil(k / N) (MoE-Prism §V-D1): with N = 4, 5 runs 8 and 4
    runs 4; checked against the smallest multiple of N not below k."""
    ke, _ = oracle.execution_budgets(np.array([0, 1, 4, 5, 7, 8, 12, 13, 32]), 32, "round_up", 4)
    assert ke.tolist() == [0, 4, 4, 8, 8, 8, 12, 16, 32]
    for n in (1, 2, 3, 4, 8):
        k_max = 24
        k = np.arange(0, k_max + 1)
        ke, st = oracle.execution_budgets(k, k_max, "round_up", n)
        assert st == 0
        assert ke.tolist() == [_smallest_multiple_at_least(int(v), n) for v in k]
        assert (ke % n == 0).all() and (ke <= k_max).all()
    with pytest.raises(ValueError):
        oracle.execution_budgets(np.array([1]), 6, "round_up", 4)   # 6 is not a multiple of 4


def test_over_serving_adds_assignments_never_removes():
    """Under both comparators a token's executed set contains its exact set
    (the same logits, a longer prefix of the same order)."""
    L = make_custom_layer(T=10, d=32, E=16, I=16, k=[1, 3, 2, 0, 5, 8, 4, 2, 7, 6], seed=44)
    a = _arrays(L)
    r0 = oracle.route(a["x"], a["w_router"], a["bias"], a["k"], 8)
    for pol, g in (("batch_max", 1), ("round_up", 4)):
        ke, _ = oracle.execution_budgets(a["k"], 8, pol, g)
        r1 = oracle.route(a["x"], a["w_router"], a["bias"], ke, 8)
        for t in range(10):
            s0 = r0["ids"][r0["tok_off"][t]:r0["tok_off"][t + 1]].tolist()
            s1 = r1["ids"][r1["tok_off"][t]:r1["tok_off"][t + 1]].tolist()
            assert s1[:len(s0)] == s0


def test_eq7_budget_generator():
    """Eq. (7) of MoE-Prism §IV-B2: rounded normal draws clipped to [1, k_max];
    seeded, so the same draw every time."""
    from workloads import draw_k_eq7
    k = draw_k_eq7(20000, 16.0, 8.0, 32, seed=3).numpy()
    assert k.dtype == np.int32 and k.min() >= 1 and k.max() <= 32
    np.testing.assert_array_equal(k, draw_k_eq7(20000, 16.0, 8.0, 32, seed=3).numpy())
    # P(k = 1) = P(x < 1.5), P(k = 32) = P(x >= 31.5) for x ~ N(16, 64)
    p_lo = 0.5 * (1 + math.erf((1.5 - 16) / (8 * math.sqrt(2))))
    p_hi = 1 - 0.5 * (1 + math.erf((31.5 - 16) / (8 * math.sqrt(2))))
    assert abs((k == 1).mean() - p_lo) < 0.01 and abs((k == 32).mean() - p_hi) < 0.01
    inner = k[(k > 1) & (k < 32)]
    assert abs(inner.mean() - 16.0) < 0.3


# ---------------------------------------------------------------- expert folding

def _fold_golden():
    with open(os.path.join(os.path.dirname(__file__), "golden", "fold_hand_worked.json")) as f:
        return json.load(f)


def test_fold_token_hand_worked():
    g = _fold_golden()
    S, L = np.array(g["S"], np.float32), np.array(g["L"], np.float32)
    tk = g["token"]
    for c in tk["cases"]:
        to, ids, w = oracle.fold_token(tk["tok_off"], tk["ids"], tk["w"], S, L, np.array(c["H"], np.float32), c["K"])
        assert to.tolist() == c["tok_off"] and ids.tolist() == c["ids"], c["note"]
        np.testing.assert_allclose(w, c["w"], rtol=1e-6, err_msg=c["note"])


def test_fold_pool_hand_worked():
    g = _fold_golden()
    S, L = np.array(g["S"], np.float32), np.array(g["L"], np.float32)
    pl = g["pool"]
    for c in pl["cases"]:
        to, ids, w, pool = oracle.fold_pool(pl["tok_off"], pl["ids"], pl["w"], S, L, np.array(pl["H"], np.float32),
                                            c["D"], g["E"])
        assert np.flatnonzero(pool).tolist() == c["pool"], c["note"]
        assert to.tolist() == c["tok_off"] and ids.tolist() == c["ids"], c["note"]
        np.testing.assert_allclose(w, c["w"], rtol=1e-6, err_msg=c["note"])


def _random_routes(T, E, kmax, seed):
    rng = np.random.default_rng(seed)
    k = rng.integers(0, kmax + 1, size=T)
    tok_off = np.concatenate([[0], np.cumsum(k)])
    ids = np.concatenate([rng.permutation(E)[:kk] for kk in k]) if k.sum() else np.zeros(0, np.int64)
    w = rng.random(int(k.sum())).astype(np.float32)
    return tok_off, ids.astype(np.int64), w.astype(np.float64)


def test_fold_invariants():
    """Budgets respected, weights conserved when every projector is 1, kept
    routes keep their order, pool routes stay inside the pool, no expert twice
    in a token, and nothing changes when the budget covers everything."""
    from workloads import make_fold_tables
    E = 24
    S, L, H = (t.numpy() for t in make_fold_tables(E, seed=5))
    ones = np.ones((E, E), np.float32)
    for seed in range(6):
        tok_off, ids, w = _random_routes(40, E, 9, seed)
        T = 40
        k = np.diff(tok_off)
        for K in (1, 3, 9):
            to, i2, w2 = oracle.fold_token(tok_off, ids, w, S, L, H, K)
            assert (np.diff(to) == np.minimum(k, K)).all()
            for t in range(T):
                src = ids[tok_off[t]:tok_off[t + 1]].tolist()
                got = i2[to[t]:to[t + 1]].tolist()
                assert all(e in src for e in got)
                assert got == [e for e in src if e in got]          # original order kept
            _, _, w1 = oracle.fold_token(tok_off, ids, w, ones, L, H, K)
            for t in range(T):
                assert np.isclose(w1[to[t]:to[t + 1]].sum(), w[tok_off[t]:tok_off[t + 1]].sum())
        _, i_same, w_same = oracle.fold_token(tok_off, ids, w, S, L, H, 9)
        assert (i_same == ids).all() and (w_same == w).all()
        n_act = len(set(ids.tolist()))
        for D in (1, 4, 10):
            to, i2, w2, pool = oracle.fold_pool(tok_off, ids, w, S, L, H, D, E)
            assert pool.sum() == min(D, n_act) and all(pool[e] for e in i2)
            for t in range(T):
                got = i2[to[t]:to[t + 1]].tolist()
                assert len(got) == len(set(got)) and len(got) <= k[t]
            _, _, w1, _ = oracle.fold_pool(tok_off, ids, w, ones, L, H, D, E)
            for t in range(T):
                assert np.isclose(w1[to[t]:to[t + 1]].sum(), w[tok_off[t]:tok_off[t + 1]].sum())
        to, i_same, w_same, pool = oracle.fold_pool(tok_off, ids, w, S, L, H, n_act, E)
        assert (to == tok_off).all() and (i_same == ids).all() and np.allclose(w_same, w)


def test_forward_routes_matches_forward():
    L = make_custom_layer(T=9, d=32, E=8, I=16, k=[1, 3, 2, 0, 5, 8, 4, 2, 7], I_shared=8, seed=21)
    a = _arrays(L)
    ref, r = _oracle_forward(a, 8)
    got = oracle.forward_routes(a["x"], r["tok_off"], r["ids"], r["w"], a["w_gate"], a["w_up"], a["w_down"],
                                shared=a["shared"])
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- proxy gating (split layer)

def test_kappa_balanced():
    for m in (1, 3, 8):
        for N in (1, 2, 4):
            for k in range(m * N + 1):
                kv = oracle.kappa_balanced(k, m, N)
                assert sum(kv) == k and all(0 <= v <= N for v in kv)
                assert max(kv) - min(kv) <= 1 and kv == sorted(kv, reverse=True)
    with pytest.raises(ValueError):
        oracle.kappa_balanced(9, 2, 4)


def test_proxy_scores_match_scalar_definition():
    """s_n = mean over the gate neurons of |SiLU(g) u|, recomputed neuron by
    neuron with exact sums (math.fsum, then one rounding to float32 each, the
    precision contract) and scipy's logistic function."""
    L = make_custom_layer(T=3, d=24, E=8, I=16, k=[1, 1, 1], seed=31)
    a = _arrays(L)
    rng = np.random.default_rng(2)
    gate_idx = np.stack([rng.permutation(16)[:5] for _ in range(8)])
    for t in range(3):
        for e in range(2):
            s = oracle.proxy_scores(a["x"][t], a["w_gate"], a["w_up"], gate_idx, e, 4)
            for n in range(4):
                sub = 4 * e + n
                vals = []
                for c in gate_idx[sub]:
                    g = float(np.float32(math.fsum(float(p) * float(q) for p, q in zip(a["x"][t], a["w_gate"][sub][c]))))
                    u = float(np.float32(math.fsum(float(p) * float(q) for p, q in zip(a["x"][t], a["w_up"][sub][c]))))
                    vals.append(abs(g * float(scipy.special.expit(g)) * u))
                assert abs(s[n] - math.fsum(vals) / len(vals)) <= 1e-12 * max(1.0, abs(s[n]))


def _split_layer(T, d, E0, I0, N, m, seed):
    """A whole-expert layer and its contiguous split into N sub-experts per
    expert (neuron slices, MoE-Prism Eq. (3))."""
    L = make_custom_layer(T=T, d=d, E=E0, I=I0, k=[m] * T, seed=seed)
    a = _arrays(L)
    I = I0 // N
    wg = np.stack([a["w_gate"][e][n * I:(n + 1) * I] for e in range(E0) for n in range(N)])
    wu = np.stack([a["w_up"][e][n * I:(n + 1) * I] for e in range(E0) for n in range(N)])
    wd = np.stack([a["w_down"][e][:, n * I:(n + 1) * I] for e in range(E0) for n in range(N)])
    return a, wg, wu, wd


def test_proxy_route_all_subexperts_reconstruct_whole_experts():
    """Choosing all N sub-experts of every selected expert (k = m N) gives the
    whole-expert layer's top-m output (MoE-Prism §III-B2: selecting all N
    reconstructs the original contribution)."""
    T, d, E0, I0, N, m = 7, 32, 6, 24, 4, 3
    a, wg, wu, wd = _split_layer(T, d, E0, I0, N, m, seed=33)
    gate_idx = np.stack([np.arange(3)] * (E0 * N))
    kappa = {m * N: [N] * m}
    r = oracle.proxy_route(a["x"], a["w_router"], a["bias"], [m * N] * T, m * N, m, N, kappa, gate_idx, wg, wu)
    got = oracle.forward_routes(a["x"], r["tok_off"], r["ids"], r["w"], wg, wu, wd)
    ref, _ = _oracle_forward(a, m, k=np.full(T, m))
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13)


def test_proxy_route_selection_properties():
    T, d, E0, I0, N, m = 9, 32, 6, 24, 4, 3
    a, wg, wu, wd = _split_layer(T, d, E0, I0, N, m, seed=34)
    rng = np.random.default_rng(3)
    gate_idx = np.stack([rng.permutation(I0 // N)[:4] for _ in range(E0 * N)])
    k = np.array([0, 1, 2, 5, 7, 12, 3, 13, -1])
    kappa = [oracle.kappa_balanced(v, m, N) for v in range(m * N + 1)]
    r = oracle.proxy_route(a["x"], a["w_router"], a["bias"], k, m * N, m, N, kappa, gate_idx, wg, wu)
    assert r["status"] == 1
    base = r["base"]
    for t in range(T):
        got = r["ids"][r["tok_off"][t]:r["tok_off"][t + 1]].tolist()
        if not 0 <= k[t] <= m * N:
            assert got == []
            continue
        assert len(got) == k[t]
        pos = 0
        for j in range(m):
            e = int(base["ids"][base["tok_off"][t] + j])
            kj = kappa[k[t]][j]
            mine = got[pos:pos + kj]
            pos += kj
            assert all(v // N == e for v in mine)                   # sub-experts of the j-th expert
            s = r["scores"][t, j]
            chosen = [v % N for v in mine]
            rest = [n for n in range(N) if n not in chosen]
            assert all(s[c] >= s[o] for c in chosen for o in rest)  # the top kappa_j by proxy score
            assert chosen == sorted(chosen, key=lambda n: (-s[n], n))
            wj = base["w"][base["tok_off"][t] + j]
            assert all(r["w"][r["tok_off"][t] + q] == wj for q in range(pos - kj, pos))


def test_proxy_route_rejects_vectors_off_the_budget():
    """A configured vector must have every kappa_j in [0, N] and sum to its
    budget (MoE-Prism §III-B2): a token whose budget maps to a vector that
    breaks this runs nothing and sets the status; the others are unaffected."""
    T, d, E0, I0, N, m = 6, 32, 6, 24, 4, 3
    a, wg, wu, _ = _split_layer(T, d, E0, I0, N, m, seed=35)
    gate_idx = np.stack([np.arange(3)] * (E0 * N))
    good = [oracle.kappa_balanced(v, m, N) for v in range(m * N + 1)]
    bad = [list(v) for v in good]
    bad[5] = [5, 0, 0]          # entry above N
    bad[4] = [2, 1, 0]          # sums to 3, not 4
    k = np.array([5, 4, 3, 2, 6, 4])
    r_bad = oracle.proxy_route(a["x"], a["w_router"], a["bias"], k, m * N, m, N, bad, gate_idx, wg, wu)
    r_good = oracle.proxy_route(a["x"], a["w_router"], a["bias"], k, m * N, m, N, good, gate_idx, wg, wu)
    assert r_bad["status"] == 1 and r_good["status"] == 0
    for t in range(T):
        got = r_bad["ids"][r_bad["tok_off"][t]:r_bad["tok_off"][t + 1]].tolist()
        ref = r_good["ids"][r_good["tok_off"][t]:r_good["tok_off"][t + 1]].tolist()
        assert got == ([] if k[t] in (4, 5) else ref)


# ---------------------------------------------------------------- compositional paths (PCoMoE)

def test_path_route_hand_worked():
    g = json.load(open(os.path.join(HERE, "golden", "path_hand_worked.json")))
    arr = lambda v: np.array(v, dtype=np.float64)
    P = np.array(g["paths"], dtype=np.float64)
    r = oracle.path_route(arr(g["x"]), arr(g["w_router"]), None, arr(g["w_tgt"]), g["lam"], P[:, 0].astype(int),
                          P[:, 1].astype(int), P[:, 2], np.array(g["k"]), g["k_max"], g["routed_scale"])
    assert r["tok_off"].tolist() == g["tok_off"]
    assert r["src"].tolist() == g["src"] and r["tgt"].tolist() == g["tgt"]
    np.testing.assert_allclose(r["w"], g["w"], rtol=1e-15)
    assert r["status"] == g["status"]
    s_off, s_ids, p2s = oracle.path_sources(r["tok_off"], r["src"])
    assert s_off.tolist() == g["src_tok_off"] and s_ids.tolist() == g["src_ids"]
    assert p2s.tolist() == g["path_src_route"]


def _path_layer(seed, E=6, d=24, I=16, T=11):
    L = make_custom_layer(T=T, d=d, E=E, I=I, k=[2] * T, seed=seed)
    a = _arrays(L)
    rng = np.random.default_rng(seed)
    a["w_tgt"] = rng.standard_normal((E, d)) / math.sqrt(d)
    return a


def test_path_diagonal_mask_reproduces_vanilla():
    """Diagonal-only paths with zero biases and no target term (or lambda = 0)
    give the vanilla routes and weights bit for bit, and the vanilla output
    (PCoMoE: restricting to diagonal paths recovers the original layer)."""
    E, T = 6, 11
    a = _path_layer(41, E=E, T=T)
    k = np.array([0, 1, 2, 3, 6, 4, 2, 1, 5, 3, 2])
    diag = np.arange(E)
    ref = oracle.route(a["x"], a["w_router"], a["bias"], k, E, 1.5)
    for w_tgt, lam in ((None, 0.7), (a["w_tgt"], 0.0)):
        r = oracle.path_route(a["x"], a["w_router"], a["bias"], w_tgt, lam, diag, diag, np.zeros(E), k, E, 1.5)
        assert (r["tok_off"] == ref["tok_off"]).all()
        assert (r["src"] == ref["ids"]).all() and (r["tgt"] == ref["ids"]).all()
        assert (r["w"] == ref["w"]).all()
    out = oracle.path_forward(a["x"], r["tok_off"], r["src"], r["tgt"], r["w"], a["w_gate"], a["w_up"], a["w_down"])
    want, _ = oracle.forward(a["x"], a["w_router"], a["bias"], k, E, a["w_gate"], a["w_up"], a["w_down"],
                             routed_scale=1.5)
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-14)
    # with an always-on shared expert, on a layer that has one
    L = make_custom_layer(T=T, d=24, E=E, I=16, k=k, I_shared=8, seed=44)
    b = _arrays(L)
    r = oracle.path_route(b["x"], b["w_router"], b["bias"], None, 0.0, diag, diag, np.zeros(E), k, E)
    out = oracle.path_forward(b["x"], r["tok_off"], r["src"], r["tgt"], r["w"], b["w_gate"], b["w_up"], b["w_down"],
                              shared=b["shared"])
    want, _ = oracle.forward(b["x"], b["w_router"], b["bias"], k, E, b["w_gate"], b["w_up"], b["w_down"],
                             shared=b["shared"])
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-14)


def test_path_forward_is_the_sum_over_paths():
    """Source-grouped evaluation equals the plain sum over paths of
    beta * W_down[j] (SiLU(W_gate[i] h) * (W_up[i] h)), each path on its own
    (scipy's logistic function), and runs U once per distinct source."""
    E = 6
    a = _path_layer(42, E=E)
    src = np.array([0, 0, 1, 2, 2, 5, 3, 3, 3, 4, 1])
    tgt = np.array([0, 3, 1, 2, 0, 5, 3, 1, 4, 4, 2])
    p_bias = np.linspace(-0.5, 0.3, len(src))
    k = np.array([3, 4, 0, 2, 5, 1, 3, 2, 6, 4, 3])
    r = oracle.path_route(a["x"], a["w_router"], None, a["w_tgt"], 0.4, src, tgt, p_bias, k, 6)
    cnt = {}
    got = oracle.path_forward(a["x"], r["tok_off"], r["src"], r["tgt"], r["w"], a["w_gate"], a["w_up"],
                              a["w_down"], counter=cnt)
    want = np.zeros_like(got)
    n_src = 0
    for t in range(a["x"].shape[0]):
        lo, hi = r["tok_off"][t], r["tok_off"][t + 1]
        n_src += len(set(r["src"][lo:hi].tolist()))
        for q in range(lo, hi):
            i, j = r["src"][q], r["tgt"][q]
            gl = a["w_gate"][i] @ a["x"][t]
            z = gl * scipy.special.expit(gl) * (a["w_up"][i] @ a["x"][t])
            want[t] += r["w"][q] * (a["w_down"][j] @ z)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)
    assert cnt == {"U": n_src, "D": int(r["tok_off"][-1])}
    assert n_src < r["tok_off"][-1]           # some paths share their source


def test_path_route_invariances():
    """A constant added to every pair bias changes no selection and no
    weight (softmax shift invariance, up to the one float32 rounding); a large
    bias on one pair puts it first for every token with k_t >= 1; every
    selection is the top k_t of the scores."""
    E = 6
    a = _path_layer(43, E=E)
    src = np.array([0, 0, 1, 1, 2, 3, 3, 4, 5, 5])
    tgt = np.array([0, 4, 1, 2, 2, 3, 0, 4, 1, 5])
    p_bias = np.array([0, -0.3, 0, -0.1, 0, 0, -0.2, 0, -0.4, 0])
    k = np.array([1, 2, 3, 4, 5, 6, 7, 8, 2, 3, 1])
    base = oracle.path_route(a["x"], a["w_router"], None, a["w_tgt"], 0.6, src, tgt, p_bias, k, 10)
    shifted = oracle.path_route(a["x"], a["w_router"], None, a["w_tgt"], 0.6, src, tgt, p_bias + 0.25, k, 10)
    assert (base["src"] == shifted["src"]).all() and (base["tgt"] == shifted["tgt"]).all()
    np.testing.assert_allclose(base["w"], shifted["w"], rtol=1e-6)
    boosted = p_bias.copy()
    boosted[6] = 50.0
    b = oracle.path_route(a["x"], a["w_router"], None, a["w_tgt"], 0.6, src, tgt, boosted, k, 10)
    for t in range(len(k)):
        assert (b["src"][b["tok_off"][t]], b["tgt"][b["tok_off"][t]]) == (3, 0)
    for t in range(len(k)):
        s = base["scores"][t]
        chosen = base["src"][base["tok_off"][t]:base["tok_off"][t + 1]] * E + \
            base["tgt"][base["tok_off"][t]:base["tok_off"][t + 1]]
        pos = [int(np.nonzero(src * E + tgt == c)[0][0]) for c in chosen]
        rest = [p for p in range(len(src)) if p not in pos]
        assert all(s[p] >= s[q] for p in pos for q in rest)
        assert all(s[pos[i]] >= s[pos[i + 1]] for i in range(len(pos) - 1))
