"""CPU oracle of the MoE layer forward with a per-token routing top-k.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The HIP library never calls it and
shares no code with it.

What it computes (plain definition, numpy, float64 unless a step fixes a
precision):

* Router: logits over all E experts, one linear map of the token's hidden
  state plus an optional bias.  The pages do not fix the precision; the
  contract used on both sides is "exact dot product, accumulated in float64,
  rounded once to float32", so that the integer decision taken from it (which
  experts, in which order) is taken on the same float32 values everywhere.
* Selection: the token's budget k_t is external (MoE-Prism, arXiv 2510.19366,
  §III-C1: the request tuple carries its own routing budget, counted in
  routed experts excluding shared ones, §II-B).  The k_t experts with the
  largest logits are taken, ordered by router probability (§III-B2, proxy
  gating paragraph: the router orders the selected experts by probability);
  equal float32 logits are ordered by the lower expert index.
* Weights: softmax over the selected logits, i.e. the softmax over all E
  renormalised to the selected set, times the routed scaling factor (§III-B2:
  the router weights are normalised, then scaled; the expanded linear gate
  keeps the model's routing normalisation and an N-adjusted routed scaling).
* Executed budgets: a token runs its own k_t, or under the over-serving
  comparators the batch's largest budget (§III-C1) or k_t rounded up to a
  multiple of N (§V-D1).
* Expert folding (ExFold summary, arXiv 2608.24938): token-level top-K and
  batch-level expert-pool folding of the routes into kept targets with
  scalar projectors S and projection losses L (fold_token, fold_pool).
* Proxy gating of a split layer (MoE-Prism §III-B2, training-free path):
  whole-expert routing, then the top kappa_j sub-experts by a gate-neuron
  proxy score, each inheriting its expert's weight (proxy_route).
* Compositional paths (PCoMoE, arXiv 2609.01024): scores over a fixed active
  path mask, per-token top-k_t paths, and the source-grouped output in which
  each distinct source's expansion runs once (path_route, path_sources,
  path_forward).
* Expert FFN: SwiGLU, §III-B1 Eq. (1): A = SiLU(X W_gate) * (X W_up) and
  X' = A W_down, with SiLU(z) = z * sigmoid(z).  Weights are stored in the
  [out, in] layout, so X W_gate of the page is x @ w_gate[e].T here.
* Output: sum over the token's selected experts of weight times expert
  output, plus an always-on shared expert with weight 1 when present.
* Permutation (dispatch metadata): per-expert counts, their exclusive scan,
  and the assignments sorted by (expert, token) -- a stable counting sort.
  The activated-expert count is the number of distinct experts with at least
  one assignment (METRO reading notes, arXiv 2512.09277, Q1: decode runtime
  follows the activated experts' weight loads).

Pinned by tests/test_oracle_pins.py against closed forms, brute force on tiny
inputs, exact rational arithmetic, library routines and the identities the
pages state (dense limit, single expert, neuron additivity Eq. (2)/(3), the
split-expert / repeated-router-row identity of the expanded linear gate).
"""
from __future__ import annotations

from typing import Any, Optional, Sequence

import numpy as np

__all__ = [
    "execution_budgets",
    "fold_token",
    "fold_pool",
    "forward_routes",
    "kappa_balanced",
    "proxy_scores",
    "proxy_route",
    "path_scores",
    "path_route",
    "path_sources",
    "path_forward",
    "router_logits",
    "select_experts",
    "route",
    "permute",
    "silu",
    "swiglu_expert",
    "forward",
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def router_logits(x, w_router, bias=None) -> np.ndarray:
    """Router logits, float32 [T, E].

    l[t, e] = fp32( sum_i x[t, i] * w_router[e, i] + bias[e] ), the sum taken
    in float64 (products of float32 or bfloat16 values are exact in float64)
    and rounded once to float32.
    """
    acc = _f64(x) @ _f64(w_router).T
    if bias is not None:
        acc = acc + _f64(bias)[None, :]
    return acc.astype(np.float32)


def select_experts(logits_row: np.ndarray, k: int) -> np.ndarray:
    """The k experts of one token, ordered by (logit descending, index
    ascending).  A stable sort on the negated float32 logits gives exactly
    that order (equal logits keep ascending index order; -0.0 == +0.0)."""
    order = np.argsort(-np.asarray(logits_row, dtype=np.float32), kind="stable")
    return order[:k].astype(np.int64)


def execution_budgets(k, k_max: int, policy: str = "exact", granule: int = 1):
    """Budgets the layer executes, and the invalid-budget status.

    A k_t outside [0, k_max] is invalid: it sets the status to 1 and the token
    runs no routed expert under every policy.  For the valid ones:
      exact      k_t itself (MoE-Prism §III-C1: the request's own budget);
      batch_max  the largest valid budget of the whole batch, for every valid
                 token (§III-C1: one dispatch mixing budgets runs the batch
                 maximum, over-serving the smaller requests);
      round_up   N * ceil(k_t / N) with N = granule (§V-D1: a layout of whole
                 experts, each N sub-experts wide, executes only multiples of
                 N); k_max must be a multiple of N.
    Returns (int64 [T] executed budgets, status 0 or 1).
    """
    k = np.asarray(k, dtype=np.int64)
    valid = (k >= 0) & (k <= k_max)
    status = int((~valid).any())
    kv = np.where(valid, k, 0)
    if policy == "exact":
        ke = kv
    elif policy == "batch_max":
        kb = int(kv.max()) if kv.size else 0
        ke = np.where(valid, kb, 0)
    elif policy == "round_up":
        if granule < 1 or k_max % granule:
            raise ValueError("round_up needs granule >= 1 dividing k_max")
        ke = -(-kv // granule) * granule
    else:
        raise ValueError(f"unknown budget policy {policy!r}")
    return ke.astype(np.int64), status


def route(x, w_router, bias, k, k_max: int, routed_scale: float = 1.0,
          invalid: str = "raise"):
    """Route every token.

    Returns a dict with
      logits  float32 [T, E]
      k       int64 [T]    (budgets after validation)
      tok_off int64 [T+1]  exclusive prefix sum of k; tok_off[T] = A
      ids     int64 [A]    selected experts, token-major, best first
      w       float64 [A]  routing weights
      status  int          1 if some k_t was outside [0, k_max] (invalid="zero")

    A k_t outside [0, k_max] raises (invalid="raise") or, with
    invalid="zero", is treated as k_t = 0 and flagged in status.
    """
    k = np.asarray(k, dtype=np.int64).copy()
    T = k.shape[0]
    E = np.asarray(w_router).shape[0]
    status = 0
    bad = (k < 0) | (k > k_max)
    if bad.any():
        if invalid == "raise":
            raise ValueError(f"k_t outside [0, {k_max}] at tokens {np.nonzero(bad)[0][:8]}")
        status = 1
        k[bad] = 0
    if k_max > E:
        raise ValueError("k_max exceeds the number of experts")
    logits = router_logits(x, w_router, bias) if T else np.zeros((0, E), np.float32)
    tok_off = np.zeros(T + 1, dtype=np.int64)
    tok_off[1:] = np.cumsum(k)
    A = int(tok_off[T])
    ids = np.zeros(A, dtype=np.int64)
    w = np.zeros(A, dtype=np.float64)
    for t in range(T):
        kt = int(k[t])
        if kt == 0:
            continue
        sel = select_experts(logits[t], kt)
        l_sel = logits[t, sel].astype(np.float64)
        p = np.exp(l_sel - l_sel[0])          # l_sel[0] is the largest
        ids[tok_off[t]:tok_off[t + 1]] = sel
        w[tok_off[t]:tok_off[t + 1]] = routed_scale * p / p.sum()
    return {"logits": logits, "k": k, "tok_off": tok_off, "ids": ids, "w": w,
            "status": status}


def permute(tok_off, ids, E: int):
    """Dispatch metadata for the grouped expert FFN.

    Returns a dict with
      counts     int64 [E]    assignments per expert
      expert_off int64 [E+1]  exclusive scan of counts
      perm_tok   int64 [A]    token of sorted row p
      perm_src   int64 [A]    flat assignment index (tok_off[t] + j) of row p
      inv_perm   int64 [A]    sorted row of flat assignment a
      n_active   int          experts with at least one assignment
    Rows are sorted by (expert ascending, token ascending).
    """
    tok_off = np.asarray(tok_off, dtype=np.int64)
    ids = np.asarray(ids, dtype=np.int64)
    T = tok_off.shape[0] - 1
    A = int(tok_off[T])
    counts = np.zeros(E, dtype=np.int64)
    triples = []
    for t in range(T):
        for a in range(int(tok_off[t]), int(tok_off[t + 1])):
            e = int(ids[a])
            counts[e] += 1
            triples.append((e, t, a))
    triples.sort()                           # (expert, token); a is unique per (e, t)
    expert_off = np.zeros(E + 1, dtype=np.int64)
    expert_off[1:] = np.cumsum(counts)
    perm_tok = np.array([tr[1] for tr in triples], dtype=np.int64).reshape(A)
    perm_src = np.array([tr[2] for tr in triples], dtype=np.int64).reshape(A)
    inv_perm = np.zeros(A, dtype=np.int64)
    inv_perm[perm_src] = np.arange(A, dtype=np.int64)
    return {"counts": counts, "expert_off": expert_off, "perm_tok": perm_tok,
            "perm_src": perm_src, "inv_perm": inv_perm,
            "n_active": int((counts > 0).sum())}


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    z = _f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_expert(x_rows, w_gate_e, w_up_e, w_down_e) -> np.ndarray:
    """One SwiGLU expert on a set of rows (MoE-Prism §III-B1, Eq. (1)).

    x_rows [M, d]; w_gate_e, w_up_e [I, d]; w_down_e [d, I]  ->  [M, d]
    """
    x_rows = _f64(x_rows)
    a = silu(x_rows @ _f64(w_gate_e).T) * (x_rows @ _f64(w_up_e).T)
    return a @ _f64(w_down_e).T


def forward(x, w_router, bias, k, k_max: int, w_gate, w_up, w_down,
            shared: Optional[Sequence[Any]] = None, routed_scale: float = 1.0,
            tokens: Optional[Sequence[int]] = None, invalid: str = "raise"):
    """Layer forward for the tokens listed in ``tokens`` (all by default).

    ``w_gate``, ``w_up``, ``w_down`` only need ``[e]`` indexing that returns
    expert e's matrix ([I, d], [I, d], [d, I]); each expert is read once.
    ``shared`` is (ws_gate [Is, d], ws_up [Is, d], ws_down [d, Is]) or None.
    Returns (out float64 [len(tokens), d], routing dict of those tokens).
    """
    x = np.asarray(x)
    k = np.asarray(k)
    if tokens is None:
        tokens = np.arange(x.shape[0])
    tokens = np.asarray(tokens, dtype=np.int64)
    xs = _f64(x[tokens])
    r = route(xs, w_router, bias, k[tokens], k_max, routed_scale, invalid=invalid)
    n = len(tokens)
    d = xs.shape[1]
    out = np.zeros((n, d), dtype=np.float64)
    # Expert outputs y_e(x_t) for every selected (t, e), one expert at a time.
    E = np.asarray(w_router).shape[0]
    y = {}
    by_expert = [[] for _ in range(E)]
    for i in range(n):
        for a in range(int(r["tok_off"][i]), int(r["tok_off"][i + 1])):
            by_expert[int(r["ids"][a])].append(i)
    for e in range(E):
        rows = by_expert[e]
        if not rows:
            continue
        ye = swiglu_expert(xs[rows], w_gate[e], w_up[e], w_down[e])
        for j, i in enumerate(rows):
            y[(i, e)] = ye[j]
    for i in range(n):
        for a in range(int(r["tok_off"][i]), int(r["tok_off"][i + 1])):
            out[i] += r["w"][a] * y[(i, int(r["ids"][a]))]
    if shared is not None:
        out += swiglu_expert(xs, shared[0], shared[1], shared[2])
    return out, r


# ---------------------------------------------------------------------------
# Expert folding (ExFold summary, arXiv 2608.24938: Unified Expert Folding;
# Phase-Specific Selection and Unified Folding; Phase-Specific Routing and
# Folding).  Routes a token keeps are executed; each route it drops is folded
# into a kept target: the target is the one with the smallest projection loss
# L[source][target], and the dropped route's weight, times the scalar
# projector S[source][target], is added to the target's weight.  Expert
# parameters and the router are untouched; only routing metadata changes.
# Decisions are taken on float32 values (scores are float32 products, losses
# are compared as stored); weights are accumulated here in float64.

def _routes(tok_off, ids, w):
    tok_off = np.asarray(tok_off, dtype=np.int64)
    return tok_off, np.asarray(ids, dtype=np.int64), np.asarray(w, dtype=np.float64)


def _csr(rows):
    """Per-token lists of (expert, weight) -> (tok_off, ids, w)."""
    tok_off = np.zeros(len(rows) + 1, dtype=np.int64)
    tok_off[1:] = np.cumsum([len(r) for r in rows])
    ids = np.array([e for r in rows for e, _ in r], dtype=np.int64)
    w = np.array([v for r in rows for _, v in r], dtype=np.float64)
    return tok_off, ids, w


def fold_token(tok_off, ids, w, S, L, H, K: int):
    """Token-level top-K folding (prefill; ExFold: K_pre dominant experts per
    token).  A token with more than K routes keeps the K with the largest
    estimated contribution, router weight times the expert's calibrated output
    magnitude H[e] (the ranking the ablations find best), ties to the earlier
    route; each dropped route goes to the kept route of smallest
    L[dropped][kept] (ties to the earlier kept route).  Kept routes stay in
    their original order.  Returns (tok_off, ids, w) of the folded routes."""
    tok_off, ids, w = _routes(tok_off, ids, w)
    S = np.asarray(S, dtype=np.float32)
    L = np.asarray(L, dtype=np.float32)
    H = np.asarray(H, dtype=np.float32)
    rows = []
    for t in range(tok_off.shape[0] - 1):
        a0, a1 = int(tok_off[t]), int(tok_off[t + 1])
        e = [int(v) for v in ids[a0:a1]]
        wt = [float(v) for v in w[a0:a1]]
        n = a1 - a0
        if n <= K:
            rows.append(list(zip(e, wt)))
            continue
        score = [np.float32(np.float32(wt[j]) * H[e[j]]) for j in range(n)]
        order = sorted(range(n), key=lambda j: (-score[j], j))
        kept = sorted(order[:K])
        neww = {i: wt[i] for i in kept}
        for j in range(n):
            if j in neww:
                continue
            tgt = min(kept, key=lambda i: (L[e[j], e[i]], i))
            neww[tgt] += wt[j] * float(S[e[j], e[tgt]])
        rows.append([(e[i], neww[i]) for i in kept])
    return _csr(rows)


def fold_pool(tok_off, ids, w, S, L, H, D: int, E: int):
    """Batch-level expert-pool folding (decode; ExFold: D dominant experts per
    batch, dynamic pool).  The pool is the D activated experts with the largest
    aggregate routed contribution H[e] * sum of the weights routed to e (the
    sum in float64 over tokens in order), ties to the lower index; every route
    to an expert outside the pool goes to the pool expert of smallest
    L[source][p] (ties to the lower index).  A token's routes that land on the
    same expert are coalesced into one, at the place of the first of them, with
    the weights added in route order (the target executes once).
    Returns (tok_off, ids, w, pool bool [E])."""
    tok_off, ids, w = _routes(tok_off, ids, w)
    S = np.asarray(S, dtype=np.float32)
    L = np.asarray(L, dtype=np.float32)
    H = np.asarray(H, dtype=np.float32)
    T = tok_off.shape[0] - 1
    agg = np.zeros(E, dtype=np.float64)
    count = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for a in range(int(tok_off[t]), int(tok_off[t + 1])):
            agg[ids[a]] += float(np.float32(w[a]))
            count[ids[a]] += 1
    score = agg * H.astype(np.float64)
    active = [e for e in range(E) if count[e] > 0]
    pool_list = sorted(active, key=lambda e: (-score[e], e))[:D]
    pool = np.zeros(E, dtype=bool)
    pool[pool_list] = True
    members = sorted(pool_list)
    rows = []
    for t in range(T):
        out = {}
        order = []
        for a in range(int(tok_off[t]), int(tok_off[t + 1])):
            e = int(ids[a])
            if pool[e]:
                tgt, c = e, float(w[a])
            else:
                tgt = min(members, key=lambda p: (L[e, p], p))
                c = float(w[a]) * float(S[e, tgt])
            if tgt not in out:
                out[tgt] = 0.0
                order.append(tgt)
            out[tgt] += c
        rows.append([(p, out[p]) for p in order])
    tok_off2, ids2, w2 = _csr(rows)
    return tok_off2, ids2, w2, pool


def forward_routes(x, tok_off, ids, w, w_gate, w_up, w_down, shared: Optional[Sequence[Any]] = None,
                   tokens: Optional[Sequence[int]] = None) -> np.ndarray:
    """Layer output for explicit routes (CSR tok_off / ids / w over the whole
    batch), for the tokens listed in ``tokens`` (all by default): the weighted
    sum of the routed experts' SwiGLU outputs plus the shared expert."""
    x = np.asarray(x)
    tok_off, ids, w = _routes(tok_off, ids, w)
    if tokens is None:
        tokens = np.arange(x.shape[0])
    tokens = np.asarray(tokens, dtype=np.int64)
    xs = _f64(x[tokens])
    out = np.zeros((len(tokens), xs.shape[1]), dtype=np.float64)
    by_expert = {}
    for i, t in enumerate(tokens):
        for a in range(int(tok_off[t]), int(tok_off[t + 1])):
            by_expert.setdefault(int(ids[a]), []).append((i, float(w[a])))
    for e, lst in by_expert.items():
        rows = [i for i, _ in lst]
        ye = swiglu_expert(xs[rows], w_gate[e], w_up[e], w_down[e])
        for j, (i, wt) in enumerate(lst):
            out[i] += wt * ye[j]
    if shared is not None:
        out += swiglu_expert(xs, shared[0], shared[1], shared[2])
    return out


# ---------------------------------------------------------------------------
# Training-free proxy (complex-gate) routing of a split layer (MoE-Prism,
# arXiv 2510.19366, §III-B2, Training-Free Proxy Gating).  The original
# router picks m whole experts per token and their weights; among the N
# sub-experts of the j-th one, the kappa_j with the largest proxy scores run,
# each inheriting the whole expert's weight (no second softmax).  The proxy
# score of a sub-expert is the mean absolute SwiGLU activation over its r
# gate neurons.  Sub-expert n of whole expert e has index N*e + n.

def kappa_balanced(k: int, m: int, N: int) -> list:
    """A budget k split over the m selected experts: as evenly as possible,
    the remainder to the experts of higher router probability (the page
    leaves the configured vectors open).  Needs 0 <= k <= m*N."""
    if not 0 <= k <= m * N:
        raise ValueError("budget outside [0, m*N]")
    q, rem = divmod(k, m)
    return [q + (1 if j < rem else 0) for j in range(m)]


def proxy_scores(x_row, w_gate, w_up, gate_idx, e: int, N: int) -> np.ndarray:
    """s_n(x) = (1/r) sum over the gate neurons c of sub-expert N*e + n of
    |SiLU(g_c) * u_c| for n < N (MoE-Prism §III-B2, proxy-gating paragraph).

    The page fixes no precision; the contract is the router's: g_c = x .
    w_gate[sub][c] and u_c = x . w_up[sub][c] are taken in float64 (exact
    products) and rounded once to float32 each; the activations and their sum
    over c (in the order of gate_idx, then divided by r) are float64."""
    x = _f64(x_row)
    out = np.zeros(N, dtype=np.float64)
    for n in range(N):
        sub = N * e + n
        c = np.asarray(gate_idx[sub], dtype=np.int64)
        g = (_f64(w_gate[sub])[c] @ x).astype(np.float32).astype(np.float64)
        u = (_f64(w_up[sub])[c] @ x).astype(np.float32).astype(np.float64)
        acts = np.abs(silu(g) * u)
        total = 0.0
        for v in acts:
            total += float(v)
        out[n] = total / len(c)
    return out


def proxy_route(x, w_router_base, bias, k, k_max: int, m: int, N: int, kappa, gate_idx, w_gate, w_up,
                routed_scale: float = 1.0):
    """Routes of the split layer under proxy gating.  ``kappa[k]`` is the
    vector (kappa_1 .. kappa_m) for budget k (sub-expert units).  A k_t outside
    [0, k_max], or whose vector breaks 0 <= kappa_j <= N or sum_j kappa_j = k_t,
    runs nothing and sets status 1.  Within a whole expert the
    chosen sub-experts are listed by proxy score (descending, ties to the lower
    n).  Returns a dict with tok_off, ids, w (float64), status and the proxy
    scores [T][m][N] for the validity check of the selections."""
    k = np.asarray(k, dtype=np.int64)
    T = k.shape[0]
    base = route(x, w_router_base, bias, np.full(T, m), m, routed_scale)

    def runs(kt):
        # a configured vector has every kappa_j in [0, N] and sums to the budget
        return 0 <= kt <= k_max and all(0 <= int(v) <= N for v in kappa[kt]) and sum(int(v) for v in kappa[kt]) == kt

    status = int(any(not runs(int(kt)) for kt in k))
    rows, scores = [], np.zeros((T, m, N), dtype=np.float64)
    for t in range(T):
        kt = int(k[t])
        row = []
        if runs(kt):
            kv = kappa[kt]
            for j in range(m):
                a = int(base["tok_off"][t]) + j
                e = int(base["ids"][a])
                s = proxy_scores(x[t], w_gate, w_up, gate_idx, e, N)
                scores[t, j] = s
                order = sorted(range(N), key=lambda n: (-s[n], n))[:int(kv[j])]
                row += [(N * e + n, float(base["w"][a])) for n in order]
        rows.append(row)
    tok_off, ids, w = _csr(rows)
    return {"tok_off": tok_off, "ids": ids, "w": w, "status": status, "scores": scores, "base": base}


# ---------------------------------------------------------------------------
# Compositional path routing and source-grouped execution (PCoMoE, arXiv
# 2609.01024).  Expert e splits at its expansion/projection boundary into
# U_e(h) = SiLU(W_gate[e] h) * (W_up[e] h) and D_e(z) = W_down[e] z, so that
# F_e = D_e(U_e); a path (i, j) is D_j(U_i(h)) and the diagonal (e, e) is the
# vanilla expert.  Only the active paths of a fixed mask are candidates.

def path_scores(g_row, t_row, p_src, p_tgt, p_bias, lam: float) -> np.ndarray:
    """Scores of the active paths of one token (compatibility-aware path
    gating, Fig. 7): the source's base routing logit plus the pair's
    compatibility bias plus lambda times the target's prior logit,
        s_p = fp32( (g[src_p] + b_p) + lam * t[tgt_p] )
    evaluated in float64 in that order and rounded once to float32.  t_row
    None drops the target term."""
    g = _f64(g_row)[np.asarray(p_src, dtype=np.int64)]
    acc = g + _f64(p_bias)
    if t_row is not None:
        acc = acc + float(lam) * _f64(t_row)[np.asarray(p_tgt, dtype=np.int64)]
    return acc.astype(np.float32)


def path_route(x, w_router, bias, w_tgt, lam: float, p_src, p_tgt, p_bias, k, k_max: int,
               routed_scale: float = 1.0):
    """Per-token top-k_t over the active paths (compositional path routing).

    The active set is the list (p_src, p_tgt, p_bias), strictly increasing in
    (src, tgt).  g are the router logits of w_router (+ bias) and t those of
    w_tgt (no bias; None drops the term), both under the routing contract of
    router_logits.  The k_t paths with the largest scores are taken, equal
    scores in list order; their weights are the softmax over the selected
    scores times routed_scale (the vanilla renormalised softmax, which the
    diagonal-only mask reproduces exactly).  A k_t outside [0, k_max] runs
    nothing and sets status 1.  Returns a dict with tok_off, src, tgt, w
    (float64), status and the scores [T][P]."""
    k = np.asarray(k, dtype=np.int64)
    T = k.shape[0]
    P = len(p_src)
    g = router_logits(x, w_router, bias)
    t = router_logits(x, w_tgt, None) if w_tgt is not None else None
    status = int(((k < 0) | (k > k_max)).any())
    scores = np.zeros((T, P), dtype=np.float32)
    rows = []
    for tt in range(T):
        s = path_scores(g[tt], None if t is None else t[tt], p_src, p_tgt, p_bias, lam)
        scores[tt] = s
        kt = int(k[tt])
        row = []
        if 0 <= kt <= k_max:
            order = np.argsort(-s, kind="stable")[:kt]
            sel = s[order].astype(np.float64)
            p = np.exp(sel - sel[0]) if kt else sel
            for q, idx in enumerate(order):
                row.append((int(p_src[idx]), int(p_tgt[idx]), routed_scale * p[q] / p.sum()))
        rows.append(row)
    tok_off = np.zeros(T + 1, dtype=np.int64)
    tok_off[1:] = np.cumsum([len(r) for r in rows])
    src = np.array([a for r in rows for a, _, _ in r], dtype=np.int64)
    tgt = np.array([b for r in rows for _, b, _ in r], dtype=np.int64)
    w = np.array([c for r in rows for _, _, c in r], dtype=np.float64)
    return {"tok_off": tok_off, "src": src, "tgt": tgt, "w": w, "status": status, "scores": scores}


def path_sources(tok_off, src):
    """Source groups (source-grouped compute reuse, Fig. 8): per token, the
    distinct sources of its paths in ascending order.  Returns (src_tok_off,
    src_ids, path_src_route) where path_src_route[a] is the source route of
    path a."""
    tok_off = np.asarray(tok_off, dtype=np.int64)
    src = np.asarray(src, dtype=np.int64)
    T = tok_off.shape[0] - 1
    s_off = np.zeros(T + 1, dtype=np.int64)
    ids, p2s = [], np.zeros(src.shape[0], dtype=np.int64)
    for t in range(T):
        mine = src[tok_off[t]:tok_off[t + 1]]
        uniq = sorted(set(int(v) for v in mine))
        for a in range(int(tok_off[t]), int(tok_off[t + 1])):
            p2s[a] = len(ids) + uniq.index(int(src[a]))
        ids += uniq
        s_off[t + 1] = len(ids)
    return s_off, np.array(ids, dtype=np.int64), p2s


def path_forward(x, tok_off, src, tgt, w, w_gate, w_up, w_down, tokens: Optional[Sequence[int]] = None,
                 counter: Optional[dict] = None, shared: Optional[Sequence[Any]] = None) -> np.ndarray:
    """Layer output over paths, source-grouped: for each token, U_i runs once
    per distinct source i and D_j once per path (i, j):
        y = sum_i sum_{j in T_i} beta_ij D_j(U_i(h)),
    plus the always-on shared expert with weight 1 when given (as in the
    vanilla layer, MoE-Prism §II-B).  counter, if given, receives the number
    of U and D evaluations."""
    x = np.asarray(x)
    tok_off = np.asarray(tok_off, dtype=np.int64)
    if tokens is None:
        tokens = np.arange(x.shape[0])
    tokens = np.asarray(tokens, dtype=np.int64)
    out = np.zeros((len(tokens), x.shape[1]), dtype=np.float64)
    n_u = n_d = 0
    for r, t in enumerate(tokens):
        h = _f64(x[t])
        groups = {}
        for a in range(int(tok_off[t]), int(tok_off[t + 1])):
            groups.setdefault(int(src[a]), []).append((int(tgt[a]), float(w[a])))
        for i, paths in groups.items():
            z = silu(_f64(w_gate[i]) @ h) * (_f64(w_up[i]) @ h)
            n_u += 1
            for j, b in paths:
                out[r] += b * (_f64(w_down[j]) @ z)
                n_d += 1
    if shared is not None:
        out += swiglu_expert(_f64(x[tokens]), shared[0], shared[1], shared[2])
    if counter is not None:
        counter["U"] = n_u
        counter["D"] = n_d
    return out
