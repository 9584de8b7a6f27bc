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
    "router_logits",
    "select_experts",
    "route",
    "permute",
    "silu",
    "swiglu_expert",
    "forward",
    "activated_weight_bytes",
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


def activated_weight_bytes(n_active: int, d: int, I: int, elem_bytes: int) -> int:
    """Routed-expert weight bytes a batch must load: gate, up and down of every
    activated expert (METRO reading notes, Q1: decode runtime follows these
    loads; activations are a small fraction of the traffic)."""
    return 3 * n_active * d * I * elem_bytes
