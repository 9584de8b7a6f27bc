"""Pure-Python brute force of the MoE layer on tiny inputs.

Independent of oracle/: plain lists and loops, math.fsum for the router dot
products (the correctly rounded float64 sum of exact products, then one
rounding to float32), selection by counting ranks instead of sorting, and the
SwiGLU expert of MoE-Prism (arXiv 2510.19366) §III-B1 Eq. (1) written neuron by
neuron as in Eq. (2).
"""
import math

import numpy as np


def _f32(v: float) -> float:
    return float(np.float32(v))


def sigmoid(z: float) -> float:
    if z >= 0:
        return 1.0 / (1.0 + math.exp(-z))
    ez = math.exp(z)
    return ez / (1.0 + ez)


def brute_logits(x_t, w_router, bias):
    E = len(w_router)
    out = []
    for e in range(E):
        terms = [x_t[i] * w_router[e][i] for i in range(len(x_t))]
        if bias is not None:
            terms.append(bias[e])
        out.append(_f32(math.fsum(terms)))
    return out


def brute_select(logits, k):
    """Expert e is picked iff fewer than k experts beat it, where e' beats e
    when its logit is larger, or equal with a lower index.  The rank is the
    number of experts that beat it; picked experts are listed by rank."""
    E = len(logits)
    rank = {}
    for e in range(E):
        rank[e] = sum(1 for f in range(E)
                      if logits[f] > logits[e] or (logits[f] == logits[e] and f < e))
    picked = [e for e in range(E) if rank[e] < k]
    return sorted(picked, key=lambda e: rank[e])


def brute_expert(x_t, wg, wu, wd):
    """y_q = sum_c SiLU(<x, wg[c]>) * <x, wu[c]> * wd[q][c]."""
    I = len(wg)
    d_out = len(wd)
    acts = []
    for c in range(I):
        g = math.fsum(x_t[i] * wg[c][i] for i in range(len(x_t)))
        u = math.fsum(x_t[i] * wu[c][i] for i in range(len(x_t)))
        acts.append(g * sigmoid(g) * u)
    return [math.fsum(acts[c] * wd[q][c] for c in range(I)) for q in range(d_out)]


def brute_layer(x, w_router, bias, k, w_gate, w_up, w_down, shared=None, scale=1.0):
    """Returns (out, ids per token, weights per token) as Python lists."""
    T = len(x)
    outs, all_ids, all_w = [], [], []
    for t in range(T):
        lg = brute_logits(x[t], w_router, bias)
        ids = brute_select(lg, k[t])
        if ids:
            m = lg[ids[0]]
            ex = [math.exp(lg[e] - m) for e in ids]
            z = math.fsum(ex)
            w = [scale * v / z for v in ex]
        else:
            w = []
        d = len(x[t])
        out = [0.0] * d
        for e, we in zip(ids, w):
            y = brute_expert(x[t], w_gate[e], w_up[e], w_down[e])
            out = [out[q] + we * y[q] for q in range(d)]
        if shared is not None:
            ys = brute_expert(x[t], shared[0], shared[1], shared[2])
            out = [out[q] + ys[q] for q in range(d)]
        outs.append(out)
        all_ids.append(ids)
        all_w.append(w)
    return outs, all_ids, all_w


def tolist64(a):
    return np.asarray(a, dtype=np.float64).tolist()
