"""Helpers of the GPU parity tests: run the HIP path stage by stage or fused
through the C ABI, and compare with the CPU oracle."""
from __future__ import annotations

import numpy as np
import torch

import mixture_experts_layer_token_amd as moe
import oracle
from workloads import ExpertView, Layer, to_f64

TOL = {"bf16": dict(rel_l2=1e-2, max_abs=5e-2), "f32": dict(rel_l2=1e-5, max_abs=None)}


def desc_of(layer: Layer, path: str = "auto", router: str = "auto", k_policy: str = "exact",
            k_granule: int = 1) -> moe.moe_desc:
    c = layer.cfg
    E, I, d = layer.w_gate.shape
    Is = layer.ws_gate.shape[0] if layer.ws_gate is not None else 0
    return moe.make_desc(layer.x.shape[0], d, E, I, c.k_max, I_shared=Is, dtype=layer.x.dtype,
                         path=path, router=router, routed_scale=c.routed_scale, k_policy=k_policy,
                         k_granule=k_granule)


def shared_of(layer: Layer):
    return None if layer.ws_gate is None else (layer.ws_gate, layer.ws_up, layer.ws_down)


def run_stages(layer: Layer, path: str = "auto", router: str = "auto", k_policy: str = "exact",
               k_granule: int = 1) -> dict:
    """moe_route -> moe_permute -> moe_ffn -> moe_combine; returns host copies."""
    dev = layer.device
    desc = desc_of(layer, path, router, k_policy, k_granule)
    T, d, E, km = desc.T, desc.d, desc.E, desc.k_max
    i32 = dict(dtype=torch.int32, device=dev)
    tok_off = torch.full((T + 1,), -7, **i32)
    ids = torch.full((max(T * km, 1),), -7, **i32)
    w = torch.full((max(T * km, 1),), float("nan"), dtype=torch.float32, device=dev)
    status = torch.full((1,), -7, **i32)
    moe.moe_route(desc, layer.x, layer.w_router, layer.router_bias, layer.k, tok_off, ids, w, status,
                  moe.alloc_workspace(desc, moe.MOE_OP_ROUTE, dev))
    counts = torch.full((E,), -7, **i32)
    expert_off = torch.full((E + 1,), -7, **i32)
    perm_tok = torch.full((max(T * km, 1),), -7, **i32)
    perm_src = torch.full_like(perm_tok, -7)
    inv_perm = torch.full_like(perm_tok, -7)
    n_active = torch.full((1,), -7, **i32)
    moe.moe_permute(desc, tok_off, ids, counts, expert_off, perm_tok, perm_src, inv_perm, n_active,
                    moe.alloc_workspace(desc, moe.MOE_OP_PERMUTE, dev))
    y = torch.empty((max(T * km, 1), d), dtype=layer.x.dtype, device=dev)
    sh = shared_of(layer)
    y_sh = torch.empty((T, d), dtype=layer.x.dtype, device=dev) if sh else None
    moe.moe_ffn(desc, layer.x, layer.w_gate, layer.w_up, layer.w_down, *(sh or (None, None, None)),
                expert_off, perm_tok, y, y_sh, moe.alloc_workspace(desc, moe.MOE_OP_FFN, dev))
    out = torch.empty((T, d), dtype=layer.x.dtype, device=dev)
    moe.moe_combine(desc, y, y_sh, tok_off, w, inv_perm, out)
    torch.cuda.synchronize()
    A = int(tok_off[T].item())
    c = lambda t, n=None: (t[:n] if n is not None else t).cpu().numpy().astype(np.int64)
    return dict(tok_off=c(tok_off), ids=c(ids, A), w=w[:A].cpu().double().numpy(), status=int(status.item()),
                counts=c(counts), expert_off=c(expert_off), perm_tok=c(perm_tok, A),
                perm_src=c(perm_src, A), inv_perm=c(inv_perm, A), n_active=int(n_active.item()),
                out=out, A=A)


def run_forward(layer: Layer, path: str = "auto", router: str = "auto", k_policy: str = "exact",
                k_granule: int = 1):
    out, stats, status = moe.forward(layer.x, layer.w_router, layer.router_bias, layer.k, layer.w_gate,
                                     layer.w_up, layer.w_down, shared_of(layer), k_max=layer.cfg.k_max,
                                     routed_scale=layer.cfg.routed_scale, path=path, router=router,
                                     k_policy=k_policy, k_granule=k_granule)
    torch.cuda.synchronize()
    return out, stats.cpu().numpy().astype(np.int64), int(status.item())


def oracle_routing(layer: Layer, k_policy: str = "exact", k_granule: int = 1):
    c = layer.cfg
    ke, status = oracle.execution_budgets(to_f64(layer.k), c.k_max, k_policy, k_granule)
    r = oracle.route(to_f64(layer.x), to_f64(layer.w_router), to_f64(layer.router_bias), ke,
                     c.k_max, c.routed_scale, invalid="zero")
    r["status"] = status
    p = oracle.permute(r["tok_off"], r["ids"], layer.w_gate.shape[0])
    return r, p


def check_routing(got: dict, r: dict, p: dict) -> None:
    """Bit-exact integer routing and permutation; weights to float32 rounding."""
    assert got["status"] == r["status"]
    np.testing.assert_array_equal(got["tok_off"], r["tok_off"])
    np.testing.assert_array_equal(got["ids"], r["ids"])
    np.testing.assert_allclose(got["w"], r["w"], rtol=2e-6, atol=2e-7)
    for key in ("counts", "expert_off", "perm_tok", "perm_src", "inv_perm"):
        np.testing.assert_array_equal(got[key], p[key], err_msg=key)
    assert got["n_active"] == p["n_active"]


def oracle_out(layer: Layer, tokens, k_policy: str = "exact", k_granule: int = 1) -> np.ndarray:
    c = layer.cfg
    sh = None
    if layer.ws_gate is not None:
        sh = (to_f64(layer.ws_gate), to_f64(layer.ws_up), to_f64(layer.ws_down))
    ke, _ = oracle.execution_budgets(to_f64(layer.k), c.k_max, k_policy, k_granule)
    ref, _ = oracle.forward(to_f64(layer.x), to_f64(layer.w_router), to_f64(layer.router_bias),
                            ke, c.k_max, ExpertView(layer.w_gate), ExpertView(layer.w_up),
                            ExpertView(layer.w_down), shared=sh, routed_scale=c.routed_scale,
                            tokens=tokens, invalid="zero")
    return ref


def compare_out(got: torch.Tensor, ref: np.ndarray, dtype: str, tokens) -> dict:
    g = to_f64(got[torch.as_tensor(tokens, device=got.device)])
    err = g - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(err) / nref if nref > 0 else np.linalg.norm(err)
    mx = float(np.abs(err).max()) if err.size else 0.0
    tol = TOL[dtype]
    assert rel <= tol["rel_l2"], f"relative L2 error {rel:.3e} > {tol['rel_l2']}"
    if tol["max_abs"] is not None:
        assert mx <= tol["max_abs"], f"max abs error {mx:.3e} > {tol['max_abs']}"
    return dict(rel_l2=rel, max_abs=mx)


def sample_tokens(T: int, n: int) -> np.ndarray:
    """n tokens spread over the batch, always including the first and last."""
    if T <= n:
        return np.arange(T)
    return np.unique(np.linspace(0, T - 1, n).round().astype(np.int64))


def covering_tokens(got: dict, T: int, block: int = 64, shared: bool = False) -> np.ndarray:
    """Tokens whose outputs, taken together, touch every (expert, block of
    `block` permuted rows) at least once -- the row tiles of both FFN paths
    are unions of such blocks (64, 128 or 256 rows), so a fault confined to
    one row tile shows in some checked output row -- and, with `shared`, every
    `block`-token range of the always-on expert's rows.  Plus the first and
    the last token.  `got` is run_stages' host copy of the routing."""
    eoff, ptok = got["expert_off"], got["perm_tok"]
    chosen = {0, T - 1} if T > 0 else set()
    for e in range(len(eoff) - 1):
        for p0 in range(int(eoff[e]), int(eoff[e + 1]), block):
            chosen.add(int(ptok[p0]))
    if shared:
        chosen.update(range(0, T, block))
    return np.array(sorted(chosen), dtype=np.int64)


def compare_rows(a: torch.Tensor, b: torch.Tensor, dtype: str) -> dict:
    """Every row of two device outputs of the same layer against each other,
    to the output tolerance (rel. L2 over the whole output; max abs)."""
    a64, b64 = a.double(), b.double()
    diff = (a64 - b64)
    nref = float(torch.linalg.vector_norm(b64))
    rel = float(torch.linalg.vector_norm(diff)) / nref if nref > 0 else float(torch.linalg.vector_norm(diff))
    mx = float(diff.abs().max()) if diff.numel() else 0.0
    # per row as well: a fault confined to a few rows would vanish in the global norm
    rn = torch.linalg.vector_norm(diff, dim=1) / torch.linalg.vector_norm(b64, dim=1).clamp_min(1e-30)
    worst = float(rn.max()) if rn.numel() else 0.0
    tol = TOL[dtype]
    assert rel <= tol["rel_l2"], f"relative L2 error {rel:.3e} > {tol['rel_l2']}"
    assert worst <= 4 * tol["rel_l2"], f"worst row relative L2 error {worst:.3e}"
    if tol["max_abs"] is not None:
        assert mx <= tol["max_abs"], f"max abs error {mx:.3e} > {tol['max_abs']}"
    return dict(rel_l2=rel, worst_row=worst, max_abs=mx)

