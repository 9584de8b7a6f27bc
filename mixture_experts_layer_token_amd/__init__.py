"""MI355X-native MoE layer forward with a per-token routing top-k.

Thin Python binding over the C ABI of libmoe_mi355x.so (include/moe.h).  The
functions below only marshal arguments: torch tensors supply device memory and
the current HIP stream; every step of the layer runs in the HIP kernels.  If
the library has not been built, importing works but every call raises.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import (MOE_BF16, MOE_DEV_BAD_K, MOE_F32, MOE_OP_COMBINE, MOE_OP_FFN,  # noqa: F401
                   MOE_OP_FORWARD, MOE_OP_PERMUTE, MOE_OP_ROUTE, MOE_PATH_AUTO, MOE_PATH_GEMM,
                   MOE_PATH_STREAM, MOE_ROUTER_AUTO, MOE_ROUTER_FLOAT64, MOE_ROUTER_SCREENED, MOE_ROUTER_FUSED, MOE_K_EXACT,
                   MOE_K_BATCH_MAX, MOE_K_ROUND_UP, MOE_OP_FOLD, MOE_OP_PATH, MOE_FOLD_TOKEN, MOE_FOLD_POOL,
                   MOE_W_ROWMAJOR, MOE_W_BLOCKED64, moe_desc)

__all__ = [
    "MoeError", "make_desc", "pack_weights", "workspace_size", "resolve_path", "alloc_workspace", "moe_route", "moe_permute",
    "moe_ffn", "moe_ffn_plan", "moe_ffn_gateup", "moe_ffn_down", "moe_combine", "moe_fold", "moe_proxy_kappa_balanced",
    "moe_proxy_pack", "moe_path_table", "moe_path_route", "moe_path_sources", "moe_path_rows", "moe_ffn_down_rows",
    "PathLayer",
    "moe_proxy_route", "moe_forward", "moe_forward_noalloc",
    "forward", "proxy_width", "proxy_pack", "ProxyRouter", "probe_read",
    "library_path",
]

_DTYPES = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}
_PATHS = {"auto": MOE_PATH_AUTO, "stream": MOE_PATH_STREAM, "gemm": MOE_PATH_GEMM}
_ROUTERS = {"auto": MOE_ROUTER_AUTO, "float64": MOE_ROUTER_FLOAT64, "screened": MOE_ROUTER_SCREENED,
            "fused": MOE_ROUTER_FUSED}
_K_POLICIES = {"exact": MOE_K_EXACT, "batch_max": MOE_K_BATCH_MAX, "round_up": MOE_K_ROUND_UP}
_LAYOUTS = {"rowmajor": MOE_W_ROWMAJOR, "blocked": MOE_W_BLOCKED64}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = _lib.load()
        msg = lib.moe_status_str(status).decode()
        super().__init__(f"{fn}: {_lib.STATUS_NAMES.get(status, status)} ({msg})")
        self.status = status


def library_path() -> str:
    return _lib.LIB_PATH


def make_desc(T: int, d: int, E: int, I: int, k_max: int, *, I_shared: int = 0,
              dtype=torch.bfloat16, path: str = "auto", router: str = "auto",
              routed_scale: float = 1.0, k_policy: str = "exact", k_granule: int = 1,
              weight_layout: str = "rowmajor") -> moe_desc:
    """Layer descriptor.  k_policy: "exact" (each token runs its own k_t),
    "batch_max" (every valid token runs the batch's largest budget) or
    "round_up" (k_t rounded up to a multiple of k_granule).  weight_layout:
    "rowmajor" or "blocked" (expert weights converted by pack_weights)."""
    return moe_desc(T, d, E, I, k_max, I_shared, _DTYPES[dtype], _PATHS[path], _ROUTERS[router],
                    routed_scale, _K_POLICIES[k_policy], k_granule, _LAYOUTS[weight_layout])


def pack_weights(w: torch.Tensor, stream=None) -> torch.Tensor:
    """moe_pack_weights: a new tensor of w's shape ([G, N, K] or [N, K]) whose
    storage holds w's matrices in the blocked order (64-row x 128-byte blocks).
    Its elements are no longer addressed by (n, k) in torch terms; pass it to
    the entry points with weight_layout="blocked"."""
    if w.dim() not in (2, 3) or not w.is_contiguous():
        raise ValueError("pack_weights expects a contiguous [G, N, K] or [N, K] tensor")
    G = w.shape[0] if w.dim() == 3 else 1
    N, K = w.shape[-2], w.shape[-1]
    out = torch.empty_like(w)
    _check("moe_pack_weights", _lib.load().moe_pack_weights(
        _DTYPES[w.dtype], G, N, K, _dev(w, "w"), _dev(out, "out"), _stream(stream)))
    return out


def _ptr(t: Optional[torch.Tensor]):
    """Address of a host tensor (the host-side arguments of moe_path_table and
    moe_proxy_kappa_balanced)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("host argument must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


_ELT = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16}


def _elt(desc: moe_desc) -> torch.dtype:
    return _ELT[desc.dtype]


def _dev(t: Optional[torch.Tensor], name: str, dtype: Optional[torch.dtype] = None, numel: Optional[int] = None):
    """Address of a device argument, after checking what the C ABI cannot:
    a contiguous tensor on a GPU, of the element type the call reads, holding
    at least `numel` elements.  (An int64 budget vector passed as int32, for
    instance, would otherwise be read as pairs of 32-bit halves.)"""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, at least {numel} needed")
    return ctypes.c_void_p(t.data_ptr())


_I32, _F32 = torch.int32, torch.float32




def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MoeError(fn, status)


def workspace_size(desc: moe_desc, op: int = MOE_OP_FORWARD) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_workspace_size", _lib.load().moe_workspace_size(ctypes.byref(desc), op, ctypes.byref(n)))
    return n.value


def resolve_path(desc: moe_desc):
    """(routed, shared) FFN path names that desc.path resolves to."""
    r, sh = ctypes.c_int32(0), ctypes.c_int32(0)
    _check("moe_resolve_path", _lib.load().moe_resolve_path(ctypes.byref(desc), ctypes.byref(r), ctypes.byref(sh)))
    names = {MOE_PATH_STREAM: "stream", MOE_PATH_GEMM: "gemm"}
    return names[r.value], names[sh.value]


def alloc_workspace(desc: moe_desc, op: int = MOE_OP_FORWARD, device="cuda") -> Optional[torch.Tensor]:
    n = workspace_size(desc, op)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def moe_route(desc, x, w_router, router_bias, k, tok_off, topk_ids, topk_w, dev_status, ws,
              stream=None) -> None:
    T, d, E, el = desc.T, desc.d, desc.E, _elt(desc)
    _check("moe_route", _lib.load().moe_route(
        ctypes.byref(desc), _dev(x, "x", el, T * d), _dev(w_router, "w_router", el, E * d),
        _dev(router_bias, "router_bias", _F32, E), _dev(k, "k", _I32, T), _dev(tok_off, "tok_off", _I32, T + 1),
        _dev(topk_ids, "topk_ids", _I32), _dev(topk_w, "topk_w", _F32), _dev(dev_status, "dev_status", _I32, 1),
        _dev(ws, "ws"), _nbytes(ws), _stream(stream)))


def moe_permute(desc, tok_off, topk_ids, expert_counts, expert_off, perm_tok, perm_src, inv_perm,
                n_active, ws, stream=None) -> None:
    T, E = desc.T, desc.E
    _check("moe_permute", _lib.load().moe_permute(
        ctypes.byref(desc), _dev(tok_off, "tok_off", _I32, T + 1), _dev(topk_ids, "topk_ids", _I32),
        _dev(expert_counts, "expert_counts", _I32, E), _dev(expert_off, "expert_off", _I32, E + 1),
        _dev(perm_tok, "perm_tok", _I32), _dev(perm_src, "perm_src", _I32), _dev(inv_perm, "inv_perm", _I32),
        _dev(n_active, "n_active", _I32, 1), _dev(ws, "ws"), _nbytes(ws), _stream(stream)))


def moe_ffn(desc, x, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, expert_off, perm_tok, y_perm,
            y_shared, ws, stream=None) -> None:
    T, d, E, I, Is, el = desc.T, desc.d, desc.E, desc.I, desc.I_shared, _elt(desc)
    _check("moe_ffn", _lib.load().moe_ffn(
        ctypes.byref(desc), _dev(x, "x", el, T * d), _dev(w_gate, "w_gate", el, E * I * d),
        _dev(w_up, "w_up", el, E * I * d), _dev(w_down, "w_down", el, E * d * I), _dev(ws_gate, "ws_gate", el, Is * d),
        _dev(ws_up, "ws_up", el, Is * d), _dev(ws_down, "ws_down", el, d * Is), _dev(expert_off, "expert_off", _I32, E + 1),
        _dev(perm_tok, "perm_tok", _I32), _dev(y_perm, "y_perm", el), _dev(y_shared, "y_shared", el, T * d),
        _dev(ws, "ws"), _nbytes(ws), _stream(stream)))


def moe_ffn_plan(desc, expert_off, ws, stream=None) -> None:
    _check("moe_ffn_plan", _lib.load().moe_ffn_plan(
        ctypes.byref(desc), _dev(expert_off, "expert_off", _I32, desc.E + 1), _dev(ws, "ws"), _nbytes(ws),
        _stream(stream)))


def moe_ffn_gateup(desc, x, w_gate, w_up, expert_off, perm_tok, h, ws=None, stream=None) -> None:
    T, d, E, I, el = desc.T, desc.d, desc.E, desc.I, _elt(desc)
    _check("moe_ffn_gateup", _lib.load().moe_ffn_gateup(
        ctypes.byref(desc), _dev(x, "x", el, T * d), _dev(w_gate, "w_gate", el, E * I * d),
        _dev(w_up, "w_up", el, E * I * d), _dev(expert_off, "expert_off", _I32, E + 1),
        _dev(perm_tok, "perm_tok", _I32), _dev(h, "h", el), _dev(ws, "ws"), _nbytes(ws), _stream(stream)))


def moe_ffn_down(desc, h, w_down, expert_off, y_perm, ws=None, stream=None) -> None:
    d, E, I, el = desc.d, desc.E, desc.I, _elt(desc)
    _check("moe_ffn_down", _lib.load().moe_ffn_down(
        ctypes.byref(desc), _dev(h, "h", el), _dev(w_down, "w_down", el, E * d * I),
        _dev(expert_off, "expert_off", _I32, E + 1), _dev(y_perm, "y_perm", el), _dev(ws, "ws"),
        _nbytes(ws), _stream(stream)))


_FOLD_MODES = {"token": MOE_FOLD_TOKEN, "pool": MOE_FOLD_POOL}


def moe_fold(desc, mode: str, budget: int, S, L, H, tok_off, topk_ids, topk_w, expert_off, perm_src,
             tok_off_out, ids_out, w_out, pool_out, ws, stream=None) -> None:
    """mode "token" (at most `budget` routes per token) or "pool" (a pool of
    `budget` experts; expert_off / perm_src of moe_permute on the input routes)."""
    _check("moe_fold", _lib.load().moe_fold(
        ctypes.byref(desc), _FOLD_MODES[mode], budget, _dev(S, "S", _F32), _dev(L, "L", _F32), _dev(H, "H", _F32),
        _dev(tok_off, "tok_off", _I32, desc.T + 1), _dev(topk_ids, "topk_ids", _I32), _dev(topk_w, "topk_w", _F32),
        _dev(expert_off, "expert_off", _I32), _dev(perm_src, "perm_src", _I32),
        _dev(tok_off_out, "tok_off_out", _I32, desc.T + 1), _dev(ids_out, "ids_out", _I32), _dev(w_out, "w_out", _F32),
        _dev(pool_out, "pool_out", _I32), _dev(ws, "ws"), _nbytes(ws), _stream(stream)))


def moe_proxy_kappa_balanced(k_max: int, m: int, N: int) -> torch.Tensor:
    """int32 [k_max+1][m] CPU tensor: each budget split evenly over the m
    whole-expert picks, the remainder to the earlier picks."""
    kappa = torch.empty((k_max + 1, m), dtype=torch.int32)
    _check("moe_proxy_kappa_balanced", _lib.load().moe_proxy_kappa_balanced(k_max, m, N, _ptr(kappa)))
    return kappa


def moe_proxy_pack(desc, N: int, r: int, gate_idx, w_gate, w_up, wp_gate, wp_up, stream=None) -> None:
    _check("moe_proxy_pack", _lib.load().moe_proxy_pack(
        ctypes.byref(desc), N, r, _dev(gate_idx, "gate_idx", _I32), _dev(w_gate, "w_gate", _elt(desc)),
        _dev(w_up, "w_up", _elt(desc)), _dev(wp_gate, "wp_gate", _elt(desc)), _dev(wp_up, "wp_up", _elt(desc)),
        _stream(stream)))


def moe_proxy_route(desc, N: int, r: int, m: int, k, kappa, base_tok_off, base_ids, base_w, base_expert_off,
                    base_perm_tok, base_perm_src, x, wp_gate, wp_up, tok_off, topk_ids, topk_w, dev_status,
                    stream=None) -> None:
    _check("moe_proxy_route", _lib.load().moe_proxy_route(
        ctypes.byref(desc), N, r, m, _dev(k, "k", _I32, desc.T), _dev(kappa, "kappa", _I32),
        _dev(base_tok_off, "base_tok_off", _I32), _dev(base_ids, "base_ids", _I32), _dev(base_w, "base_w", _F32),
        _dev(base_expert_off, "base_expert_off", _I32), _dev(base_perm_tok, "base_perm_tok", _I32),
        _dev(base_perm_src, "base_perm_src", _I32), _dev(x, "x", _elt(desc)), _dev(wp_gate, "wp_gate", _elt(desc)), _dev(wp_up, "wp_up", _elt(desc)),
        _dev(tok_off, "tok_off", _I32, desc.T + 1),
        _dev(topk_ids, "topk_ids", _I32), _dev(topk_w, "topk_w", _F32), _dev(dev_status, "dev_status", _I32),
        _stream(stream)))


def moe_combine(desc, y_perm, y_shared, tok_off, topk_w, inv_perm, out, stream=None) -> None:
    T, d, el = desc.T, desc.d, _elt(desc)
    _check("moe_combine", _lib.load().moe_combine(
        ctypes.byref(desc), _dev(y_perm, "y_perm", el), _dev(y_shared, "y_shared", el, T * d),
        _dev(tok_off, "tok_off", _I32, T + 1), _dev(topk_w, "topk_w", _F32), _dev(inv_perm, "inv_perm", _I32),
        _dev(out, "out", el, T * d), _stream(stream)))


def probe_read(src: torch.Tensor, sink: torch.Tensor, nontemporal: bool = False, stream=None) -> None:
    """moe_probe_read over all of `src` (a contiguous device tensor; `sink`:
    an int32 device tensor of one element): the streaming-read probe the
    benchmark times as the practical HBM ceiling."""
    _check("moe_probe_read", _lib.load().moe_probe_read(
        _dev(src, "src"), src.numel() * src.element_size(), 1 if nontemporal else 0, _dev(sink, "sink", _I32, 1),
        _stream(stream)))


def moe_forward(desc, x, w_router, router_bias, k, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
                out, stats, dev_status, ws, stream=None) -> None:
    T, d, E, I, Is, el = desc.T, desc.d, desc.E, desc.I, desc.I_shared, _elt(desc)
    _check("moe_forward", _lib.load().moe_forward(
        ctypes.byref(desc), _dev(x, "x", el, T * d), _dev(w_router, "w_router", el, E * d),
        _dev(router_bias, "router_bias", _F32, E), _dev(k, "k", _I32, T), _dev(w_gate, "w_gate", el, E * I * d),
        _dev(w_up, "w_up", el, E * I * d), _dev(w_down, "w_down", el, E * d * I), _dev(ws_gate, "ws_gate", el, Is * d),
        _dev(ws_up, "ws_up", el, Is * d), _dev(ws_down, "ws_down", el, d * Is), _dev(out, "out", el, T * d),
        _dev(stats, "stats", _I32, E + 2), _dev(dev_status, "dev_status", _I32, 1), _dev(ws, "ws"), _nbytes(ws),
        _stream(stream)))


def moe_forward_noalloc(desc, x, w_router, router_bias, k, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
                        out, stats, dev_status, stream=None) -> None:
    """moe_forward with the library-held scratch array (no workspace argument;
    for callers that cannot allocate device memory)."""
    T, d, E, I, Is, el = desc.T, desc.d, desc.E, desc.I, desc.I_shared, _elt(desc)
    _check("moe_forward_noalloc", _lib.load().moe_forward_noalloc(
        ctypes.byref(desc), _dev(x, "x", el, T * d), _dev(w_router, "w_router", el, E * d),
        _dev(router_bias, "router_bias", _F32, E), _dev(k, "k", _I32, T), _dev(w_gate, "w_gate", el, E * I * d),
        _dev(w_up, "w_up", el, E * I * d), _dev(w_down, "w_down", el, E * d * I), _dev(ws_gate, "ws_gate", el, Is * d),
        _dev(ws_up, "ws_up", el, Is * d), _dev(ws_down, "ws_down", el, d * Is), _dev(out, "out", el, T * d),
        _dev(stats, "stats", _I32, E + 2), _dev(dev_status, "dev_status", _I32, 1), _stream(stream)))


def forward(x: torch.Tensor, w_router: torch.Tensor, router_bias: Optional[torch.Tensor],
            k: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
            shared: Optional[Sequence[torch.Tensor]] = None, *, k_max: int, routed_scale: float = 1.0,
            path: str = "auto", router: str = "auto", k_policy: str = "exact", k_granule: int = 1,
            weight_layout: str = "rowmajor", ws: Optional[torch.Tensor] = None, stream=None):
    """Allocate the outputs (and a workspace unless given) and run moe_forward.
    Returns (out [T, d], stats int32 [E+2] = counts, n_active, A, dev_status int32 [1])."""
    T, d = x.shape
    E, I, _ = w_gate.shape
    Is = shared[0].shape[0] if shared is not None else 0
    desc = make_desc(T, d, E, I, k_max, I_shared=Is, dtype=x.dtype, path=path, router=router,
                     routed_scale=routed_scale, k_policy=k_policy, k_granule=k_granule,
                     weight_layout=weight_layout)
    if ws is None:
        ws = alloc_workspace(desc, MOE_OP_FORWARD, x.device)
    out = torch.empty((T, d), dtype=x.dtype, device=x.device)
    stats = torch.empty(E + 2, dtype=torch.int32, device=x.device)
    status = torch.empty(1, dtype=torch.int32, device=x.device)
    sg, su, sd = shared if shared is not None else (None, None, None)
    moe_forward(desc, x, w_router, router_bias, k, w_gate, w_up, w_down, sg, su, sd, out, stats,
                status, ws, stream)
    return out, stats, status


def proxy_width(N: int, r: int) -> int:
    """Rows of one whole expert's packed proxy weights: N*r rounded up to 128."""
    return (N * r + 127) // 128 * 128


def proxy_pack(w_gate: torch.Tensor, w_up: torch.Tensor, gate_idx: torch.Tensor, N: int, stream=None,
               weight_layout: str = "rowmajor"):
    """Allocate and fill the packed proxy weights (wp_gate, wp_up), each
    [E/N, Ip, d], of a split layer with sub-expert weights [E, I, d] (input
    and output in `weight_layout`)."""
    E, I, d = w_gate.shape
    r = gate_idx.shape[1]
    desc = make_desc(0, d, E, I, 1, dtype=w_gate.dtype, weight_layout=weight_layout)
    Ip = proxy_width(N, r)
    wp_g = torch.empty((E // N, Ip, d), dtype=w_gate.dtype, device=w_gate.device)
    wp_u = torch.empty_like(wp_g)
    moe_proxy_pack(desc, N, r, gate_idx, w_gate, w_up, wp_g, wp_u, stream)
    return wp_g, wp_u


class ProxyRouter:
    """Buffers and calls of proxy-gated routing for a fixed shape: the
    whole-expert router (moe_route with every k_t = m), its permutation, and
    moe_proxy_route, which scores the picks' sub-experts from x and the packed
    weights.
    ``run`` only launches (no allocation), so it can be captured in a HIP
    graph."""

    def __init__(self, desc: moe_desc, N: int, r: int, m: int, kappa: torch.Tensor, device="cuda"):
        self.desc, self.N, self.r, self.m = desc, N, r, m
        T, d = desc.T, desc.d
        self.Ip = proxy_width(N, r)
        dtype = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16}[desc.dtype]
        self.base = make_desc(T, d, desc.E // N, self.Ip, m, dtype=dtype, routed_scale=desc.routed_scale)
        self.base.weight_layout = desc.weight_layout
        i32 = dict(dtype=torch.int32, device=device)
        A = max(T * m, 1)
        self.kappa = kappa.to(device=device, dtype=torch.int32).contiguous()
        self.k_base = torch.full((max(T, 1),), m, **i32)
        self.b_tok_off = torch.empty(T + 1, **i32)
        self.b_ids = torch.empty(A, **i32)
        self.b_w = torch.empty(A, dtype=torch.float32, device=device)
        self.b_status = torch.empty(1, **i32)
        self.b_counts = torch.empty(self.base.E, **i32)
        self.b_eoff = torch.empty(self.base.E + 1, **i32)
        self.b_ptok = torch.empty(A, **i32)
        self.b_psrc = torch.empty(A, **i32)
        self.b_inv = torch.empty(A, **i32)
        self.b_nact = torch.empty(1, **i32)
        self.ws_route = alloc_workspace(self.base, MOE_OP_ROUTE, device)
        self.ws_perm = alloc_workspace(self.base, MOE_OP_PERMUTE, device)
        km = desc.k_max
        self.tok_off = torch.empty(T + 1, **i32)
        self.ids = torch.empty(max(T * km, 1), **i32)
        self.w = torch.empty(max(T * km, 1), dtype=torch.float32, device=device)
        self.status = torch.empty(1, **i32)

    def run(self, x, w_router_base, router_bias, k, wp_gate, wp_up, stream=None):
        b = self.base
        moe_route(b, x, w_router_base, router_bias, self.k_base, self.b_tok_off, self.b_ids, self.b_w,
                  self.b_status, self.ws_route, stream)
        moe_permute(b, self.b_tok_off, self.b_ids, self.b_counts, self.b_eoff, self.b_ptok, self.b_psrc,
                    self.b_inv, self.b_nact, self.ws_perm, stream)
        moe_proxy_route(self.desc, self.N, self.r, self.m, k, self.kappa, self.b_tok_off, self.b_ids, self.b_w,
                        self.b_eoff, self.b_ptok, self.b_psrc, x, wp_gate, wp_up, self.tok_off, self.ids, self.w,
                        self.status, stream)
        return self.tok_off, self.ids, self.w, self.status


def moe_path_table(E: int, src, tgt, bias, device="cuda", stream=None) -> torch.Tensor:
    """Validate the active path list (host sequences, strictly increasing
    (src, tgt)) and upload it; returns the device table (uint8 tensor)."""
    P = len(src)
    n = ctypes.c_size_t(0)
    _check("moe_path_table_bytes", _lib.load().moe_path_table_bytes(P, ctypes.byref(n)))
    s = torch.as_tensor(src, dtype=torch.int32).contiguous()
    t = torch.as_tensor(tgt, dtype=torch.int32).contiguous()
    b = torch.as_tensor(bias, dtype=torch.float32).contiguous()
    table = torch.empty(n.value, dtype=torch.uint8, device=device)
    _check("moe_path_table", _lib.load().moe_path_table(E, P, _ptr(s), _ptr(t), _ptr(b), _dev(table, "table"), n.value,
                                                         _stream(stream)))
    return table


def moe_path_route(desc, x, w_router, router_bias, w_tgt, lam: float, table, P: int, k, tok_off, path_src, path_tgt,
                   path_w, dev_status, ws, stream=None) -> None:
    _check("moe_path_route", _lib.load().moe_path_route(
        ctypes.byref(desc), _dev(x, "x", _elt(desc)), _dev(w_router, "w_router", _elt(desc)),
        _dev(router_bias, "router_bias", _F32), _dev(w_tgt, "w_tgt", _elt(desc)), lam, _dev(table, "table"), P,
        _dev(k, "k", _I32, desc.T), _dev(tok_off, "tok_off", _I32, desc.T + 1), _dev(path_src, "path_src", _I32),
        _dev(path_tgt, "path_tgt", _I32), _dev(path_w, "path_w", _F32), _dev(dev_status, "dev_status", _I32),
        _dev(ws, "ws"), _nbytes(ws),
        _stream(stream)))


def moe_path_sources(desc, tok_off, path_src, src_tok_off, src_ids, path_src_route, unit_off, ws,
                     stream=None) -> None:
    _check("moe_path_sources", _lib.load().moe_path_sources(
        ctypes.byref(desc), _dev(tok_off, "tok_off", _I32), _dev(path_src, "path_src", _I32),
        _dev(src_tok_off, "src_tok_off", _I32), _dev(src_ids, "src_ids", _I32),
        _dev(path_src_route, "path_src_route", _I32), _dev(unit_off, "unit_off", _I32), _dev(ws, "ws"), _nbytes(ws),
        _stream(stream)))


def moe_path_rows(desc, tok_off, perm_path, path_src_route, src_inv_perm, row_map, stream=None) -> None:
    _check("moe_path_rows", _lib.load().moe_path_rows(
        ctypes.byref(desc), _dev(tok_off, "tok_off", _I32), _dev(perm_path, "perm_path", _I32),
        _dev(path_src_route, "path_src_route", _I32), _dev(src_inv_perm, "src_inv_perm", _I32),
        _dev(row_map, "row_map", _I32),
        _stream(stream)))


def moe_ffn_down_rows(desc, h, row_map, w_down, expert_off, y_perm, ws, stream=None) -> None:
    _check("moe_ffn_down_rows", _lib.load().moe_ffn_down_rows(
        ctypes.byref(desc), _dev(h, "h", _elt(desc)), _dev(row_map, "row_map", _I32), _dev(w_down, "w_down", _elt(desc)),
        _dev(expert_off, "expert_off", _I32), _dev(y_perm, "y_perm", _elt(desc)), _dev(ws, "ws"),
        _nbytes(ws), _stream(stream)))


class PathLayer:
    """Buffers and calls of the compositional-path layer for a fixed shape:
    path routing, source groups, the expansions over the source routes
    (permute + gate/up), the projections over the paths grouped by target
    (one-per-row permute, row map, down with row gather) and the combine.
    ``run`` only launches (no allocation), so it can be captured in a graph."""

    def __init__(self, desc: moe_desc, table: torch.Tensor, P: int, lam: float = 0.0, device="cuda"):
        self.desc, self.table, self.P, self.lam = desc, table, P, float(lam)
        T, d, E, I, km = desc.T, desc.d, desc.E, desc.I, desc.k_max
        dtype = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16}[desc.dtype]
        # the paths one per row: T*k_max "tokens" of one route each
        self.unit = moe_desc(T * km, d, E, I, 1, 0, desc.dtype, desc.path, desc.router, desc.routed_scale,
                             MOE_K_EXACT, 1, desc.weight_layout)
        i32 = dict(dtype=torch.int32, device=device)
        A = max(T * km, 1)
        self.tok_off = torch.empty(T + 1, **i32)
        self.src = torch.empty(A, **i32)
        self.tgt = torch.empty(A, **i32)
        self.w = torch.empty(A, dtype=torch.float32, device=device)
        self.status = torch.empty(1, **i32)
        self.src_off = torch.empty(T + 1, **i32)
        self.src_ids = torch.empty(A, **i32)
        self.p2s = torch.empty(A, **i32)
        self.unit_off = torch.empty(T * km + 1, **i32)
        self.s_counts, self.t_counts = torch.empty(E, **i32), torch.empty(E, **i32)
        self.s_eoff, self.t_eoff = torch.empty(E + 1, **i32), torch.empty(E + 1, **i32)
        self.s_ptok, self.s_psrc, self.s_inv = (torch.empty(A, **i32) for _ in range(3))
        self.t_ptok, self.t_psrc, self.t_inv = (torch.empty(A, **i32) for _ in range(3))
        self.s_nact, self.t_nact = torch.empty(1, **i32), torch.empty(1, **i32)
        self.row_map = torch.empty(A, **i32)
        self.h = torch.empty((A, I), dtype=dtype, device=device)
        self.y = torch.empty((A, d), dtype=dtype, device=device)
        # the always-on shared expert: moe_ffn over an empty routed set
        self.zero_eoff = torch.zeros(E + 1, **i32)
        self.y_sh = torch.empty((max(T, 1), d), dtype=dtype, device=device) if desc.I_shared else None
        self.ws_path = alloc_workspace(desc, MOE_OP_PATH, device)
        self.ws_perm = alloc_workspace(desc, MOE_OP_PERMUTE, device)
        self.ws_uperm = alloc_workspace(self.unit, MOE_OP_PERMUTE, device)
        self.ws_ffn = alloc_workspace(desc, MOE_OP_FFN, device)

    def run(self, x, w_router, router_bias, w_tgt, k, w_gate, w_up, w_down, out, shared=None, stream=None):
        """shared = (ws_gate, ws_up, ws_down) when the descriptor has I_shared > 0."""
        d, u = self.desc, self.unit
        if d.I_shared and shared is None:
            raise ValueError("the descriptor has a shared expert: pass its weights")
        moe_path_route(d, x, w_router, router_bias, w_tgt, self.lam, self.table, self.P, k, self.tok_off, self.src,
                       self.tgt, self.w, self.status, self.ws_path, stream)
        moe_path_sources(d, self.tok_off, self.src, self.src_off, self.src_ids, self.p2s, self.unit_off,
                         self.ws_path, stream)
        moe_permute(d, self.src_off, self.src_ids, self.s_counts, self.s_eoff, self.s_ptok, self.s_psrc, self.s_inv,
                    self.s_nact, self.ws_perm, stream)
        moe_ffn_plan(d, self.s_eoff, self.ws_ffn, stream)
        moe_ffn_gateup(d, x, w_gate, w_up, self.s_eoff, self.s_ptok, self.h, self.ws_ffn, stream)
        moe_permute(u, self.unit_off, self.tgt, self.t_counts, self.t_eoff, self.t_ptok, self.t_psrc, self.t_inv,
                    self.t_nact, self.ws_uperm, stream)
        moe_path_rows(d, self.tok_off, self.t_ptok, self.p2s, self.s_inv, self.row_map, stream)
        moe_ffn_plan(u, self.t_eoff, self.ws_ffn, stream)
        moe_ffn_down_rows(u, self.h, self.row_map, w_down, self.t_eoff, self.y, self.ws_ffn, stream)
        if d.I_shared:
            moe_ffn(d, x, w_gate, w_up, w_down, *shared, self.zero_eoff, self.s_ptok, self.y, self.y_sh, self.ws_ffn,
                    stream)
        moe_combine(d, self.y, self.y_sh if d.I_shared else None, self.tok_off, self.w, self.t_inv, out, stream)
