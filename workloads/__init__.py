"""Seeded synthetic MoE layers: the one input source shared by the oracle and
the HIP path.

This module holds no arithmetic of the layer itself (no routing, no FFN, no
combine).  It only draws inputs: hidden states, router weights, stacked expert
weights, an optional router bias and the per-token top-k vector, with the
shapes and value distributions of the workloads below.

The pages measure on serving traces and datasets (an Azure request trace,
8,192-token prefill prompts, 32-token decode batches); none ships here, so
these seeded Gaussian layers stand in for them, shaped like the models the
pages serve (Mixtral, Qwen3-30B-A3B, a MoE-Prism sub-expert layer and a
DeepSeek-V3-shaped layer).

Generation rules
----------------
* Every tensor, and every expert of a stacked tensor, is drawn from its own
  ``torch.Generator`` seeded by :func:`derived_seed`, so a layer can be drawn
  expert by expert without holding fp32 copies of all weights.
* Gaussians are drawn in fp32 and, for bf16 layers, rounded to bf16 with
  round-to-nearest-even (torch's ``.to(torch.bfloat16)``).  Both sides of a
  parity test see the same bits.
* Init scale: x ~ N(0, 1); router and gate/up weights ~ N(0, 1/d); down
  weights ~ N(0, 1/fan_in) where fan_in is the (base) expert's intermediate
  size.
* The Zipf(1.1) router bias is b_e = -1.1 * ln(e + 1) (fp32): a prior
  proportional to rank^-1.1 with expert 0 the most popular, added to the
  logits before selection.
* The sub-expert layer follows MoE-Prism (arXiv 2510.19366) §III-B1, Eq. (3):
  each base expert of intermediate size C is cut into N contiguous, equal
  neuron slices S_n = [n*C/N, (n+1)*C/N); sub-expert N*j + n holds the rows
  S_n of base expert j's gate/up matrices and the columns S_n of its down
  matrix.
* Per-token k is drawn from the workload's discrete law with its own
  generator (the request-level budget of MoE-Prism §III-C1; one request per
  decode token).

Layouts (row-major, the ``nn.Linear`` [out, in] convention):
  x [T, d], w_router [E, d], router_bias [E] fp32 or None, k [T] int32,
  w_gate [E, I, d], w_up [E, I, d], w_down [E, d, I],
  ws_gate [Is, d], ws_up [Is, d], ws_down [d, Is] (shared expert, or None).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

__all__ = [
    "LayerConfig",
    "Layer",
    "CONFIGS",
    "derived_seed",
    "make_layer",
    "make_tokens",
    "make_custom_layer",
    "to_f64",
    "torch_dtype",
    "ExpertView",
    "draw_k_eq7",
    "make_fold_tables",
    "make_proxy_inputs",
    "make_path_mask",
    "make_target_router",
]


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """Shape and distribution recipe of one synthetic MoE layer."""

    name: str
    dtype: str                      # "f32" or "bf16"
    T: int                          # tokens in the batch
    d: int                          # hidden size
    E: int                          # routed experts (sub-experts after a split)
    I: int                          # routed expert intermediate size
    k_values: Sequence[int]         # support of the per-token k law
    k_probs: Sequence[float]        # its probabilities
    k_max: int                      # bound the layer is configured with
    I_shared: int = 0               # always-on shared expert, 0 = none
    zipf_bias: float = 0.0          # s of the Zipf(s) router bias, 0 = none
    split: int = 1                  # sub-experts per base expert
    routed_scale: float = 1.0
    seed: int = 0

    @property
    def E_base(self) -> int:
        return self.E // self.split

    @property
    def I_base(self) -> int:
        return self.I * self.split

    def with_(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


# The five workloads (the DeepSeek-V3-shaped one at two batch sizes).
CONFIGS = {
    # Tiny fp32 layer: fixed top-2 over 8 experts.
    "tiny_fp32": LayerConfig("tiny_fp32", "f32", T=16, d=256, E=8, I=512,
                             k_values=(2,), k_probs=(1.0,), k_max=2),
    # Mixtral-8x7B-shaped decode layer: 64 one-token requests, top-2.
    "mixtral_decode": LayerConfig("mixtral_decode", "bf16", T=64, d=4096, E=8,
                                  I=14336, k_values=(2,), k_probs=(1.0,),
                                  k_max=2),
    # Qwen3-30B-A3B-shaped decode layer with Zipf(1.1)-skewed expert
    # popularity and k ~ U{2,4,6,8}.
    "qwen3_30b_a3b_decode": LayerConfig(
        "qwen3_30b_a3b_decode", "bf16", T=256, d=2048, E=128, I=768,
        k_values=(2, 4, 6, 8), k_probs=(0.25, 0.25, 0.25, 0.25), k_max=8,
        zipf_bias=1.1),
    # MoE-Prism-style sub-expert prefill layer: 64 base experts of I=1536,
    # each cut into 4 contiguous sub-experts (E=256, I=384).
    "subexpert_prefill": LayerConfig(
        "subexpert_prefill", "bf16", T=8192, d=2048, E=256, I=384,
        k_values=(8, 16, 24, 32), k_probs=(0.4, 0.3, 0.2, 0.1), k_max=32,
        split=4),
    # DeepSeek-V3-shaped layer on one GPU: 256 routed experts + 1 shared.
    "dsv3_decode": LayerConfig(
        "dsv3_decode", "bf16", T=128, d=7168, E=256, I=2048,
        k_values=(4, 8), k_probs=(0.5, 0.5), k_max=8, I_shared=2048),
    "dsv3_prefill": LayerConfig(
        "dsv3_prefill", "bf16", T=4096, d=7168, E=256, I=2048,
        k_values=(4, 8), k_probs=(0.5, 0.5), k_max=8, I_shared=2048),
}

_TENSOR_IDS = {
    "x": 1, "w_router": 2, "k": 3, "w_gate": 4, "w_up": 5, "w_down": 6,
    "ws_gate": 7, "ws_up": 8, "ws_down": 9,
}


def derived_seed(seed: int, tensor: str, index: int = 0) -> int:
    """Seed of one tensor (or one expert slice of it): a fixed mixing of
    (layer seed, tensor id, expert index) into 63 bits."""
    h = (seed * 0x9E3779B97F4A7C15 + _TENSOR_IDS[tensor] * 0xBF58476D1CE4E5B9
         + (index + 1) * 0x94D049BB133111EB) & ((1 << 64) - 1)
    h ^= h >> 31
    h = (h * 0xD6E8FEB86659FD93) & ((1 << 64) - 1)
    h ^= h >> 32
    return h & ((1 << 63) - 1)


def torch_dtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def _gauss(shape, std: float, seed: int, device, dtype: torch.dtype) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


@dataclasses.dataclass
class Layer:
    """One drawn layer.  Tensors live on ``device``; ``cfg`` is the recipe."""

    cfg: LayerConfig
    x: torch.Tensor
    w_router: torch.Tensor
    router_bias: Optional[torch.Tensor]
    k: torch.Tensor
    w_gate: torch.Tensor
    w_up: torch.Tensor
    w_down: torch.Tensor
    ws_gate: Optional[torch.Tensor] = None
    ws_up: Optional[torch.Tensor] = None
    ws_down: Optional[torch.Tensor] = None

    @property
    def device(self) -> torch.device:
        return self.x.device

    def to(self, device) -> "Layer":
        mv = lambda t: None if t is None else t.to(device)
        return Layer(self.cfg, mv(self.x), mv(self.w_router), mv(self.router_bias),
                     mv(self.k), mv(self.w_gate), mv(self.w_up), mv(self.w_down),
                     mv(self.ws_gate), mv(self.ws_up), mv(self.ws_down))


def draw_k(cfg: LayerConfig, T: Optional[int] = None) -> torch.Tensor:
    """Per-token budgets k_t drawn i.i.d. from the workload's discrete law."""
    T = cfg.T if T is None else T
    g = torch.Generator(device="cpu")
    g.manual_seed(derived_seed(cfg.seed, "k"))
    if len(cfg.k_values) == 1 or T == 0:
        return torch.full((T,), int(cfg.k_values[0]), dtype=torch.int32)
    probs = torch.tensor(cfg.k_probs, dtype=torch.float64)
    idx = torch.multinomial(probs, T, replacement=True, generator=g)
    vals = torch.tensor(cfg.k_values, dtype=torch.int32)
    return vals[idx]


def draw_k_eq7(T: int, mu: float, sigma: float, k_max: int, seed: int) -> torch.Tensor:
    """Budgets from a rounded, clipped normal law (MoE-Prism, arXiv 2510.19366,
    §IV-B2, Eq. (7)): k = clip(round(x), 1, k_max), x ~ N(mu, sigma^2), i.i.d.
    per token.  Rounding is half to even (numpy/torch round)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(derived_seed(seed, "k", 7))
    x = mu + sigma * torch.randn(T, generator=g, dtype=torch.float64)
    return torch.clamp(torch.round(x), 1, k_max).to(torch.int32)


def make_fold_tables(E: int, seed: int = 0):
    """Synthetic stand-ins for the calibrated folding tables of ExFold (the
    calibrated ones need a model and data): scalar projectors S [E][E] drawn
    from N(1, 0.25^2) and clipped to [-4, 4] with S[e][e] = 1, projection
    losses L [E][E] uniform in [0, 1) with L[e][e] = 0, output magnitudes H [E]
    uniform in [0.5, 2).  float32, CPU tensors."""
    g = torch.Generator(device="cpu")
    g.manual_seed(derived_seed(seed, "k", 11))
    S = torch.clamp(1.0 + 0.25 * torch.randn(E, E, generator=g), -4.0, 4.0)
    S.fill_diagonal_(1.0)
    L = torch.rand(E, E, generator=g)
    L.fill_diagonal_(0.0)
    H = 0.5 + 1.5 * torch.rand(E, generator=g)
    return S.float(), L.float(), H.float()


def zipf_bias(E: int, s: float) -> torch.Tensor:
    """b_e = -s * ln(e + 1) in fp32 (expert 0 most popular)."""
    return torch.tensor([-s * math.log(e + 1) for e in range(E)], dtype=torch.float32)


def make_tokens(cfg: LayerConfig, device="cpu"):
    """The batch of ``cfg`` alone: hidden states x [T, d] and budgets k [T],
    drawn exactly as :func:`make_layer` draws them.  Two configs that differ
    only in T (the DeepSeek-V3-shaped decode and prefill batches) share their
    weights, so a second batch can run over weights already drawn."""
    device = torch.device(device)
    x = _gauss((cfg.T, cfg.d), 1.0, derived_seed(cfg.seed, "x"), device, torch_dtype(cfg.dtype))
    return x, draw_k(cfg).to(device)


def make_layer(cfg: LayerConfig, device="cpu") -> Layer:
    """Draw the layer described by ``cfg`` directly on ``device``.

    The stream of random numbers depends on the device type (CPU and GPU
    generators differ), never on anything else.
    """
    device = torch.device(device)
    dt = torch_dtype(cfg.dtype)
    T, d, E, I = cfg.T, cfg.d, cfg.E, cfg.I
    s = cfg.seed
    x, k = make_tokens(cfg, device)
    w_router = _gauss((E, d), 1.0 / math.sqrt(d), derived_seed(s, "w_router"), device, dt)
    bias = zipf_bias(E, cfg.zipf_bias).to(device) if cfg.zipf_bias else None

    w_gate = torch.empty((E, I, d), dtype=dt, device=device)
    w_up = torch.empty((E, I, d), dtype=dt, device=device)
    w_down = torch.empty((E, d, I), dtype=dt, device=device)
    N, C = cfg.split, cfg.I_base
    for j in range(cfg.E_base):
        g = _gauss((C, d), 1.0 / math.sqrt(d), derived_seed(s, "w_gate", j), device, dt)
        u = _gauss((C, d), 1.0 / math.sqrt(d), derived_seed(s, "w_up", j), device, dt)
        dn = _gauss((d, C), 1.0 / math.sqrt(C), derived_seed(s, "w_down", j), device, dt)
        for n in range(N):
            sl = slice(n * I, (n + 1) * I)       # neuron slice S_n (Eq. 3)
            w_gate[N * j + n].copy_(g[sl])
            w_up[N * j + n].copy_(u[sl])
            w_down[N * j + n].copy_(dn[:, sl])
        del g, u, dn

    ws_gate = ws_up = ws_down = None
    if cfg.I_shared:
        Is = cfg.I_shared
        ws_gate = _gauss((Is, d), 1.0 / math.sqrt(d), derived_seed(s, "ws_gate"), device, dt)
        ws_up = _gauss((Is, d), 1.0 / math.sqrt(d), derived_seed(s, "ws_up"), device, dt)
        ws_down = _gauss((d, Is), 1.0 / math.sqrt(Is), derived_seed(s, "ws_down"), device, dt)
    return Layer(cfg, x, w_router, bias, k, w_gate, w_up, w_down, ws_gate, ws_up, ws_down)


def make_custom_layer(T: int, d: int, E: int, I: int, k, *, dtype: str = "f32",
                      k_max: Optional[int] = None, I_shared: int = 0,
                      zipf: float = 0.0, seed: int = 0, device="cpu") -> Layer:
    """A layer of arbitrary small shape with an explicit k vector (list or
    tensor of length T), for edge cases and ragged tails."""
    k = torch.as_tensor(k, dtype=torch.int32)
    assert k.numel() == T
    km = int(k.max().item()) if (k_max is None and T > 0) else (k_max or 1)
    cfg = LayerConfig(f"custom_T{T}_d{d}_E{E}_I{I}", dtype, T=T, d=d, E=E, I=I,
                      k_values=(1,), k_probs=(1.0,), k_max=max(1, km),
                      I_shared=I_shared, zipf_bias=zipf, seed=seed)
    layer = make_layer(cfg, device)
    layer.k = k.to(device)
    return layer


def to_f64(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Exact upcast of an fp32/bf16 tensor (any device) to a float64 numpy
    array; int tensors come back as int64."""
    if t is None:
        return None
    t = t.detach().cpu()
    if t.dtype in (torch.int32, torch.int64):
        return t.numpy().astype(np.int64)
    return t.float().numpy().astype(np.float64)


class ExpertView:
    """``view[e]`` is expert e of a stacked weight tensor (any device) as a
    float64 numpy array, copied on demand, so a CPU check can read a few
    experts of a layer that only fits in device memory."""

    def __init__(self, stacked: torch.Tensor):
        self.stacked = stacked

    def __getitem__(self, e: int) -> np.ndarray:
        return to_f64(self.stacked[e])

    def __len__(self) -> int:
        return self.stacked.shape[0]


def make_proxy_inputs(cfg: LayerConfig, r: int, device="cpu"):
    """Inputs of proxy gating on a split layer (cfg.split = N sub-experts per
    whole expert): the whole-expert router w_router_base [E/N][d] (same law as
    the layer's router) and gate_idx int32 [E][r], r distinct neurons of each
    sub-expert drawn uniformly and sorted (a stand-in for the neurons a
    co-activation calibration would keep, which needs a model and data)."""
    device = torch.device(device)
    dt = torch_dtype(cfg.dtype)
    w_base = _gauss((cfg.E_base, cfg.d), 1.0 / math.sqrt(cfg.d), derived_seed(cfg.seed, "w_router", 1), device, dt)
    g = torch.Generator(device="cpu")
    g.manual_seed(derived_seed(cfg.seed, "k", 13))
    idx = torch.stack([torch.sort(torch.randperm(cfg.I, generator=g)[:r]).values for _ in range(cfg.E)])
    return w_base, idx.to(torch.int32).to(device)


def make_path_mask(E: int, extra: int, seed: int = 0, offset: float = -0.5, noise: float = 0.1):
    """A synthetic active path list for compositional path routing (the
    learned, pruned mask needs training): every diagonal path (e, e) with bias
    0, plus `extra` off-diagonal targets per source drawn without replacement,
    each with bias offset + U(-noise, noise) (a negative prior with bounded
    noise, as at initialisation).  Returns (src, tgt, bias) numpy arrays
    sorted by (src, tgt): int32, int32, float32."""
    g = torch.Generator(device="cpu")
    g.manual_seed(derived_seed(seed, "k", 17))
    rows = []
    for i in range(E):
        others = [j for j in range(E) if j != i]
        pick = torch.randperm(len(others), generator=g)[:extra].tolist()
        rows.append((i, i, 0.0))
        for q in pick:
            b = offset + noise * (2.0 * torch.rand(1, generator=g).item() - 1.0)
            rows.append((i, others[q], b))
    rows.sort()
    src = np.array([r[0] for r in rows], dtype=np.int32)
    tgt = np.array([r[1] for r in rows], dtype=np.int32)
    bias = np.array([r[2] for r in rows], dtype=np.float32)
    return src, tgt, bias


def make_target_router(cfg: LayerConfig, device="cpu") -> torch.Tensor:
    """The projection-side prior's weights w_tgt [E][d] (same law as the
    router's)."""
    return _gauss((cfg.E, cfg.d), 1.0 / math.sqrt(cfg.d), derived_seed(cfg.seed, "w_router", 2), torch.device(device),
                  torch_dtype(cfg.dtype))
