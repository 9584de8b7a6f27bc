"""Benchmark of the MoE layer forward with per-token top-k on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--eager]
                    [--no-flush] [--no-cpu-baseline]

One step = one moe_forward over one batch (router + top-k, histogram/scan/
permutation, gate/up + SwiGLU, down projection, shared expert if any, weighted
combine), on a seeded synthetic layer already resident in HBM.  The default
workload is the DeepSeek-V3-shaped layer at mixed per-token budgets k in
{4, 8}: the 4,096-token batch is the headline, and a 128-token decode batch
over the same weights is reported beside it.

Timing: each step is replayed from a captured HIP graph (the library's launch
grids depend only on the layer shape, so one graph serves every k mix) and
timed with its own pair of HIP events; between steps, outside the events, a
1 GiB write evicts the 256 MB last-level cache, so no step finds the previous
step's weights there.  --no-flush times the steps back to back instead (G
steps per graph replay); both figures are printed.  Prints one JSON line.

Beside the layer throughput it reports, for the dominant kernel (the gate/up
SwiGLU FFN), the algorithmic bytes (HBM-bound) or FLOPs (MFMA-bound) per launch
over its average launch time measured with HIP events on its own stream
inside the layer; the read rate of a plain streaming-read kernel (the
practical HBM ceiling); and the CPU oracle timed on a bounded sample of the
same workload on the host cores.
"""
from __future__ import annotations

import argparse
import copy
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at mixed per-token k; % HBM roofline (decode) / % MFMA (prefill)"
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3        # MI355X fp32 (matrix and vector)
DEFAULT_WORKLOAD = "dsv3"       # the DeepSeek-V3-shaped layer: 4,096-token headline + 128-token decode
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
FLUSH_BYTES = 1 << 30           # written between timed steps (> the 256 MB last-level cache)
CPU_SAMPLE = {"mixtral_decode": 64, "qwen3_30b_a3b_decode": 256, "tiny_fp32": 16, "subexpert_prefill": 64,
              "dsv3_decode": 8, "dsv3_prefill": 8}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-seconds", type=float, default=0.5,
                    help="keep warming up (after --warmup steps) until this much time has passed, so the "
                         "GPU clocks have settled before timing")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="dsv3 (default: dsv3_prefill headline + dsv3_decode on the same weights) or one "
                         "workload name")
    ap.add_argument("--eager", action="store_true", help="time plain launches instead of a HIP graph")
    ap.add_argument("--no-flush", action="store_true",
                    help="headline from back-to-back steps (no cache-evicting write between steps)")
    ap.add_argument("--graph-steps", type=int, default=4,
                    help="layer steps captured back to back in one HIP graph for the back-to-back timing, as a "
                         "model's layers would be (the largest divisor of --steps not above this)")
    ap.add_argument("--router", default="auto", choices=["auto", "float64", "screened", "fused"],
                    help="router algorithm (both give identical routing; they differ in cost)")
    ap.add_argument("--path", default="auto", choices=["auto", "stream", "gemm"], help="FFN path")
    ap.add_argument("--weight-layout", default="blocked", choices=["blocked", "rowmajor"],
                    help="storage order of the expert weights (blocked: converted once by moe_pack_weights "
                         "before timing, as at load time)")
    ap.add_argument("--k-dist", default="",
                    help="eq7:MU,SIGMA draws the budgets k = clip(round(N(MU, SIGMA^2)), 1, k_max) "
                         "instead of the workload's own law")
    ap.add_argument("--fold", default="",
                    help="token:K or pool:D: fold the routes (ExFold) before the permutation, with "
                         "synthetic projector / loss tables; the step then runs the staged calls")
    ap.add_argument("--proxy", type=int, default=0,
                    help="R > 0: route the split layer by training-free proxy gating (MoE-Prism) with R "
                         "gate neurons per sub-expert over a synthetic whole-expert router picking "
                         "k_max / split experts; the step then runs the staged calls")
    ap.add_argument("--paths", default="",
                    help="EXTRA[:LAMBDA]: run the layer as compositional paths (PCoMoE) over a synthetic active "
                         "list of the diagonal plus EXTRA off-diagonal paths per source, with a synthetic "
                         "target prior scaled by LAMBDA (default 0.5); the step then runs the staged calls")
    ap.add_argument("--k-policy", default="exact",
                    help="budget each token executes: exact (its own k_t; the headline), batch_max "
                         "(every token runs the batch maximum) or round_up:N (k_t rounded up to a "
                         "multiple of N) -- the over-serving comparators")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the streaming-read ceiling")
    ap.add_argument("--cpu-sample", type=int, default=0,
                    help="tokens in the CPU-oracle sample (0 = workload default)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="also time the vendor library's dense bf16 GEMM (torch.matmul) on matrices of the "
                         "routed FFN's shapes and FLOPs (A x d by d x 2I, A x I by I x d): a reference for "
                         "the grouped kernels' MFMA fraction, outside the layer's timing")
    ap.add_argument("--calib-copy", action="store_true",
                    help="before timing, run a plain elementwise copy (torch.neg) of 512 MiB fp32 three "
                         "times: the known-size kernel that scales rocprofv3 FETCH_SIZE/WRITE_SIZE")
    return ap.parse_args()


KERNEL_SOURCES = {"stream": ("ffn_stream.hip", "common.h"), "gemm": ("ffn_gemm.hip", "common.h")}


def kernel_source_hash(path: str) -> str:
    """Hash of the source files of the gate/up kernel of FFN path `path`."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_layer_token_amd", "csrc")
    for f in KERNEL_SOURCES[path]:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, path: str, layout: str):
    """Per-launch HBM bytes of the gate/up kernel from the committed rocprofv3
    counter runs, or None when absent or taken on other kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))[workload]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("path") != path or rec.get("source_hash") != kernel_source_hash(path):
        return None
    if rec.get("weight_layout", "rowmajor") != layout:
        return None
    return rec.get("bytes_per_launch")


class HostExperts:
    """``view[e]``: expert e of a stacked bf16/fp32 weight tensor held in host
    memory in its own element type, upcast to float64 when the oracle reads it
    (the oracle reads each expert once per call)."""

    def __init__(self, host: dict):
        self.host = host

    def __getitem__(self, e: int):
        import numpy as np
        return self.host[int(e)].float().numpy().astype(np.float64)


def cpu_baseline(layer, n_tokens: int, min_seconds: float = 10.0):
    """The oracle as it stands, on the first n_tokens of the same batch.  The
    experts the sample reaches are copied to host memory in their own element
    type beforehand (bounded host RAM); the upcast to float64 happens inside
    the timed calls.  The sample runs repeatedly until min_seconds have
    passed; `cores` is the process CPU time over the wall time of the timed
    runs (the cores the oracle actually kept busy)."""
    import numpy as np
    import threadpoolctl

    import oracle
    from workloads import to_f64

    cfg = layer.cfg
    tokens = np.arange(min(n_tokens, cfg.T))
    r = oracle.route(to_f64(layer.x[:len(tokens)]), to_f64(layer.w_router), to_f64(layer.router_bias),
                     to_f64(layer.k[:len(tokens)]), cfg.k_max, cfg.routed_scale)
    used = sorted(set(r["ids"].tolist()))
    wg = HostExperts({e: layer.w_gate[e].cpu() for e in used})
    wu = HostExperts({e: layer.w_up[e].cpu() for e in used})
    wd = HostExperts({e: layer.w_down[e].cpu() for e in used})
    sh = None
    if layer.ws_gate is not None:
        sh = (to_f64(layer.ws_gate), to_f64(layer.ws_up), to_f64(layer.ws_down))
    x, wr = to_f64(layer.x[:len(tokens)]), to_f64(layer.w_router)
    b = to_f64(layer.router_bias)
    k = layer.k[:len(tokens)].cpu().numpy()
    info = threadpoolctl.threadpool_info()
    blas = max((p.get("num_threads", 1) for p in info), default=1)
    reps = 0
    t0, c0 = time.perf_counter(), time.process_time()
    while True:
        oracle.forward(x, wr, b, k, cfg.k_max, wg, wu, wd, shared=sh, routed_scale=cfg.routed_scale)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    busy = (time.process_time() - c0) / dt
    n = reps * len(tokens)
    return {"value": n / dt, "unit": "tokens/s", "cores": max(1, int(round(busy))), "kind": "oracle",
            "sample": f"first {len(tokens)} of {cfg.T} tokens of {cfg.name} ({len(used)} experts reached), run "
                      f"{reps} times: {n} token-forwards in {dt:.1f} s, float64 numpy oracle, expert weights "
                      f"held on the host in their element type and upcast per expert; {busy:.1f} cores busy on "
                      f"average (BLAS pool {blas} threads)"}


def read_ceiling(dev, stream, flush, kernel_bytes=None):
    """GB/s of the streaming-read probe (moe_probe_read) over 4 GiB, ordinary
    and non-temporal loads, best of 5 launches each.  With kernel_bytes, also
    the non-temporal probe over the dominant kernel's own algorithmic bytes
    (at most 4 GiB), each launch after the same cache-evicting write as the
    timed steps, median of 5: the read rate a plain stream of that size
    reaches from a cold cache (it falls with the size: the ramp and the tail
    of a launch weigh more on a short one)."""
    import torch

    import mixture_experts_layer_token_amd as moe
    buf = torch.ones(1 << 30, dtype=torch.int32, device=dev)  # 4 GiB
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    nbytes = buf.numel() * 4
    res = {}
    with torch.cuda.stream(stream):
        for nt in (False, True):
            moe.probe_read(buf, sink, nt)
            best = None
            for _ in range(5):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                moe.probe_read(buf, sink, nt)
                b.record(stream)
                b.synchronize()
                ms = a.elapsed_time(b)
                best = ms if best is None else min(best, ms)
            res["nontemporal" if nt else "ordinary"] = round(nbytes / (best * 1e-3) / 1e9, 1)
        at_size = None
        if kernel_bytes:
            n_at = min(int(kernel_bytes), nbytes) // 16 * 4   # int32 elements, whole 16-byte chunks
            part = buf[:n_at]
            per = []
            for _ in range(5):
                flush()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                moe.probe_read(part, sink, True)
                b.record(stream)
                b.synchronize()
                per.append(a.elapsed_time(b))
            med = statistics.median(per)
            at_size = {"bytes": n_at * 4, "GBps": round(n_at * 4 / (med * 1e-3) / 1e9, 1),
                       "timing": "non-temporal loads, 1 GiB cache-evicting write before each launch, median of 5"}
    del buf
    torch.cuda.synchronize()
    return {"GBps": max(res.values()), "ordinary_GBps": res["ordinary"], "nontemporal_GBps": res["nontemporal"],
            "bytes": nbytes, "kernel": "moe_probe_read (16-byte loads, 4 KB runs round-robin, 2 workgroups/CU)",
            "at_kernel_bytes": at_size}


def library_gemm(dev, stream, A, d, I, flush):
    """Dense bf16 GEMMs of the vendor library (torch.matmul) with the routed
    FFN's FLOPs: [A, d] x [d, 2I] (gate and up side by side) and [A, I] x
    [I, d], no gather, no grouping, no SwiGLU.  The right operand is timed
    both as [N, K] (K contiguous, the experts' storage; a transposed 2-D view)
    and as [K, N]; the faster is reported.  Median of 9 launches, each after
    the cache-evicting write."""
    import torch
    out = {}
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    for name, (M, K, N) in (("gateup", (A, d, 2 * I)), ("down", (A, I, d))):
        a = torch.randn(M, K, device=dev, dtype=torch.bfloat16, generator=g)
        c = torch.empty(M, N, device=dev, dtype=torch.bfloat16)
        best = None
        for layout in ("NK", "KN"):
            w = torch.randn((N, K) if layout == "NK" else (K, N), device=dev, dtype=torch.bfloat16, generator=g)
            rhs = w.t() if layout == "NK" else w
            ts = []
            with torch.cuda.stream(stream):
                for i in range(12):
                    flush()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    torch.matmul(a, rhs, out=c)
                    e1.record(stream)
                    e1.synchronize()
                    if i >= 3:
                        ts.append(e0.elapsed_time(e1) * 1e3)
            ts.sort()
            us = ts[len(ts) // 2]
            if best is None or us < best[0]:
                best = (us, layout)
            del w, rhs
        us, layout = best
        tf = 2.0 * M * N * K / (us * 1e-6) / 1e12
        out[name] = {"M": M, "K": K, "N": N, "weights": layout, "us": round(us, 1), "TFLOPs": round(tf, 1),
                     "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4)}
        del a, c
    torch.cuda.synchronize()
    return out


class Bench:
    """One workload's layer step, its timing and its dominant kernel."""

    def __init__(self, args, layer, layer_rm, dev, stream, flush):
        import torch

        import mixture_experts_layer_token_amd as moe
        self.args, self.layer, self.layer_rm, self.dev, self.stream, self.flush = \
            args, layer, layer_rm, dev, stream, flush
        cfg = layer.cfg
        self.cfg = cfg
        T, d, E, I = cfg.T, cfg.d, cfg.E, cfg.I
        Is = cfg.I_shared
        kpol, _, kgran = args.k_policy.partition(":")
        kgran = int(kgran) if kgran else 1
        self.kp = dict(k_policy=kpol, k_granule=kgran, weight_layout=args.weight_layout)
        self.desc = moe.make_desc(T, d, E, I, cfg.k_max, I_shared=Is, dtype=layer.x.dtype,
                                  routed_scale=cfg.routed_scale, path=args.path, router=args.router, **self.kp)
        desc = self.desc
        ws = moe.alloc_workspace(desc, moe.MOE_OP_FORWARD, dev)
        self.out = out = torch.empty((T, d), dtype=layer.x.dtype, device=dev)
        self.stats = stats = torch.empty(E + 2, dtype=torch.int32, device=dev)
        self.status = status = torch.empty(1, dtype=torch.int32, device=dev)
        sh = (layer.ws_gate, layer.ws_up, layer.ws_down) if Is else (None, None, None)
        self.sh = sh

        def step():
            moe.moe_forward(desc, layer.x, layer.w_router, layer.router_bias, layer.k, layer.w_gate,
                            layer.w_up, layer.w_down, *sh, out, stats, status, ws)

        self.fold = self.proxy = self.paths = None
        if args.fold:
            step = self._fold_step()
        if args.proxy:
            step = self._proxy_step()
        if args.paths:
            step = self._paths_step()
        self.step = step

    # ---- variants of the step (next rows of the method) ----
    def _fold_step(self):
        import torch

        import mixture_experts_layer_token_amd as moe
        from workloads import make_fold_tables
        args, layer, dev, desc, cfg = self.args, self.layer, self.dev, self.desc, self.cfg
        T, d, E = cfg.T, cfg.d, cfg.E
        fmode, _, fb = args.fold.partition(":")
        fold = dict(mode=fmode, budget=int(fb), tables=[t.to(dev) for t in make_fold_tables(E, seed=cfg.seed)])
        i32 = dict(dtype=torch.int32, device=dev)
        A_cap = T * cfg.k_max
        f = {n: torch.empty(T + 1, **i32) for n in ("to0", "to1")}
        f.update({n: torch.empty(A_cap, **i32) for n in ("ids0", "ids1", "pt0", "ps0", "iv0", "pt1", "ps1", "iv1")})
        f.update({n: torch.empty(A_cap, dtype=torch.float32, device=dev) for n in ("w0", "w1")})
        f.update({n: torch.empty(E + 1, **i32) for n in ("eo0", "eo1")})
        f.update({n: torch.empty(E, **i32) for n in ("c0", "c1")})
        f.update({n: torch.empty(1, **i32) for n in ("na0", "na1")})
        f["y"] = torch.empty((A_cap, d), dtype=layer.x.dtype, device=dev)
        f["ysh"] = torch.empty((T, d), dtype=layer.x.dtype, device=dev) if cfg.I_shared else None
        f["ws"] = {op: moe.alloc_workspace(desc, op, dev)
                   for op in (moe.MOE_OP_ROUTE, moe.MOE_OP_PERMUTE, moe.MOE_OP_FOLD, moe.MOE_OP_FFN)}
        fold["buf"] = f
        self.fold = fold
        sh, out, status = self.sh, self.out, self.status

        def step():
            # route -> (permute: pool mode) -> fold -> permute -> FFN -> combine
            S_, L_, H_ = fold["tables"]
            wsd = f["ws"]
            moe.moe_route(desc, layer.x, layer.w_router, layer.router_bias, layer.k, f["to0"], f["ids0"], f["w0"],
                          status, wsd[moe.MOE_OP_ROUTE])
            if fmode == "pool":
                moe.moe_permute(desc, f["to0"], f["ids0"], f["c0"], f["eo0"], f["pt0"], f["ps0"], f["iv0"],
                                f["na0"], wsd[moe.MOE_OP_PERMUTE])
            moe.moe_fold(desc, fmode, fold["budget"], S_, L_, H_, f["to0"], f["ids0"], f["w0"], f["eo0"],
                         f["ps0"], f["to1"], f["ids1"], f["w1"], None, wsd[moe.MOE_OP_FOLD])
            moe.moe_permute(desc, f["to1"], f["ids1"], f["c1"], f["eo1"], f["pt1"], f["ps1"], f["iv1"], f["na1"],
                            wsd[moe.MOE_OP_PERMUTE])
            moe.moe_ffn(desc, layer.x, layer.w_gate, layer.w_up, layer.w_down, *sh, f["eo1"], f["pt1"], f["y"],
                        f["ysh"], wsd[moe.MOE_OP_FFN])
            moe.moe_combine(desc, f["y"], f["ysh"], f["to1"], f["w1"], f["iv1"], out)
        return step

    def _proxy_step(self):
        import torch

        import mixture_experts_layer_token_amd as moe
        from workloads import make_proxy_inputs
        args, layer, dev, desc, cfg = self.args, self.layer, self.dev, self.desc, self.cfg
        T, d, E = cfg.T, cfg.d, cfg.E
        if cfg.split < 2 or args.fold or args.k_policy != "exact":
            raise SystemExit("--proxy needs a split workload, no --fold and the exact k policy")
        Np, rp = cfg.split, args.proxy
        mp = -(-cfg.k_max // Np)
        w_base, gate_idx = make_proxy_inputs(cfg, rp, dev)
        wp_g, wp_u = moe.proxy_pack(layer.w_gate, layer.w_up, gate_idx, Np, weight_layout=args.weight_layout)
        pr = moe.ProxyRouter(desc, Np, rp, mp, moe.moe_proxy_kappa_balanced(cfg.k_max, mp, Np), dev)
        i32 = dict(dtype=torch.int32, device=dev)
        A_cap = T * cfg.k_max
        pb = {n: torch.empty(A_cap, **i32) for n in ("pt", "ps", "iv")}
        pb.update(eo=torch.empty(E + 1, **i32), c=torch.empty(E, **i32), na=torch.empty(1, **i32),
                  y=torch.empty((A_cap, d), dtype=layer.x.dtype, device=dev),
                  ysh=torch.empty((T, d), dtype=layer.x.dtype, device=dev) if cfg.I_shared else None,
                  wsp=moe.alloc_workspace(desc, moe.MOE_OP_PERMUTE, dev),
                  wsf=moe.alloc_workspace(desc, moe.MOE_OP_FFN, dev))
        self.proxy = proxy = dict(r=rp, m=mp, N=Np, router=pr, buf=pb,
                                  run=lambda: pr.run(layer.x, w_base, None, layer.k, wp_g, wp_u))
        sh, out = self.sh, self.out

        def step():
            # whole-expert route -> proxy scores and routes -> permute -> FFN -> combine
            proxy["run"]()
            moe.moe_permute(desc, pr.tok_off, pr.ids, pb["c"], pb["eo"], pb["pt"], pb["ps"], pb["iv"], pb["na"],
                            pb["wsp"])
            moe.moe_ffn(desc, layer.x, layer.w_gate, layer.w_up, layer.w_down, *sh, pb["eo"], pb["pt"], pb["y"],
                        pb["ysh"], pb["wsf"])
            moe.moe_combine(desc, pb["y"], pb["ysh"], pr.tok_off, pr.w, pb["iv"], out)
        return step

    def _paths_step(self):
        import mixture_experts_layer_token_amd as moe
        from workloads import make_path_mask, make_target_router
        args, layer, dev, desc, cfg = self.args, self.layer, self.dev, self.desc, self.cfg
        if args.fold or args.proxy:
            raise SystemExit("--paths excludes --fold and --proxy")
        extra, _, lam = args.paths.partition(":")
        lam = float(lam) if lam else 0.5
        p_src, p_tgt, p_bias = make_path_mask(cfg.E, int(extra), seed=cfg.seed)
        table = moe.moe_path_table(cfg.E, p_src, p_tgt, p_bias, dev)
        pl = moe.PathLayer(desc, table, len(p_src), lam, dev)
        w_tgt = make_target_router(cfg, dev)
        sh_w = (layer.ws_gate, layer.ws_up, layer.ws_down) if cfg.I_shared else None
        self.paths = paths = dict(layer=pl, P=len(p_src), extra=int(extra), lam=lam,
                                  run=lambda o: pl.run(layer.x, layer.w_router, layer.router_bias, w_tgt, layer.k,
                                                       layer.w_gate, layer.w_up, layer.w_down, o, shared=sh_w))
        out = self.out

        def step():
            # path route -> sources -> expansions once per source -> projections by target -> combine
            paths["run"](out)
        return step

    # ---- timing of the whole step ----
    def time_steps(self):
        """Warm-up, then the timed steps: flushed (one event pair per step,
        the cache-evicting write between steps outside the events) and back
        to back (G steps per graph replay, one event pair around them)."""
        import torch
        args, stream, step = self.args, self.stream, self.step
        with torch.cuda.stream(stream):
            step()
        stream.synchronize()
        g_steps = 1
        graph1 = graphg = None
        if not args.eager:
            g_steps = max(g for g in range(1, max(1, args.graph_steps) + 1) if args.steps % g == 0)
            graph1 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph1, stream=stream):
                step()
            graphg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graphg, stream=stream):
                for _ in range(g_steps):
                    step()
        run1 = graph1.replay if graph1 is not None else step
        rung = graphg.replay if graphg is not None else step
        if graphg is None:
            g_steps = 1

        with torch.cuda.stream(stream):
            w_start = time.perf_counter()
            n = 0
            while n < args.warmup or time.perf_counter() - w_start < args.warmup_seconds:
                run1()
                n += 1
                if n % 8 == 0:
                    stream.synchronize()
            stream.synchronize()
            n_warm = n

            # flushed: exactly --steps steps, each between its own events
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
            torch.cuda.synchronize()
            w0 = time.perf_counter()
            for a, b in ev:
                self.flush()
                a.record(stream)
                run1()
                b.record(stream)
            torch.cuda.synchronize()
            wall_flushed = time.perf_counter() - w0
            per = [a.elapsed_time(b) for a, b in ev]

            # back to back: exactly --steps steps, G per graph replay
            t_start = torch.cuda.Event(enable_timing=True)
            t_end = torch.cuda.Event(enable_timing=True)
            for _ in range(2):
                rung()
            torch.cuda.synchronize()
            w1 = time.perf_counter()
            t_start.record(stream)
            for _ in range(args.steps // g_steps):
                rung()
            t_end.record(stream)
            torch.cuda.synchronize()
            wall_b2b = time.perf_counter() - w1
        b2b_ms = t_start.elapsed_time(t_end) / args.steps
        flushed_ms = sum(per) / len(per)
        self.n_warm = n_warm
        self.g_steps = g_steps
        self.timing = {"flushed_ms_per_step": round(flushed_ms, 4),
                       "flushed_median_ms": round(statistics.median(per), 4),
                       "flushed_min_ms": round(min(per), 4), "flushed_max_ms": round(max(per), 4),
                       "back_to_back_ms_per_step": round(b2b_ms, 4),
                       "back_to_back_execution": "eager" if args.eager else f"hip_graph ({g_steps} steps per replay)",
                       "wall_s": round(wall_flushed + wall_b2b, 3)}
        self.ms_step = b2b_ms if args.no_flush else flushed_ms
        self.wall = wall_b2b if args.no_flush else wall_flushed
        return self.ms_step

    def counts(self):
        """(n_active, A) of the gate/up launch's routes."""
        cfg = self.cfg
        T, E = cfg.T, cfg.E
        status = self.status
        if self.proxy is not None:
            status = self.proxy["router"].status
        if self.paths is not None:
            status = self.paths["layer"].status
        assert int(status.item()) == 0
        if self.paths is not None:
            pl = self.paths["layer"]
            self.paths["routes"] = int(pl.tok_off[T].item())
            self.paths["targets_active"] = int(pl.t_nact.item())
            return int(pl.s_nact.item()), int(pl.src_off[T].item())
        if self.proxy is not None:
            return int(self.proxy["buf"]["na"].item()), int(self.proxy["router"].tok_off[T].item())
        if self.fold is not None:
            return int(self.fold["buf"]["na1"].item()), int(self.fold["buf"]["to1"][T].item())
        st = self.stats.cpu().numpy()
        return int(st[E]), int(st[E + 1])

    # ---- the dominant kernel, timed inside the layer ----
    def dominant(self, n_act, A):
        """The gate/up SwiGLU FFN timed inside the layer: the routed layer runs
        as its separate calls (route, permute, plan, gate/up, down, combine)
        on the same stream, with the cache-evicting write before each pass and
        HIP events around each gate/up launch, so the kernel meets the
        caches, clocks and power state it has in the layer.  Also timed back
        to back on its own."""
        import torch

        import mixture_experts_layer_token_amd as moe
        args, layer, dev, stream, cfg = self.args, self.layer, self.dev, self.stream, self.cfg
        T, d, E, I = cfg.T, cfg.d, cfg.E, cfg.I
        desc_r = moe.make_desc(T, d, E, I, cfg.k_max, dtype=layer.x.dtype, routed_scale=cfg.routed_scale,
                               path=args.path, router=args.router, **self.kp)
        i32 = dict(dtype=torch.int32, device=dev)
        tok_off = torch.empty(T + 1, **i32)
        ids = torch.empty(T * cfg.k_max, **i32)
        wts = torch.empty(T * cfg.k_max, dtype=torch.float32, device=dev)
        counts = torch.empty(E, **i32)
        eoff = torch.empty(E + 1, **i32)
        ptok = torch.empty(T * cfg.k_max, **i32)
        psrc = torch.empty_like(ptok)
        inv = torch.empty_like(ptok)
        nact = torch.empty(1, **i32)
        h = torch.empty((T * cfg.k_max, I), dtype=layer.x.dtype, device=dev)
        y = torch.empty((T * cfg.k_max, d), dtype=layer.x.dtype, device=dev)
        out_r = torch.empty((T, d), dtype=layer.x.dtype, device=dev)
        ws_route = moe.alloc_workspace(desc_r, moe.MOE_OP_ROUTE, dev)
        ws_perm = moe.alloc_workspace(desc_r, moe.MOE_OP_PERMUTE, dev)
        ws_ffn = moe.alloc_workspace(desc_r, moe.MOE_OP_FFN, dev)
        routed_path, _ = moe.resolve_path(self.desc)
        assert moe.resolve_path(desc_r)[0] == routed_path
        status = self.status
        fold, proxy, paths = self.fold, self.proxy, self.paths

        def gateup():
            moe.moe_ffn_gateup(desc_r, layer.x, layer.w_gate, layer.w_up, eoff, ptok, h, ws_ffn)

        n_in = max(args.steps, 10)
        warm = 3
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_in)]
        with torch.cuda.stream(stream):
            for i in range(warm + n_in):
                self.flush()
                if paths is not None:
                    paths["run"](out_r)
                    tok_off.copy_(paths["layer"].src_off)
                    ids.copy_(paths["layer"].src_ids)
                elif proxy is not None:
                    proxy["run"]()
                    tok_off.copy_(proxy["router"].tok_off)
                    ids.copy_(proxy["router"].ids)
                    wts.copy_(proxy["router"].w)
                else:
                    moe.moe_route(desc_r, layer.x, layer.w_router, layer.router_bias, layer.k, tok_off, ids, wts,
                                  status, ws_route)
                if fold is not None:
                    fb_ = fold["buf"]
                    moe.moe_permute(desc_r, tok_off, ids, counts, eoff, ptok, psrc, inv, nact, ws_perm)
                    moe.moe_fold(desc_r, fold["mode"], fold["budget"], *fold["tables"], tok_off, ids, wts, eoff,
                                 psrc, fb_["to1"], fb_["ids1"], fb_["w1"], None, fb_["ws"][moe.MOE_OP_FOLD])
                    tok_off.copy_(fb_["to1"])
                    ids.copy_(fb_["ids1"])
                    wts.copy_(fb_["w1"])
                moe.moe_permute(desc_r, tok_off, ids, counts, eoff, ptok, psrc, inv, nact, ws_perm)
                moe.moe_ffn_plan(desc_r, eoff, ws_ffn)
                j = i - warm
                if j >= 0:
                    pairs[j][0].record(stream)
                gateup()
                if j >= 0:
                    pairs[j][1].record(stream)
                moe.moe_ffn_down(desc_r, h, layer.w_down, eoff, y, ws_ffn)
                moe.moe_combine(desc_r, y, None, tok_off, wts, inv, out_r)
                if i % 8 == 7:
                    stream.synchronize()
            torch.cuda.synchronize()
            k_ms = sum(a.elapsed_time(b) for a, b in pairs) / n_in
            # back to back, on its own (same routing)
            for _ in range(3):
                gateup()
            k_start = torch.cuda.Event(enable_timing=True)
            k_end = torch.cuda.Event(enable_timing=True)
            k_start.record(stream)
            for _ in range(n_in):
                gateup()
            k_end.record(stream)
            torch.cuda.synchronize()
        alone_ms = k_start.elapsed_time(k_end) / n_in
        esz = layer.x.element_size()
        gu_bytes = 2 * n_act * I * d * esz + T * d * esz + A * I * esz   # weights + x rows + H
        gu_flops = 4.0 * d * I * A
        # The bound is the roofline's: arithmetic intensity (algorithmic FLOPs per
        # algorithmic byte) against the ridge point peak FLOP/s / peak HBM bytes/s.
        peak_f = PEAK_BF16_TFLOPS if esz == 2 else PEAK_FP32_TFLOPS
        intensity = gu_flops / gu_bytes
        ridge = peak_f * 1e12 / (PEAK_HBM_GBS * 1e9)
        mfma_bound = intensity >= ridge
        if mfma_bound:
            ach = gu_flops / (k_ms * 1e-3) / 1e12
            roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak_f, "unit": "TFLOP/s",
                    "frac": round(ach / peak_f, 4)}
        else:
            ach = gu_bytes / (k_ms * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(ach / PEAK_HBM_GBS, 4)}
        roof["kernel"] = ("ffn_gemm_kernel (routed gate/up + SwiGLU)" if routed_path == "gemm"
                          else "ffn_stream_kernel (routed gate/up + SwiGLU)")
        roof["avg_launch_us"] = round(k_ms * 1e3, 2)
        roof["timing"] = ("in the layer (separate calls, cache-evicting write before each pass, events around "
                          "each gate/up launch)")
        roof["back_to_back_us"] = round(alone_ms * 1e3, 2)
        roof["algorithmic_per_launch"] = gu_flops if mfma_bound else gu_bytes
        roof["intensity_flop_per_byte"] = round(intensity, 1)
        roof["ridge_flop_per_byte"] = round(ridge, 1)
        plain = (args.k_policy == "exact" and not args.k_dist and not args.fold and not args.proxy
                 and not args.paths)
        roof["traffic"] = measured_traffic(cfg.name, routed_path, args.weight_layout) if plain else None
        self.routed_path = routed_path
        return roof

    def layer_info(self, n_act, A):
        cfg = self.cfg
        T, d, E, I, Is = cfg.T, cfg.d, cfg.E, cfg.I, cfg.I_shared
        esz = self.layer.x.element_size()
        w_bytes = 3 * n_act * d * I * esz
        ffn_flops = 6.0 * d * I * A + 6.0 * d * Is * T
        if self.paths is not None:
            # expansions (gate/up) over the active sources, projections over the active targets
            w_bytes = (2 * n_act + self.paths["targets_active"]) * d * I * esz
            ffn_flops = 4.0 * d * I * A + 2.0 * d * I * self.paths["routes"] + 6.0 * d * Is * T
        all_bytes = w_bytes + 3 * d * Is * esz + E * d * esz + 2 * T * d * esz
        layer_s = self.ms_step * 1e-3
        peak_f = PEAK_BF16_TFLOPS if esz == 2 else PEAK_FP32_TFLOPS
        return {"activated_weight_bytes": w_bytes,
                "activated_weight_GBps": round(w_bytes / layer_s / 1e9, 1),
                "activated_weight_frac_hbm": round(w_bytes / layer_s / 1e9 / PEAK_HBM_GBS, 4),
                "all_bytes_GBps": round(all_bytes / layer_s / 1e9, 1),
                "ffn_TFLOPs": round(ffn_flops / layer_s / 1e12, 2),
                "ffn_frac_mfma": round(ffn_flops / layer_s / 1e12 / peak_f, 4)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on exactly one GPU; --gpus above 1 is not supported "
              "(multi-GPU sharding of the layer is a design note only)", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixture_experts_layer_token_amd as moe
    from workloads import CONFIGS, Layer, make_layer, make_tokens

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    moe._lib.load()
    combined = args.workload == "dsv3"
    cfg = CONFIGS["dsv3_prefill" if combined else args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] drawing {cfg.name}", file=sys.stderr, flush=True)
    layer = make_layer(cfg, dev)
    if args.k_dist:
        kind, _, params = args.k_dist.partition(":")
        if kind != "eq7":
            raise SystemExit(f"unknown --k-dist {args.k_dist!r}")
        mu, sigma = (float(v) for v in params.split(","))
        from workloads import draw_k_eq7
        layer.k = draw_k_eq7(cfg.T, mu, sigma, cfg.k_max, cfg.seed).to(dev)
    # the CPU baseline reads the row-major weights; the GPU runs read `layer`
    layer_rm = layer
    if args.weight_layout == "blocked":
        layer = copy.copy(layer_rm)
        for name in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
            t = getattr(layer_rm, name)
            if t is not None:
                setattr(layer, name, moe.pack_weights(t))
    torch.cuda.synchronize()

    flush_buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flush_val = [0.0]

    def flush():
        flush_val[0] += 1.0
        flush_buf.fill_(flush_val[0])

    if args.calib_copy:
        src = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.Stream()
    main_b = Bench(args, layer, layer_rm, dev, stream, flush)
    print(f"[bench] timing {cfg.name}", file=sys.stderr, flush=True)
    ms_step = main_b.time_steps()
    n_act, A = main_b.counts()
    roof = main_b.dominant(n_act, A)
    layer_info = main_b.layer_info(n_act, A)

    decode = None
    if combined:
        # the 128-token decode batch over the same (already resident) weights
        cfg_d = CONFIGS["dsv3_decode"]
        print(f"[bench] timing {cfg_d.name} on the same weights", file=sys.stderr, flush=True)
        xd, kd = make_tokens(cfg_d, dev)
        lay_d = Layer(cfg_d, xd, layer.w_router, layer.router_bias, kd, layer.w_gate, layer.w_up, layer.w_down,
                      layer.ws_gate, layer.ws_up, layer.ws_down)
        dec_b = Bench(args, lay_d, lay_d, dev, stream, flush)
        dms = dec_b.time_steps()
        dn, dA = dec_b.counts()
        droof = dec_b.dominant(dn, dA)
        decode = {"workload": cfg_d.name, "T": cfg_d.T, "value": round(cfg_d.T / (dms * 1e-3), 1),
                  "unit": "tokens/s", "ms_per_step": round(dms, 4), "A": dA, "n_active": dn,
                  "ffn_path": dec_b.routed_path, "timing": dec_b.timing, "layer": dec_b.layer_info(dn, dA),
                  "roofline": droof}

    ceiling = None
    if not args.no_probe:
        hbm = roof.get("bound") == "hbm"
        ceiling = read_ceiling(dev, stream, flush, roof["algorithmic_per_launch"] if hbm else None)
        if hbm and ceiling["at_kernel_bytes"]:
            # the dominant kernel against the plain read of its own size
            roof["frac_of_read_at_size"] = round(roof["achieved"] / ceiling["at_kernel_bytes"]["GBps"], 4)
        if decode is not None and decode["roofline"].get("bound") == "hbm":
            dr = decode["roofline"]
            at = read_ceiling(dev, stream, flush, dr["algorithmic_per_launch"])["at_kernel_bytes"]
            decode["read_ceiling_at_kernel_bytes"] = at
            dr["frac_of_read_at_size"] = round(dr["achieved"] / at["GBps"], 4)
    lib_gemm = library_gemm(dev, stream, A, cfg.d, cfg.I, flush) if args.library_gemm else None

    cpu = None
    if (not args.no_cpu_baseline and args.k_policy == "exact" and not args.fold and not args.proxy
            and not args.paths):
        n = args.cpu_sample or CPU_SAMPLE[cfg.name]
        print(f"[bench] timing the CPU oracle on {n} tokens", file=sys.stderr, flush=True)
        cpu = cpu_baseline(layer_rm, n)

    T = cfg.T
    k_desc = args.k_dist if args.k_dist else "/".join(str(v) for v in cfg.k_values)
    paths = main_b.paths
    proxy_info = None
    if main_b.proxy is not None:
        # the proxy routing stage (whole-expert route, permute, plan, proxy
        # SwiGLU, selection) back to back on its own
        proxy = main_b.proxy
        with torch.cuda.stream(stream):
            for _ in range(3):
                proxy["run"]()
            p_start = torch.cuda.Event(enable_timing=True)
            p_end = torch.cuda.Event(enable_timing=True)
            n_in = max(args.steps, 10)
            p_start.record(stream)
            for _ in range(n_in):
                proxy["run"]()
            p_end.record(stream)
            torch.cuda.synchronize()
        proxy_info = {"r": proxy["r"], "m": proxy["m"], "N": proxy["N"], "Ip": proxy["router"].Ip,
                      "stage_us": round(p_start.elapsed_time(p_end) / n_in * 1e3, 2)}
    rec = {
        "metric": METRIC,
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": main_b.n_warm,
        "warmup_requested": args.warmup,
        "warmup_note": (f"at least --warmup steps and {args.warmup_seconds} s of steps, so the GPU clocks settle "
                        "before timing (the first milliseconds of a process run ~9 % slow)"),
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if layer.x.element_size() == 2 else "f32",
        "data": "synthetic (seeded Gaussian layer, random-init weights)",
        "config": {"workload": cfg.name, "T": T, "d": cfg.d, "E": cfg.E, "I": cfg.I, "I_shared": cfg.I_shared,
                   "k_values": k_desc, "k_max": cfg.k_max, "A": A, "n_active": n_act,
                   "timing": ("back to back" if args.no_flush else
                              "one event pair per step, 1 GiB cache-evicting write between steps"),
                   "execution": "eager" if args.eager else "hip_graph",
                   "ffn_path": main_b.routed_path, "weight_layout": args.weight_layout,
                   "router": args.router, "k_policy": args.k_policy, "k_dist": args.k_dist or "workload",
                   "fold": args.fold or "none", "proxy": proxy_info or "none",
                   "paths": ({"P": paths["P"], "extra_per_source": paths["extra"], "lambda": paths["lam"],
                              "routes": paths["routes"], "expansions": A, "sources_active": n_act,
                              "targets_active": paths["targets_active"]} if paths else "none"),
                   "wall_s": round(main_b.wall, 3)},
        "timing": main_b.timing,
        "layer": layer_info,
        "roofline": roof,
        "read_ceiling": ceiling,
        "decode": decode,
        "cpu_baseline": cpu,
    }
    if lib_gemm is not None:
        rec["library_gemm"] = lib_gemm
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
