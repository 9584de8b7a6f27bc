"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/moe.h declares, sizes workspaces and rejects bad
arguments before launching anything."""
import ctypes
import os
import re

import pytest

import mixture_experts_layer_token_amd as moe
from mixture_experts_layer_token_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    hdr = open(os.path.join(ROOT, "include", "moe.h")).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char\*)\s+(moe_\w+)\s*\(", hdr, re.M)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = _declared()
    assert "moe_forward" in names and len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES)


def _desc(**kw):
    base = dict(T=64, d=4096, E=8, I=14336, k_max=2, I_shared=0, dtype=moe.MOE_BF16, path=0,
                router=0, routed_scale=1.0, k_policy=0, k_granule=1)
    base.update(kw)
    return _lib.moe_desc(**base)


def _ws(desc, op):
    n = ctypes.c_size_t(0)
    st = _lib.load().moe_workspace_size(ctypes.byref(desc), op, ctypes.byref(n))
    return st, n.value


def test_workspace_sizes():
    d = _desc()
    st, fwd = _ws(d, moe.MOE_OP_FORWARD)
    assert st == 0 and fwd % 256 == 0
    A = 64 * 2
    # forward holds at least H [A, I] and Y [A, d] in bf16
    assert fwd >= A * 14336 * 2 + A * 4096 * 2
    for op in (moe.MOE_OP_PERMUTE, moe.MOE_OP_FFN):
        st, n = _ws(d, op)
        assert st == 0 and 0 < n <= fwd
    # the small-batch router needs no partial sums; the split-K one does
    assert _ws(d, moe.MOE_OP_ROUTE) == (0, 0)
    st, n = _ws(_desc(router=moe.MOE_ROUTER_FLOAT64), moe.MOE_OP_ROUTE)
    assert st == 0 and 0 < n <= _ws(_desc(router=moe.MOE_ROUTER_FLOAT64), moe.MOE_OP_FORWARD)[1]
    assert _ws(d, moe.MOE_OP_COMBINE) == (0, 0)
    assert _ws(_desc(T=0), moe.MOE_OP_FORWARD)[0] == 0


@pytest.mark.parametrize("kw,code", [
    (dict(d=100), 2), (dict(I=64), 2), (dict(E=0), 2), (dict(E=1025, k_max=1), 2),
    (dict(k_max=9), 2), (dict(k_max=0), 2), (dict(T=-1), 2), (dict(I_shared=100), 2),
    (dict(T=1 << 28, k_max=8), 2), (dict(dtype=7), 3), (dict(path=5), 3), (dict(router=4), 3),
    (dict(router=3, E=256, k_max=2), 3), (dict(router=3, T=1025), 3),
    (dict(k_policy=3), 3), (dict(k_policy=-1), 3), (dict(k_policy=2, k_granule=0), 2),
    (dict(k_policy=2, k_granule=3), 2),
    (dict(router=2, dtype=0), 3),
    (dict(routed_scale=float("inf")), 2),
    (dict(weight_layout=2), 3), (dict(weight_layout=-1), 3),
])
def test_bad_descriptors_rejected(kw, code):
    assert _ws(_desc(**kw), moe.MOE_OP_FORWARD)[0] == code


def test_entry_points_validate_before_launch():
    lib = _lib.load()
    # the split-K router, which needs a workspace (the small-batch router needs none)
    d = _desc(T=4, d=128, E=4, I=128, k_max=2, router=moe.MOE_ROUTER_FLOAT64)
    P = lambda v: ctypes.c_void_p(v)
    # NULL pointers
    assert lib.moe_route(ctypes.byref(d), None, None, None, None, None, None, None, None, None, 0, None) == 1
    assert lib.moe_forward(ctypes.byref(d), *([None] * 14), 0, None) == 1
    assert lib.moe_combine(ctypes.byref(d), None, None, None, None, None, None, None) == 1
    # workspace too small (all other pointers plausible, never dereferenced)
    fake = [P(4096 * (i + 1)) for i in range(8)]
    assert lib.moe_route(ctypes.byref(d), *fake[:7], None, P(1 << 20), 16, None) == 4
    # misaligned activation
    assert lib.moe_route(ctypes.byref(d), P(4098), *fake[1:7], None, P(1 << 20), 1 << 30, None) == 5
    # the grouped-GEMM FFN needs its workspace (tile table) and is bf16 only
    dg = _desc(T=4, d=128, E=4, I=128, k_max=2, path=moe.MOE_PATH_GEMM)
    assert lib.moe_ffn_gateup(ctypes.byref(dg), *fake[:6], None, 0, None) == 4
    assert lib.moe_ffn_down(ctypes.byref(dg), *fake[:4], None, 0, None) == 4
    df = _desc(T=4, d=128, E=4, I=128, k_max=2, path=moe.MOE_PATH_GEMM, dtype=moe.MOE_F32)
    assert lib.moe_ffn_gateup(ctypes.byref(df), *fake[:6], None, 0, None) == 3
    assert lib.moe_ffn_plan(ctypes.byref(dg), fake[0], None, 0, None) == 4
    assert lib.moe_ffn_plan(ctypes.byref(dg), None, None, 0, None) in (1, 4)
    assert lib.moe_status_str(4) == b"workspace missing or too small"
    with pytest.raises(moe.MoeError):
        moe._check("x", 2)


def test_resolve_path_rule():
    """AUTO: grouped GEMM for bf16 when T*k_max >= 64*E (routed) / T >= 256 (shared)."""
    import mixture_experts_layer_token_amd as m
    cases = [((64, 4096, 8, 14336, 2), "stream"), ((8192, 2048, 256, 384, 32), "gemm"),
             ((4096, 7168, 256, 2048, 8), "gemm"), ((128, 7168, 256, 2048, 8), "stream"),
             ((256, 2048, 128, 768, 8), "stream"), ((512, 128, 8, 128, 1), "gemm")]
    for (T, d, E, I, km), want in cases:
        assert m.resolve_path(m.make_desc(T, d, E, I, km))[0] == want
    assert m.resolve_path(m.make_desc(4096, 128, 8, 128, 2, I_shared=128))[1] == "gemm"
    assert m.resolve_path(m.make_desc(128, 128, 8, 128, 2, I_shared=128))[1] == "stream"
    assert m.resolve_path(m.make_desc(8192, 2048, 256, 384, 32, path="stream")) == ("stream", "stream")
    import torch
    assert m.resolve_path(m.make_desc(8192, 256, 8, 128, 8, dtype=torch.float32)) == ("stream", "stream")
    with pytest.raises(m.MoeError):
        m.resolve_path(m.make_desc(64, 256, 8, 128, 2, dtype=torch.float32, path="gemm"))


def test_fold_validates_before_launch():
    lib = _lib.load()
    d = _desc(T=4, d=128, E=4, I=128, k_max=2)
    P = lambda v: ctypes.c_void_p(v)
    x = P(1 << 20)  # never dereferenced: every call below fails validation first
    args = lambda mode, budget, **kw: [ctypes.byref(kw.get("desc", d)), mode, budget] + \
        [kw.get(n, x) for n in ("S", "L", "H", "tok_off", "ids", "w", "eoff", "psrc", "to", "io", "wo")] + \
        [None, kw.get("ws", None), kw.get("ws_bytes", 0), None]
    assert lib.moe_fold(*args(7, 2)) == 3                      # unknown mode
    assert lib.moe_fold(*args(0, 0)) == 2                      # budget < 1
    assert lib.moe_fold(*args(0, 2, desc=_desc(T=4, d=128, E=128, I=128, k_max=65))) == 2
    assert lib.moe_fold(*args(0, 2, S=None)) == 1
    assert lib.moe_fold(*args(1, 2, eoff=None)) == 1          # pool mode needs the permutation
    assert lib.moe_fold(*args(0, 2)) == 4                      # workspace missing
    st, n = _ws(d, moe.MOE_OP_FOLD)
    assert st == 0 and n > 0 and n <= _ws(d, moe.MOE_OP_FORWARD)[1]


def test_proxy_kappa_table_matches_oracle():
    """The library's host-side kappa table against the oracle's balanced split."""
    import oracle
    for k_max, m, N in [(32, 8, 4), (7, 3, 4), (1, 1, 1), (0, 2, 2), (64, 16, 4), (12, 4, 3)]:
        got = moe.moe_proxy_kappa_balanced(k_max, m, N).tolist()
        assert got == [oracle.kappa_balanced(k, m, N) for k in range(k_max + 1)]
    for k_max, m, N in [(9, 2, 4), (1, 0, 4), (1, 2, 0), (-1, 2, 2)]:
        with pytest.raises(moe.MoeError):
            moe.moe_proxy_kappa_balanced(k_max, m, N)
    assert _lib.load().moe_proxy_kappa_balanced(4, 2, 2, None) == 1


def test_proxy_validates_before_launch():
    lib = _lib.load()
    d = _desc(T=4, d=128, E=16, I=128, k_max=8)
    P = lambda v: ctypes.c_void_p(v)
    x = P(1 << 20)  # never dereferenced: every call below fails validation first
    route = lambda N, r, m, desc=d, **kw: lib.moe_proxy_route(
        ctypes.byref(desc), N, r, m, *[kw.get(n, x) for n in ("k", "kappa", "bto", "bids", "bw", "beo", "bpt", "bps",
                                                               "x", "pg", "pu", "to", "ids", "w")], None, None)
    assert route(3, 8, 4) == 2                     # E not a multiple of N
    assert route(4, 8, 1) == 2                     # k_max > m*N
    assert route(4, 0, 2) == 2                     # r < 1
    assert route(4, 8, 5) == 2                     # m > E/N
    assert route(4, 129, 2) == 2                   # r > I
    big = _desc(T=4, d=128, E=256, I=128, k_max=8)
    assert route(4, 8, 17, desc=big) == 2          # m*N > 64
    assert route(4, 8, 2, x=None) == 1
    assert route(4, 8, 2, pu=None) == 1
    assert route(4, 8, 2, beo=None) == 1
    assert route(4, 8, 2, kappa=None) == 1
    assert route(4, 8, 2, pg=P((1 << 20) + 2)) == 5  # packed weights not 16-byte aligned
    pack = lambda N, r, **kw: lib.moe_proxy_pack(ctypes.byref(d), N, r, *[kw.get(n, x) for n in (
        "gi", "wg", "wu", "pg", "pu")], None)
    assert pack(3, 8) == 2
    assert pack(4, 8, gi=None) == 1
    assert pack(4, 8, pg=P((1 << 20) + 2)) == 5


def test_path_table_validates_on_the_host():
    lib = _lib.load()
    P = ctypes.c_void_p
    n = ctypes.c_size_t(0)
    assert lib.moe_path_table_bytes(6, ctypes.byref(n)) == 0 and n.value == 72
    assert lib.moe_path_table_bytes(0, ctypes.byref(n)) == 2
    assert lib.moe_path_table_bytes(1025, ctypes.byref(n)) == 2
    i32 = lambda v: (ctypes.c_int32 * len(v))(*v)
    f32 = lambda v: (ctypes.c_float * len(v))(*v)
    fake = P(1 << 20)   # never written: every call below fails validation first
    call = lambda E, s, t, b: lib.moe_path_table(E, len(s), i32(s), i32(t), f32(b), fake, 12 * len(s), None)
    assert call(3, [0, 1, 1], [0, 2, 1], [0, 0, 0]) == 2          # not increasing
    assert call(3, [0, 0], [1, 1], [0, 0]) == 2                   # duplicate
    assert call(3, [0, 3], [0, 0], [0, 0]) == 2                   # source out of range
    assert call(3, [0, 1], [0, -1], [0, 0]) == 2                  # target out of range
    assert call(3, [0, 1], [0, 1], [0, float("nan")]) == 2        # bias not finite
    assert lib.moe_path_table(3, 1, None, i32([0]), f32([0]), fake, 12, None) == 1
    assert lib.moe_path_table(3, 1, i32([0]), i32([0]), f32([0]), P((1 << 20) + 4), 12, None) == 5


def test_path_route_validates_before_launch():
    lib = _lib.load()
    d = _desc(T=4, d=128, E=8, I=128, k_max=2)
    x = ctypes.c_void_p(1 << 20)
    route = lambda P, lam=0.5, desc=d, **kw: lib.moe_path_route(
        ctypes.byref(desc), kw.get("x", x), x, None, None, lam, kw.get("table", x), P,
        *[kw.get(n, x) for n in ("k", "to", "src", "tgt", "w")], None, kw.get("ws", None), 0, None)
    assert route(1) == 2                                     # k_max > P
    assert route(2000) == 2                                  # P too large
    assert route(8, lam=float("inf")) == 2
    assert route(8, table=None) == 1
    assert route(8) == 4                                     # workspace missing
    assert route(8, desc=_desc(T=4, d=128, E=128, I=128, k_max=65)) == 2
    st, n = _ws(d, moe.MOE_OP_PATH)
    assert st == 0 and 0 < n <= _ws(d, moe.MOE_OP_FORWARD)[1]
    assert lib.moe_path_sources(ctypes.byref(d), None, x, x, x, x, x, None, 0, None) == 1
    assert lib.moe_ffn_down_rows(ctypes.byref(d), x, None, x, x, x, None, 0, None) in (1, 4)


def test_pack_weights_validates_before_launch():
    lib = _lib.load()
    P = lambda v: ctypes.c_void_p(v)
    a, b = P(1 << 20), P(1 << 30)
    bf, f32 = moe.MOE_BF16, moe.MOE_F32
    assert lib.moe_pack_weights(7, 1, 64, 128, a, b, None) == 3             # dtype
    assert lib.moe_pack_weights(bf, -1, 64, 128, a, b, None) == 2           # G < 0
    assert lib.moe_pack_weights(bf, 1, 96, 128, a, b, None) == 2            # N % 64
    assert lib.moe_pack_weights(bf, 1, 64, 96, a, b, None) == 2             # K % 64 (bf16)
    assert lib.moe_pack_weights(f32, 1, 64, 48, a, b, None) == 2            # K % 32 (fp32)
    assert lib.moe_pack_weights(bf, 1 << 20, 1 << 14, 1 << 14, a, b, None) == 2  # 2^48 elements
    assert lib.moe_pack_weights(bf, 1, 64, 128, None, b, None) == 1         # NULL
    assert lib.moe_pack_weights(bf, 1, 64, 128, P((1 << 20) + 8), b, None) == 5  # alignment
    assert lib.moe_pack_weights(bf, 2, 64, 128, a, P((1 << 20) + 64 * 128 * 2), None) == 2  # overlap
    assert lib.moe_pack_weights(bf, 0, 64, 128, None, None, None) == 0      # empty: nothing launched


def test_noalloc_rejects_layers_beyond_its_scratch():
    """moe_forward_noalloc checks the descriptor and the scratch size on the
    host before touching the device: a layer whose forward needs more than the
    library-held array is refused with MOE_ERR_SCRATCH, a bad descriptor with
    the usual code."""
    lib = _lib.load()
    big = _desc(T=8192, d=2048, E=256, I=384, k_max=32)   # the sub-expert prefill batch: ~1.2 GB of scratch
    assert lib.moe_forward_noalloc(ctypes.byref(big), *([None] * 14)) == 7
    assert lib.moe_status_str(7) == b"the layer needs more scratch than the library-held array holds"
    assert lib.moe_forward_noalloc(ctypes.byref(_desc(E=0)), *([None] * 14)) == 2
    assert lib.moe_forward_noalloc(None, *([None] * 14)) == 1
    assert _lib.MOE_NOALLOC_SCRATCH_BYTES == 64 << 20
