"""ctypes view of the C ABI in include/moe.h (no arithmetic here)."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

c_i32 = ctypes.c_int32
c_ptr = ctypes.c_void_p
c_size = ctypes.c_size_t

MOE_F32, MOE_BF16 = 0, 1
MOE_PATH_AUTO, MOE_PATH_STREAM, MOE_PATH_GEMM = 0, 1, 2
MOE_ROUTER_AUTO, MOE_ROUTER_FLOAT64, MOE_ROUTER_SCREENED, MOE_ROUTER_FUSED = 0, 1, 2, 3
MOE_K_EXACT, MOE_K_BATCH_MAX, MOE_K_ROUND_UP = 0, 1, 2
MOE_OP_ROUTE, MOE_OP_PERMUTE, MOE_OP_FFN, MOE_OP_COMBINE, MOE_OP_FORWARD, MOE_OP_FOLD, MOE_OP_PATH = 0, 1, 2, 3, 4, 5, 6
MOE_FOLD_TOKEN, MOE_FOLD_POOL = 0, 1
MOE_DEV_BAD_K = 1
MOE_W_ROWMAJOR, MOE_W_BLOCKED64 = 0, 1
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20

STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_UNSUPPORTED",
                4: "MOE_ERR_WORKSPACE", 5: "MOE_ERR_ALIGN", 6: "MOE_ERR_LAUNCH", 7: "MOE_ERR_SCRATCH"}


class moe_desc(ctypes.Structure):
    _fields_ = [("T", c_i32), ("d", c_i32), ("E", c_i32), ("I", c_i32), ("k_max", c_i32),
                ("I_shared", c_i32), ("dtype", c_i32), ("path", c_i32), ("router", c_i32),
                ("routed_scale", ctypes.c_float), ("k_policy", c_i32), ("k_granule", c_i32),
                ("weight_layout", c_i32)]


_P = ctypes.POINTER(moe_desc)

# name -> argument types (return type is int: moe_status), as in include/moe.h
SIGNATURES = {
    "moe_workspace_size": [_P, c_i32, ctypes.POINTER(c_size)],
    "moe_resolve_path": [_P, ctypes.POINTER(c_i32), ctypes.POINTER(c_i32)],
    "moe_pack_weights": [c_i32, c_i32, c_i32, c_i32, c_ptr, c_ptr, c_ptr],
    "moe_route": [_P, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_size, c_ptr],
    "moe_permute": [_P, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_size, c_ptr],
    "moe_ffn": [_P, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr,
                c_ptr, c_size, c_ptr],
    "moe_ffn_plan": [_P, c_ptr, c_ptr, c_size, c_ptr],
    "moe_ffn_gateup": [_P, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_size, c_ptr],
    "moe_ffn_down": [_P, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_size, c_ptr],
    "moe_combine": [_P, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr],
    "moe_fold": [_P, c_i32, c_i32, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr,
                 c_ptr, c_ptr, c_ptr, c_size, c_ptr],
    "moe_path_table_bytes": [c_i32, ctypes.POINTER(c_size)],
    "moe_path_table": [c_i32, c_i32, c_ptr, c_ptr, c_ptr, c_ptr, c_size, c_ptr],
    "moe_path_route": [_P, c_ptr, c_ptr, c_ptr, c_ptr, ctypes.c_float, c_ptr, c_i32, c_ptr, c_ptr, c_ptr, c_ptr,
                       c_ptr, c_ptr, c_ptr, c_size, c_ptr],
    "moe_path_sources": [_P, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_size, c_ptr],
    "moe_path_rows": [_P, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr],
    "moe_ffn_down_rows": [_P, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_size, c_ptr],
    "moe_proxy_kappa_balanced": [c_i32, c_i32, c_i32, c_ptr],
    "moe_proxy_pack": [_P, c_i32, c_i32, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr],
    "moe_proxy_route": [_P, c_i32, c_i32, c_i32, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr,
                        c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr],
    "moe_forward": [_P, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr,
                    c_ptr, c_ptr, c_ptr, c_ptr, c_size, c_ptr],
    "moe_probe_read": [c_ptr, c_size, c_i32, c_ptr, c_ptr],
    "moe_forward_noalloc": [_P, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr,
                            c_ptr, c_ptr, c_ptr, c_ptr],
    "moe_status_str": [c_i32],
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libmoe_mi355x.so from the package directory.  Raises if it has not
    been built: there is no other implementation to fall back on."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m mixture_experts_layer_token_amd.build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    for name, args in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "moe_status_str" else c_i32
    _lib = lib
    return lib
