"""ctypes prototypes of libmoe.so (the C ABI declared in include/moe.h)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP = 0, -1, -2, -3
DTYPE = {"f32": 0, "bf16": 1}
ACT = {"relu": 0, "gelu": 1, "reglu": 2, "geglu": 3}
ROUTE = {"topk": 0, "rre": 1}
REGION = {"expert_idx": 0, "gate": 1, "slot": 2, "expert_count": 3, "slot_token": 4,
          "x_e": 5, "hidden": 6, "y_e": 7}

EXPORTS = ["moe_capacity", "moe_workspace_bytes", "moe_workspace_offset", "moe_router", "moe_router_aux",
           "moe_dispatch", "moe_expert_ffn", "moe_expert_ffn_fused", "moe_expert_up", "moe_expert_down", "moe_combine", "moe_forward", "moe_forward_noalloc", "moe_backward_workspace_bytes", "moe_backward", "moe_sparse_clip", "moe_last_error",
           "moe_version"]


class MoeConfig(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("d_model", ctypes.c_int64),
        ("d_ff", ctypes.c_int64),
        ("E", ctypes.c_int32),
        ("k", ctypes.c_int32),
        ("capacity_factor", ctypes.c_double),
        ("route", ctypes.c_int32),
        ("n_groups", ctypes.c_int32),
        ("rre_seed", ctypes.c_uint64),
        ("act", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load libmoe.so (built in-tree).  Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m sparse_mixture_experts_13_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    cfgp = ctypes.POINTER(MoeConfig)
    i64, i32 = ctypes.c_int64, ctypes.c_int32
    lib.moe_capacity.argtypes = [cfgp]
    lib.moe_capacity.restype = i64
    lib.moe_workspace_bytes.argtypes = [cfgp]
    lib.moe_workspace_bytes.restype = i64
    lib.moe_workspace_offset.argtypes = [cfgp, i32]
    lib.moe_workspace_offset.restype = i64
    lib.moe_router.argtypes = [cfgp, P, P, P, P, P, P, P, P]
    lib.moe_router.restype = ctypes.c_int
    lib.moe_router_aux.argtypes = [cfgp, P, P, P, P, P, ctypes.c_double, P, P, P]
    lib.moe_router_aux.restype = ctypes.c_int
    lib.moe_dispatch.argtypes = [cfgp, P, P, P, P, P, P, P, P]
    lib.moe_dispatch.restype = ctypes.c_int
    lib.moe_expert_ffn.argtypes = [cfgp, P, P, P, P, P, P, P]
    lib.moe_expert_ffn.restype = ctypes.c_int
    lib.moe_expert_ffn_fused.argtypes = [cfgp, P, P, P, P, P, P]
    lib.moe_expert_ffn_fused.restype = ctypes.c_int
    lib.moe_expert_up.argtypes = [cfgp, P, P, P, P, P]
    lib.moe_expert_up.restype = ctypes.c_int
    lib.moe_expert_down.argtypes = [cfgp, P, P, P, P, P]
    lib.moe_expert_down.restype = ctypes.c_int
    lib.moe_combine.argtypes = [cfgp, P, P, P, P, P, P]
    lib.moe_combine.restype = ctypes.c_int
    lib.moe_forward.argtypes = [cfgp, P, P, P, P, P, P, P, P, P]
    lib.moe_forward.restype = ctypes.c_int
    lib.moe_forward_noalloc.argtypes = [cfgp, P, P, P, P, P, P, P, P]
    lib.moe_forward_noalloc.restype = ctypes.c_int
    lib.moe_backward_workspace_bytes.argtypes = [cfgp]
    lib.moe_backward_workspace_bytes.restype = i64
    lib.moe_backward.argtypes = [cfgp] + [P] * 13
    lib.moe_backward.restype = ctypes.c_int
    lib.moe_sparse_clip.argtypes = [cfgp, P, P, P, P, ctypes.c_double, P, P, P]
    lib.moe_sparse_clip.restype = ctypes.c_int
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_version.argtypes = []
    lib.moe_version.restype = ctypes.c_char_p
    _lib = lib
    return lib
