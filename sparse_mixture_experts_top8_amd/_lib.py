"""ctypes binding of ``libmoe_gfx950.so`` (declared in include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP library.
PyTorch supplies device memory and the current stream.  There is no fallback:
if the library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_gfx950.so")

MOE_OK = 0
MOE_ERR_NULL = 1
MOE_ERR_SHAPE = 2
MOE_ERR_ALIGN = 3
MOE_ERR_WORKSPACE = 4
MOE_ERR_DEVICE = 5
MOE_ERR_LAUNCH = 6
MOE_ERR_MEMORY = 7
MOE_ERR_TIMEOUT = 8

# Exported entry points, as include/moe.h declares them.
EXPORTS = ("moe_workspace_bytes", "moe_validate", "moe_route", "moe_load_balance", "moe_forward",
           "moe_block_forward", "moe_rmsnorm", "moe_ranks", "moe_tile_experts", "moe_expert_cache_bytes", "moe_forward_streamed",
           "moe_forward_traced", "moe_workspace_control_bytes", "moe_workspace_status", "moe_set_wait_budget_us",
           "moe_forward_noalloc", "moe_strerror", "moe_last_error")


class MoeLayerT(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("expert_inner", ctypes.c_int32),
        ("shared_inner", ctypes.c_int32),
        ("router_w", ctypes.c_void_p),
        ("gate_up_w", ctypes.c_void_p),
        ("down_w", ctypes.c_void_p),
        ("shared_gate_w", ctypes.c_void_p),
        ("shared_up_w", ctypes.c_void_p),
        ("shared_down_w", ctypes.c_void_p),
        ("shared_expert_gate_w", ctypes.c_void_p),
        ("logits_bf16", ctypes.c_int32),
        ("experts_tiled", ctypes.c_int32),
    ]


class MoeError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: status {code} ({strerror(code)}): {last_error()}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          f"or python sparse_mixture_experts_top8_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    L = ctypes.POINTER(MoeLayerT)
    lib.moe_workspace_bytes.argtypes = [L, ctypes.c_int64]
    lib.moe_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_validate.argtypes = [L, P, ctypes.c_int64, P, P, ctypes.c_size_t]
    lib.moe_validate.restype = ctypes.c_int
    lib.moe_route.argtypes = [L, P, ctypes.c_int64, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_route.restype = ctypes.c_int
    lib.moe_load_balance.argtypes = [L, P, ctypes.c_int64, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_load_balance.restype = ctypes.c_int
    lib.moe_forward.argtypes = [L, P, ctypes.c_int64, P, P, ctypes.c_size_t, P]
    lib.moe_forward.restype = ctypes.c_int
    lib.moe_block_forward.argtypes = [L, P, ctypes.c_float, P, ctypes.c_int64, P, P, ctypes.c_size_t, P]
    lib.moe_block_forward.restype = ctypes.c_int
    lib.moe_rmsnorm.argtypes = [P, ctypes.c_float, P, ctypes.c_int64, ctypes.c_int64, P, P]
    lib.moe_rmsnorm.restype = ctypes.c_int
    lib.moe_tile_experts.argtypes = [L, P, P, P]
    lib.moe_tile_experts.restype = ctypes.c_int
    lib.moe_expert_cache_bytes.argtypes = [L, ctypes.c_int32]
    lib.moe_expert_cache_bytes.restype = ctypes.c_size_t
    lib.moe_forward_streamed.argtypes = [L, P, ctypes.c_int64, P, P, ctypes.c_size_t, P, ctypes.c_size_t, P]
    lib.moe_forward_streamed.restype = ctypes.c_int
    lib.moe_ranks.argtypes = [P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, P, P]
    lib.moe_ranks.restype = ctypes.c_int
    lib.moe_forward_traced.argtypes = [L, P, ctypes.c_int64, P, P, ctypes.c_size_t, P, P]
    lib.moe_forward_traced.restype = ctypes.c_int
    lib.moe_workspace_control_bytes.argtypes = []
    lib.moe_workspace_control_bytes.restype = ctypes.c_size_t
    lib.moe_workspace_status.argtypes = [P, ctypes.c_size_t, P, ctypes.POINTER(ctypes.c_uint32)]
    lib.moe_workspace_status.restype = ctypes.c_int
    lib.moe_set_wait_budget_us.argtypes = [ctypes.c_int64]
    lib.moe_set_wait_budget_us.restype = ctypes.c_int64
    lib.moe_forward_noalloc.argtypes = [L, P, ctypes.c_int64, P, P]
    lib.moe_forward_noalloc.restype = ctypes.c_int
    lib.moe_strerror.argtypes = [ctypes.c_int]
    lib.moe_strerror.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


def strerror(code: int) -> str:
    return lib.moe_strerror(int(code)).decode()


def last_error() -> str:
    return lib.moe_last_error().decode()
