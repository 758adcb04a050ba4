"""ctypes view of the C ABI in include/moe.h (argument marshalling only).

The shared library is the in-tree ``libmoe_fp4.so`` built by ``build.py``.  Loading
fails loudly when it is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_fp4.so")

MOE_ABI_VERSION = 2
MOE_SHARED_FP8 = 1
MOE_CHAIN_RESIDUAL = 1
MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_ALLOC = range(6)
MOE_PATH_AUTO, MOE_PATH_GEMV, MOE_PATH_GEMM = range(3)
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20

# Every symbol include/moe.h declares.
EXPORTS = ("moe_abi_version", "moe_device_supported", "moe_layer_create", "moe_layer_destroy",
           "moe_workspace_bytes", "moe_route", "moe_forward", "moe_forward_noalloc", "moe_pack_fp4",
           "moe_pack_fp8", "moe_residual_rmsnorm", "moe_chain_create", "moe_chain_run", "moe_chain_destroy",
           "moe_bank_create", "moe_bank_forward", "moe_bank_stats", "moe_bank_destroy",
           "moe_status_string",
           "moe_last_error",
           "moe_timing_enable", "moe_timing_read", "moe_timing_reset")


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("n_shared", ctypes.c_int32),
        ("inter", ctypes.c_int32),
        ("path", ctypes.c_int32),
        ("device", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("routed_scale", ctypes.c_float),
        ("reserved", ctypes.c_int32),
        ("w_router", ctypes.c_void_p),
        ("router_bias", ctypes.c_void_p),
        ("gate_codes", ctypes.c_void_p),
        ("gate_scales", ctypes.c_void_p),
        ("up_codes", ctypes.c_void_p),
        ("up_scales", ctypes.c_void_p),
        ("down_codes", ctypes.c_void_p),
        ("down_scales", ctypes.c_void_p),
        ("shared_gate_fp8", ctypes.c_void_p),
        ("shared_gate_fp8_scales", ctypes.c_void_p),
        ("shared_up_fp8", ctypes.c_void_p),
        ("shared_up_fp8_scales", ctypes.c_void_p),
        ("shared_down_fp8", ctypes.c_void_p),
        ("shared_down_fp8_scales", ctypes.c_void_p),
    ]


class RouteOut(ctypes.Structure):
    _fields_ = [
        ("idx", ctypes.c_void_p),
        ("weight", ctypes.c_void_p),
        ("counts", ctypes.c_void_p),
        ("offsets", ctypes.c_void_p),
        ("perm", ctypes.c_void_p),
    ]


class ChainDesc(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32),
        ("n_layers", ctypes.c_int32),
        ("tokens", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("reserved", ctypes.c_int32),
        ("layers", ctypes.POINTER(ctypes.c_void_p)),
        ("norm_weight", ctypes.POINTER(ctypes.c_void_p)),
        ("h_in", ctypes.c_void_p),
        ("h_out", ctypes.c_void_p),
        ("x", ctypes.c_void_p),
        ("y", ctypes.c_void_p),
        ("routes", ctypes.POINTER(RouteOut)),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_uint64),
    ]


_lib = None


def load(path: str = None) -> ctypes.CDLL:
    """Load (once) and type the C ABI.  Raises if the library was not built.

    ``MOE_LIB`` in the environment names another build of the same library (A/B runs)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("MOE_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is missing; run fp4_routed_expert_moe_amd/build.py "
                           "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    P, I32, U64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64
    sig = {
        "moe_abi_version": (I32, []),
        "moe_device_supported": (I32, [I32, ctypes.c_char_p, I32]),
        "moe_layer_create": (I32, [ctypes.POINTER(LayerDesc), ctypes.POINTER(P)]),
        "moe_layer_destroy": (None, [P]),
        "moe_workspace_bytes": (U64, [P, I32]),
        "moe_route": (I32, [P, P, I32, ctypes.POINTER(RouteOut), P, U64, P]),
        "moe_forward": (I32, [P, P, I32, P, ctypes.POINTER(RouteOut), P, U64, P]),
        "moe_forward_noalloc": (I32, [P, P, I32, P, ctypes.POINTER(RouteOut), P]),
        "moe_pack_fp4": (I32, [P, P, P, P, I32, I32, I32, P]),
        "moe_pack_fp8": (I32, [P, P, I32, I32, I32, P]),
        "moe_residual_rmsnorm": (I32, [P, P, P, P, ctypes.c_float, P, I32, I32, P]),
        "moe_chain_create": (I32, [ctypes.POINTER(ChainDesc), ctypes.POINTER(P)]),
        "moe_chain_run": (I32, [P, P]),
        "moe_chain_destroy": (None, [P]),
        "moe_bank_create": (I32, [P, I32, I32, ctypes.POINTER(P)]),
        "moe_bank_forward": (I32, [P, P, I32, P, ctypes.POINTER(RouteOut), P, U64, P]),
        "moe_bank_stats": (I32, [P, ctypes.POINTER(ctypes.c_int64)]),
        "moe_bank_destroy": (None, [P]),
        "moe_status_string": (ctypes.c_char_p, [I32]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_timing_enable": (I32, [I32]),
        "moe_timing_read": (I32, [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_int64),
                                  ctypes.POINTER(ctypes.c_double), I32]),
        "moe_timing_reset": (None, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.moe_abi_version() != MOE_ABI_VERSION:
        raise RuntimeError("libmoe_fp4.so ABI version mismatch")
    _lib = lib
    return lib


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def check(status: int, lib=None):
    if status != MOE_OK:
        lib = lib or load()
        raise MoeError(status, f"{lib.moe_status_string(status).decode()}: {lib.moe_last_error().decode()}")
