"""Routed FP4-expert MoE layer for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libmoe_fp4.so`` behind the C ABI in
``include/moe.h``; this package is a thin ctypes binding over it.
"""
from ._lib import load as load_library, MoeError, LIB_PATH
from .layer import MoeLayer, MoeBank, MoeChain, residual_rmsnorm, pack_fp4, pack_fp8, kernel_scale_shape, device_supported, timing_enable, timing_read, timing_reset

__all__ = ["load_library", "MoeError", "LIB_PATH", "MoeLayer", "MoeBank", "MoeChain", "residual_rmsnorm", "pack_fp4", "pack_fp8", "kernel_scale_shape", "device_supported", "timing_enable",
           "timing_read", "timing_reset"]
