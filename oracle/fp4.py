"""FP4 E2M1 codes with E8M0 block scales, decoded to float64 (oracle; test infrastructure only).

Format, from "Add DeepSeek V4 Flash CPU inference with NVMe expert streaming"
(PR #165, the review question on V4 sizes): routed experts store FP4 E2M1
values with one UE8M0 scale per group of 32 values.  Layout reading (the pages
name no byte layout for the GPU): a matrix with N output rows and reduction
length K is stored row-major as codes [N][K/2] and scales [N][K/32]; within a
code byte the low nibble is element 2i and the high nibble element 2i+1; scale
j of a row covers elements 32j .. 32j+31 of that row.
"""
from __future__ import annotations

import struct

import numpy as np


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit.

    Exponent field 0 is subnormal: magnitude = mantissa * 0.5.
    Otherwise magnitude = 2^(exp-1) * (1 + mantissa/2).
    """
    if not 0 <= code <= 15:
        raise ValueError(code)
    sign = -1.0 if code & 8 else 1.0
    exp = (code >> 1) & 3
    man = code & 1
    mag = man * 0.5 if exp == 0 else 2.0 ** (exp - 1) * (1.0 + man / 2.0)
    return sign * mag


# The 16-entry table (64 bytes as float32, as the PR #165 NEON comment notes).
E2M1_VALUES = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e8m0_value(s: int) -> float:
    """Scale of an E8M0 byte built from its bit pattern: the float32 whose bits are s << 23.

    "DeepSeek V4: the CUDA kernels, as a tier rather than an engine" (PR #772),
    the maintainer's note on the Kimi K3 MXFP4 decode: building the exponent as
    a bit pattern gives s=0 -> +0 and s=255 -> +inf.
    """
    if not 0 <= s <= 255:
        raise ValueError(s)
    return struct.unpack("<f", struct.pack("<I", (int(s) << 23) & 0xFFFFFFFF))[0]


E8M0_VALUES = np.array([e8m0_value(s) for s in range(256)], dtype=np.float64)


def dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decode codes [N][K/2] (uint8) and scales [N][K/32] (uint8) to float64 [N][K].

    Element (n, k) = E2M1(nibble k of row n) * E8M0(scale k // 32 of row n),
    formed in float64 (exact: every product is a short binary fraction).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    n, half_k = codes.shape
    k = 2 * half_k
    if scales.shape != (n, k // 32) or k % 32:
        raise ValueError(f"scales shape {scales.shape} does not match codes {codes.shape}")
    # byte b -> (value of its low nibble, value of its high nibble): elements 2i and 2i+1
    byte = np.arange(256)
    pair = np.stack([E2M1_VALUES[byte & 0x0F], E2M1_VALUES[byte >> 4]], axis=1)   # [256][2]
    vals = pair[codes].reshape(n, k // 32, 32)   # [N][K/32][32]: block j holds elements 32j..32j+31
    s = E8M0_VALUES[scales]                       # [N][K/32]
    with np.errstate(invalid="ignore"):          # 0 * inf (s=255) is NaN, as in float math
        return (vals * s[:, :, None]).reshape(n, k)
