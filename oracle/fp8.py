"""FP8 E4M3 weights with one float32 scale per 128 x 128 block, decoded to float64 (oracle; test
infrastructure only).

Format, from "Add DeepSeek V4 Flash CPU inference with NVMe expert streaming" (PR #165, the
question "Is the engine config-driven across V4 sizes?"): the V4 checkpoints store their dense
tensors as FP8 E4M3 with 128 x 128 block scales.  The E4M3 decode follows the same page's notes
on the FP8 attention kernels (the fp32 value is built from the E4M3 fields, denormals included):
1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal,
magnitude m/8 * 2^-6; the pattern S.1111.111 is NaN; there is no infinity (largest finite 448).

Readings where the pages are silent: a block's scale is a float32 (one per 128 output rows x 128
reduction values) and an element is E4M3(code) * scale; a matrix with N output rows and
reduction length K is stored row-major as codes [N][K] (one byte per value) and scales
[ceil(N/128)][ceil(K/128)].
"""
from __future__ import annotations

import math

import numpy as np

FP8_BLOCK = 128


def e4m3_value(code: int) -> float:
    """Value of an 8-bit E4M3 code (NaN for 0x7F and 0xFF; code 0x80 is -0)."""
    if not 0 <= code <= 255:
        raise ValueError(code)
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 15 and man == 7:
        return math.nan
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3_VALUES = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


class Fp8Matrix:
    """One FP8 matrix of an expert: codes [N][K] uint8 and float32 block scales
    [ceil(N/128)][ceil(K/128)] (a plain holder, so it is never unpacked as an FP4 pair)."""

    def __init__(self, codes, scales):
        self.codes = np.asarray(codes, dtype=np.uint8)
        self.scales = np.asarray(scales, dtype=np.float32)
        n, k = self.codes.shape
        if self.scales.shape != (-(-n // FP8_BLOCK), -(-k // FP8_BLOCK)):
            raise ValueError(f"scales {self.scales.shape} do not fit codes {self.codes.shape}")


def dequant_fp8_block(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decode codes [N][K] with block scales [ceil(N/128)][ceil(K/128)] to float64 [N][K]:
    element (n, k) = E4M3(codes[n][k]) * scales[n // 128][k // 128] (exact in float64)."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.float32).astype(np.float64)
    n, k = codes.shape
    if scales.shape != (-(-n // FP8_BLOCK), -(-k // FP8_BLOCK)):
        raise ValueError(f"scales {scales.shape} do not fit codes {codes.shape}")
    rows = np.arange(n) // FP8_BLOCK
    cols = np.arange(k) // FP8_BLOCK
    return E4M3_VALUES[codes] * scales[rows[:, None], cols[None, :]]
