"""Chained decode across layers, written out plainly in float64 (oracle; test infrastructure only).

The pages run the MoE stage once per transformer layer in decode ("feat(v4/cuda): the CUDA tier
wired into the DeepSeek V4 engine", PR #1055, "What it is": decode fuses routed and shared experts
in one MoE stage per layer; "Add DeepSeek V4 Flash CPU inference with NVMe expert streaming",
PR #165: 43 layers for V4 Flash).  They do not spell out what joins one layer's MoE output to the
next layer's input.  The reading taken here is the plainest pre-norm residual stream, with the
attention block and V4's hyper-connection mixing left out (they are not on the MoE path):

    x_l     = bf16( RMSNorm(h_l) * gamma_l )          the layer's MoE input
    y_l     = MoE_l(x_l)                              the layer (oracle.moe.moe_forward)
    h_{l+1} = h_l + y_l                               the residual stream

    RMSNorm(v) = v / sqrt(mean(v^2) + eps),   eps = 1e-6

h_0 is the residual-stream input of the first layer.  Everything is float64; the bf16 rounding is
round-to-nearest-even of the float64 value.
"""
from __future__ import annotations

import numpy as np

from .moe import moe_forward

RMS_EPS = 1e-6


def rms_norm(h, gamma, eps: float = RMS_EPS) -> np.ndarray:
    """Rows of ``h`` [T][H] divided by the root of (mean of their squares + eps), times ``gamma`` [H]."""
    h = np.asarray(h, dtype=np.float64)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


def f64_to_bf16_bits(v) -> np.ndarray:
    """Round float64 values to bfloat16 (nearest, ties to even) and return the 16-bit patterns.

    bfloat16 keeps 8 significant bits: a normal value m * 2^e (1 <= m < 2) is rounded on the grid of
    spacing 2^(e-7); below 2^-126 the grid stays at 2^-133 (subnormals).  Results past the largest
    finite value become infinities; NaN becomes the quiet NaN 0x7FC0."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.where(np.signbit(v), 0x8000, 0).astype(np.int64)
    a = np.abs(v)
    finite = np.isfinite(a)
    af = np.where(finite, a, 0.0)
    _, ex = np.frexp(af)                           # af = f * 2^ex with 1/2 <= f < 1 (ex = 0 for 0)
    e = np.maximum(ex.astype(np.int64) - 1, -126)  # af = m * 2^e with 1 <= m < 2, or the subnormal grid
    q = np.rint(np.ldexp(af, (7 - e).astype(np.int32)))   # exact scaling by a power of two, then ties to even
    up = q == 256.0                                 # rounded up to the next power of two
    q = np.where(up, 128.0, q).astype(np.int64)
    e = e + up
    normal = q >= 128
    bits = np.where(normal, ((e + 127) << 7) | (q - 128), q)
    bits = np.where(finite & (e > 127), 0x7F80, bits)      # overflow
    bits = np.where(np.isinf(a), 0x7F80, bits)
    bits = bits | sign
    bits = np.where(np.isnan(v), 0x7FC0, bits)
    return bits.astype(np.uint16)


def norm_input(h, gamma, eps: float = RMS_EPS) -> np.ndarray:
    """A layer's MoE input: bf16 bit patterns of RMSNorm(h) * gamma."""
    return f64_to_bf16_bits(rms_norm(h, gamma, eps))


def chain_forward(h_in, gammas, routers, biases, experts, top_k: int, n_shared: int, eps: float = RMS_EPS,
                  routed_scale: float = 1.0):
    """Run the layers in order from the residual input ``h_in`` [T][H].

    ``gammas[l]`` [H], ``routers[l]`` [E][H], ``biases[l]`` [E] or None and ``experts[l]`` (the
    per-group weights ``moe_forward`` takes) describe layer l.  Returns dict(x=[bf16 bits per
    layer], y=[float64 per layer], route=[moe_forward's routing per layer], h=float64 h_L)."""
    h = np.asarray(h_in, dtype=np.float64).copy()
    xs, ys, routes = [], [], []
    for l in range(len(routers)):
        x = norm_input(h, gammas[l], eps)
        out = moe_forward(x, routers[l], biases[l], experts[l], top_k, n_shared, routed_scale)
        h = h + out["y"]
        xs.append(x)
        ys.append(out["y"])
        routes.append({k: out[k] for k in ("idx", "w", "counts", "offsets", "perm")})
    return dict(x=xs, y=ys, route=routes, h=h)
