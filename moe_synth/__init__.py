"""Seeded synthetic inputs for the routed FP4-expert MoE layer.

This module only draws numbers.  It holds none of the layer's arithmetic
(no routing, no FP4 decoding, no matrix products): it is the one piece that
both the GPU path (through the package and ``bench.py``) and the CPU oracle
(through ``tests/``) are allowed to share.

What is drawn, and from which workload description:

* Token activations ``x``: N(0, 1) in float32, rounded to bfloat16 with
  round-to-nearest-even and handed over as the raw 16-bit patterns.
* Chained decode (workloads with ``chained``): the residual-stream input
  ``h_0`` is N(0, 1) in float32 [T][H]; each layer's RMSNorm weight is
  1 + 0.1 * N(0, 1) in float32 [H].
* Router weights ``W_r``: N(0, 0.02^2) in float32, shape [E][H].
* Router bias: only for the skewed long-prefill workload, a Zipf(1.1)
  popularity prior ``b_e = -1.1 * ln(e + 1)`` (expert 0 most popular).
* Expert weights: e2m1 code bytes uniform on 0..255 (each nibble uniform on
  0..15) and e8m0 scale bytes uniform on {123..127}, i.e. 2^U{-4..0}.
* A shared expert stored in FP8 (workloads with ``shared_fp8``): E4M3 code
  bytes uniform on the 254 finite codes (a drawn 0x7F / 0xFF, the two NaN
  patterns, becomes 0x7E / 0xFE) and one float32 scale per 128 x 128 block,
  (0.5 + U[0,1)) * 2^-7 with U on a 2^-24 grid, which gives the shared expert
  about the same root-mean-square weight as the FP4 experts.

Workload shapes follow the DeepSeek V4 Flash expert dimensions quoted on
"Add DeepSeek V4 Flash CPU inference with NVMe expert streaming" (PR #165:
hidden 4096, 256 routed experts, expert inter 2048, six experts per token).

Expert weights are large (3.4 GB per layer at those shapes), so they come from
a counter-based generator (SplitMix64, Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014) written with plain int64 torch
ops.  The same function runs on a CPU tensor or a GPU tensor and yields the
same bytes, so the GPU can fill 55 GB in seconds while the oracle regenerates
any single expert matrix on the host.  The activations and router weights are
small and come from numpy's PCG64 generator on the host.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

SEED = 0

# ---------------------------------------------------------------------------
# Workloads (named by what they are)
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    hidden: int          # H
    experts: int         # E routed experts
    top_k: int           # k
    shared: int          # S always-on shared experts (0 or 1)
    inter: int           # I expert intermediate width
    tokens: int          # T tokens per layer call
    layers: int = 1      # independent layers (stacked decode)
    steps: int = 1       # decode steps (stacked decode)
    zipf: Optional[float] = None  # router popularity bias exponent
    scale_lo: int = 123  # e8m0 scale byte range (2^-4 .. 2^0)
    scale_hi: int = 127
    shared_fp8: bool = False  # shared expert in FP8 E4M3 with 128 x 128 block scales
    chained: bool = False     # layers joined by the residual stream (RMSNorm between them)

    @property
    def groups(self) -> int:
        return self.experts + self.shared

    @property
    def fp4_groups(self) -> int:
        """Groups stored in FP4: every group, or the routed experts only when the shared one is FP8."""
        return self.experts if self.shared_fp8 else self.groups


WORKLOADS = {
    "tiny": Workload("tiny", 256, 8, 2, 1, 128, 16),
    "decode_t8": Workload("decode_t8", 4096, 256, 6, 1, 2048, 8),
    "prefill_t512": Workload("prefill_t512", 4096, 256, 6, 1, 2048, 512),
    "prefill_t4096_zipf": Workload("prefill_t4096_zipf", 4096, 256, 6, 1, 2048, 4096, zipf=1.1),
    "stacked_decode_16l": Workload("stacked_decode_16l", 4096, 256, 6, 1, 2048, 1, layers=16, steps=256),
    # DeepSeek V4 Pro scale (hidden 7168, 384 experts, same expert format); intermediate 2048
    # and top-6 are readings (the pages give neither for Pro)
    "decode_pro_t8": Workload("decode_pro_t8", 7168, 384, 6, 1, 2048, 8),
    # the V4 Flash decode shape with the shared expert kept in the checkpoint's FP8 E4M3 format
    "decode_t8_fp8shared": Workload("decode_t8_fp8shared", 4096, 256, 6, 1, 2048, 8, shared_fp8=True),
    # one token through 16 V4 Flash MoE layers, each layer's input the RMSNorm of the residual stream
    "chained_decode_16l": Workload("chained_decode_16l", 4096, 256, 6, 1, 2048, 1, layers=16, steps=256,
                                   chained=True),
    # a 512-token prefill chunk at the V4 Pro scale (same readings as decode_pro_t8)
    "prefill_pro_t512": Workload("prefill_pro_t512", 7168, 384, 6, 1, 2048, 512),
}
_WORKLOAD_IDS = {n: i + 1 for i, n in enumerate(WORKLOADS)}

TENSOR_IDS = {
    "x": 1, "w_router": 2,
    "gate_codes": 3, "gate_scales": 4,
    "up_codes": 5, "up_scales": 6,
    "down_codes": 7, "down_scales": 8,
    "gate_fp8_codes": 9, "gate_fp8_scales": 10,
    "up_fp8_codes": 11, "up_fp8_scales": 12,
    "down_fp8_codes": 13, "down_fp8_scales": 14,
    "h_in": 15, "norm_weight": 16,
}
MATRICES = ("gate", "up", "down")


def workload(name_or_wl) -> Workload:
    return name_or_wl if isinstance(name_or_wl, Workload) else WORKLOADS[name_or_wl]


def custom_workload(name, hidden, experts, top_k, shared, inter, tokens, **kw) -> Workload:
    """A workload outside the fixed table (edge cases, sweeps)."""
    return Workload(name, hidden, experts, top_k, shared, inter, tokens, **kw)


def _wl_id(wl: Workload) -> int:
    if wl.name in _WORKLOAD_IDS and WORKLOADS[wl.name] == wl:
        return _WORKLOAD_IDS[wl.name]
    # custom workloads: fold the name and every field into an id
    h = 0
    # fields added later fold in only when set, so earlier workloads keep their ids
    later = {"shared_fp8", "chained"}
    fields = tuple(getattr(wl, f.name) for f in dataclasses.fields(wl)
                   if f.name not in later or getattr(wl, f.name) != f.default)
    for ch in repr(fields).encode():
        h = (h * 1099511628211 + ch) & _MASK64
    return h | (1 << 40)


# ---------------------------------------------------------------------------
# SplitMix64 (counter-based): word i of stream `key` is mix(key + (i+1)*gamma)
# ---------------------------------------------------------------------------

_MASK64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB


def splitmix64_py(key: int, i: int) -> int:
    """Word ``i`` (0-based) of the SplitMix64 stream seeded with ``key`` (pure Python)."""
    z = (key + (i + 1) * _GAMMA) & _MASK64
    z = ((z ^ (z >> 30)) * _M1) & _MASK64
    z = ((z ^ (z >> 27)) * _M2) & _MASK64
    return z ^ (z >> 31)


def derive_key(*parts: int) -> int:
    """Fold integers into one 64-bit stream key (SplitMix64 finaliser chain)."""
    k = SEED
    for p in parts:
        k = splitmix64_py(k ^ (int(p) & _MASK64), 0)
    return k


def _signed(v: int) -> int:
    return v - (1 << 64) if v >= (1 << 63) else v


def _srl(z: torch.Tensor, s: int) -> torch.Tensor:
    # logical right shift of an int64 tensor (torch's >> is arithmetic)
    return (z >> s) & ((1 << (64 - s)) - 1)


def splitmix64_words(key: int, start: int, count: int, device="cpu") -> torch.Tensor:
    """Words [start, start+count) of the stream, as an int64 tensor (two's complement)."""
    i = torch.arange(start + 1, start + count + 1, dtype=torch.int64, device=device)
    z = i * _signed(_GAMMA) + _signed(key)
    z = (z ^ _srl(z, 30)) * _signed(_M1)
    z = (z ^ _srl(z, 27)) * _signed(_M2)
    return z ^ _srl(z, 31)


_CHUNK_WORDS = 1 << 24


def fill_code_bytes(out: torch.Tensor, key: int, start_byte: int = 0) -> torch.Tensor:
    """Fill a flat uint8 tensor with stream bytes [start_byte, start_byte + numel).

    Byte ``8*i + j`` is byte ``j`` (little-endian) of word ``i``.
    """
    flat = out.view(-1)
    n = flat.numel()
    assert start_byte % 8 == 0 and n % 8 == 0, "code byte ranges are whole words"
    w0 = start_byte // 8
    for c in range(0, n // 8, _CHUNK_WORDS):
        cnt = min(_CHUNK_WORDS, n // 8 - c)
        w = splitmix64_words(key, w0 + c, cnt, flat.device)
        flat[c * 8:(c + cnt) * 8].copy_(w.view(torch.uint8))
    return out


def fill_scale_bytes(out: torch.Tensor, key: int, lo: int, hi: int, start: int = 0) -> torch.Tensor:
    """Fill a flat uint8 tensor with scale bytes uniform on {lo..hi}; byte i uses word i."""
    flat = out.view(-1)
    n = flat.numel()
    span = hi - lo + 1
    for c in range(0, n, _CHUNK_WORDS):
        cnt = min(_CHUNK_WORDS, n - c)
        w = splitmix64_words(key, start + c, cnt, flat.device)
        v = lo + ((_srl(w, 32) * span) >> 32)
        flat[c:c + cnt].copy_(v.to(torch.uint8))
    return out


# ---------------------------------------------------------------------------
# Expert weights: codes [G][N][K/2], scales [G][N][K/32]; gate/up N=I, K=H; down N=H, K=I
# ---------------------------------------------------------------------------


def matrix_dims(wl: Workload, mat: str):
    """(N, K) of one expert matrix: rows are outputs, K is the reduction axis."""
    if mat in ("gate", "up"):
        return wl.inter, wl.hidden
    if mat == "down":
        return wl.hidden, wl.inter
    raise ValueError(mat)


def _keys(wl: Workload, layer: int, mat: str):
    wid = _wl_id(wl)
    return (derive_key(wid, layer, TENSOR_IDS[mat + "_codes"]),
            derive_key(wid, layer, TENSOR_IDS[mat + "_scales"]))


def expert_matrix(wl, layer: int, mat: str, group: int, device="cpu"):
    """Codes [N][K/2] and scales [N][K/32] (uint8 tensors) of one matrix of one group.

    ``group`` is an expert index in [0, E) or ``E`` for the shared expert.
    """
    wl = workload(wl)
    n, k = matrix_dims(wl, mat)
    kc, ks = _keys(wl, layer, mat)
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device=device)
    scales = torch.empty((n, k // 32), dtype=torch.uint8, device=device)
    fill_code_bytes(codes, kc, start_byte=group * n * (k // 2))
    fill_scale_bytes(scales, ks, wl.scale_lo, wl.scale_hi, start=group * n * (k // 32))
    return codes, scales


def layer_weights(wl, layer: int, device="cpu"):
    """All FP4 expert matrices of one layer: dict mat -> (codes [G][N][K/2], scales [G][N][K/32]),
    G = ``wl.fp4_groups`` (the shared expert is left out when it is stored in FP8)."""
    wl = workload(wl)
    out = {}
    for mat in MATRICES:
        n, k = matrix_dims(wl, mat)
        kc, ks = _keys(wl, layer, mat)
        codes = torch.empty((wl.fp4_groups, n, k // 2), dtype=torch.uint8, device=device)
        scales = torch.empty((wl.fp4_groups, n, k // 32), dtype=torch.uint8, device=device)
        fill_code_bytes(codes, kc)
        fill_scale_bytes(scales, ks, wl.scale_lo, wl.scale_hi)
        out[mat] = (codes, scales)
    return out


def shared_fp8_matrix(wl, layer: int, mat: str, device="cpu"):
    """The FP8 shared expert's matrix ``mat``: codes [N][K] (uint8 E4M3 bytes, never a NaN
    pattern) and float32 block scales [ceil(N/128)][ceil(K/128)]."""
    wl = workload(wl)
    n, k = matrix_dims(wl, mat)
    wid = _wl_id(wl)
    codes = torch.empty((n, k), dtype=torch.uint8, device=device)
    fill_code_bytes(codes, derive_key(wid, layer, TENSOR_IDS[mat + "_fp8_codes"]))
    nan = (codes & 0x7F) == 0x7F
    codes[nan] = codes[nan] - 1
    nb, kb = -(-n // 128), -(-k // 128)
    w = splitmix64_words(derive_key(wid, layer, TENSOR_IDS[mat + "_fp8_scales"]), 0, nb * kb, device)
    u = _srl(w, 40).to(torch.float32) * 2.0 ** -24          # exact: 24-bit integers
    scales = ((0.5 + u) * 2.0 ** -7).reshape(nb, kb).contiguous()
    return codes, scales


def shared_fp8_weights(wl, layer: int, device="cpu"):
    """dict mat -> (codes [N][K], scales) of the FP8 shared expert (see ``shared_fp8_matrix``)."""
    return {mat: shared_fp8_matrix(wl, layer, mat, device) for mat in MATRICES}


class LazyExperts:
    """Sequence-like access to one layer's expert weights, regenerated per group on the host.

    ``experts[g]`` returns ``dict(gate=(codes, scales), up=..., down=...)`` as numpy arrays.
    A small cache keeps recently used groups.
    """

    def __init__(self, wl, layer: int, cache: int = 8):
        self.wl = workload(wl)
        self.layer = layer
        self._cache = {}
        self._order = []
        self._cap = cache

    def __len__(self):
        return self.wl.groups

    def __getitem__(self, g: int):
        """FP4 groups as (codes, scales) pairs; with ``shared_fp8`` group E is instead
        dict mat -> ("fp8", codes [N][K], scales [N/128][K/128]) for the caller to wrap."""
        if g < 0 or g >= self.wl.groups:
            raise IndexError(g)
        if g in self._cache:
            return self._cache[g]
        d = {}
        for mat in MATRICES:
            if g >= self.wl.fp4_groups:
                c, s = shared_fp8_matrix(self.wl, self.layer, mat)
                d[mat] = ("fp8", c.numpy(), s.numpy())
                continue
            c, s = expert_matrix(self.wl, self.layer, mat, g)
            d[mat] = (c.numpy(), s.numpy())
        self._cache[g] = d
        self._order.append(g)
        if len(self._order) > self._cap:
            self._cache.pop(self._order.pop(0), None)
        return d


# ---------------------------------------------------------------------------
# Activations, router weights, bias (host, numpy PCG64)
# ---------------------------------------------------------------------------


def _rng(*parts: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(derive_key(*parts)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the uint16 bit patterns."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    if not np.isfinite(a).all():
        raise ValueError("only finite activations are drawn")
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def tokens(wl, layer: int = 0, step: int = 0, attempt: int = 0, count: Optional[int] = None) -> np.ndarray:
    """``count`` (default T) token rows of N(0,1) activations as bf16 bit patterns [count][H]."""
    wl = workload(wl)
    n = wl.tokens if count is None else count
    g = _rng(_wl_id(wl), layer, TENSOR_IDS["x"], step, attempt)
    return f32_to_bf16_bits(g.standard_normal((n, wl.hidden), dtype=np.float32))


def router_weights(wl, layer: int = 0) -> np.ndarray:
    """Router weights [E][H], float32 N(0, 0.02^2)."""
    wl = workload(wl)
    g = _rng(_wl_id(wl), layer, TENSOR_IDS["w_router"])
    return (0.02 * g.standard_normal((wl.experts, wl.hidden), dtype=np.float64)).astype(np.float32)


def router_bias(wl) -> Optional[np.ndarray]:
    """Zipf popularity prior b_e = -s*ln(e+1) (float32 [E]) or None."""
    wl = workload(wl)
    if wl.zipf is None:
        return None
    return (-wl.zipf * np.log(np.arange(1, wl.experts + 1, dtype=np.float64))).astype(np.float32)


def residual_input(wl, step: int = 0, count: Optional[int] = None) -> np.ndarray:
    """Residual-stream input h_0 of a chained workload: ``count`` (default T) rows of N(0, 1), float32 [count][H]."""
    wl = workload(wl)
    n = wl.tokens if count is None else count
    g = _rng(_wl_id(wl), 0, TENSOR_IDS["h_in"], step)
    return g.standard_normal((n, wl.hidden), dtype=np.float32)


def norm_weight(wl, layer: int) -> np.ndarray:
    """RMSNorm weight of one layer's input: 1 + 0.1 * N(0, 1), float32 [H]."""
    wl = workload(wl)
    g = _rng(_wl_id(wl), layer, TENSOR_IDS["norm_weight"])
    return (1.0 + 0.1 * g.standard_normal(wl.hidden, dtype=np.float64)).astype(np.float32)
