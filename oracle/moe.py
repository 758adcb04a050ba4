"""The routed FP4-expert MoE layer written out plainly in float64 (oracle; test infrastructure only).

What the layer computes, for tokens x[t] (bf16) of width H:

1. Router scores  l[t,e] = sum_h x[t,h] * W_r[e,h] + b[e].
   ("feat(v4/cuda): the CUDA tier wired into the DeepSeek V4 engine", PR #1055,
   "What it is", prefill MoE: routing runs on the device.)
2. The k experts with the largest scores, in descending order (ties -> lower
   expert index), weighted by a softmax taken over those k scores only
   (softmax over all E then renormalised over the k is the same number).
   k = 6 for V4 Flash ("Add DeepSeek V4 Flash CPU inference with NVMe expert
   streaming", PR #165, the aarch64 test comment's coverage note).
3. Rows grouped by expert: counts, exclusive offsets, and a permutation of the
   T*k (token, slot) pairs with ascending token inside each expert (PR #1055,
   "What it is": expert-grouped GEMM rows).
4. Each expert is a SwiGLU FFN on FP4 weights: h = silu(x Wg^T) * (x Wu^T),
   y_e = h Wd^T, gate/up [I][H] and down [H][I] (PR #165, anrasi's kernel bench
   at the V4 Flash expert shapes 2048x4096 and 4096x2048).
5. One shared expert runs on every token with weight 1 (PR #1055, "What it
   is": decode fuses routed and shared experts in one MoE stage).
6. y[t] = y_shared[t] + r * sum_j w[t,j] * y_{idx[t,j]}[t].

Readings where the pages are silent: softmax (not sigmoid) scoring, the
bias added before both selection and weighting, a routed scale r that
multiplies the routed sum only (default 1.0; the shared expert keeps weight 1),
plain SwiGLU without clamping, silu(z) = z / (1 + exp(-z)).

Precision: everything is float64, except that the top-k *decision* is taken on
the scores rounded to float32 -- the precision the GPU kernel decides in -- so
both sides order the same numbers.  The weights are computed in float64 from
those float32 scores.
"""
from __future__ import annotations

import numpy as np

from .fp4 import dequant
from .fp8 import Fp8Matrix, dequant_fp8_block


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) to float64: the float32 with those 16 high bits."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def router_logits(x_bits: np.ndarray, w_router: np.ndarray, bias=None) -> np.ndarray:
    """Scores l[t,e] = x[t] . W_r[e] (+ b[e]) in float64, [T][E]."""
    x = bf16_bits_to_f64(x_bits)
    w = np.asarray(w_router, dtype=np.float64)
    l = x @ w.T
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float64)[None, :]
    return l


def select_experts(logits: np.ndarray, k: int):
    """Top-k per token and the renormalised softmax weights.

    Returns (idx int32 [T][k], w float64 [T][k], l32 float32 [T][E]).
    Order: score descending, ties to the lower expert index, decided on the
    float32-rounded scores.  w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0).
    """
    l32 = np.asarray(logits, dtype=np.float64).astype(np.float32)
    t, e = l32.shape
    if not 1 <= k <= e:
        raise ValueError(f"top_k={k} with {e} experts")
    expert_ids = np.broadcast_to(np.arange(e), (t, e))
    neg = -l32.astype(np.float64)
    order = np.lexsort((expert_ids, neg), axis=-1)      # primary: -score, secondary: index
    idx = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(l32, idx, axis=1).astype(np.float64)
    p = np.exp(sel - sel[:, :1])
    w = p / p.sum(axis=1, keepdims=True)
    return idx, w, l32


def group_rows(idx: np.ndarray, n_experts: int):
    """counts [E], offsets [E+1] (exclusive scan), perm [T*k] with ascending token per expert.

    perm[r] = t*k + j names the (token, slot) pair placed at grouped row r.
    """
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=n_experts).astype(np.int32)
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    return counts, offsets, perm


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z)) in float64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def dequant_matrix(w) -> np.ndarray:
    """An expert matrix in either stored format, as float64: an FP4 (codes, scales) pair (e2m1 +
    e8m0 per 32), or FP8 (e4m3 + float32 per 128 x 128 block; the V4 dense format of
    "Add DeepSeek V4 Flash CPU inference with NVMe expert streaming", PR #165, the question on
    V4 sizes) given as an Fp8Matrix or as the tagged triple ("fp8", codes, scales)."""
    if isinstance(w, Fp8Matrix):
        return dequant_fp8_block(w.codes, w.scales)
    if len(w) == 3 and isinstance(w[0], str):
        if w[0] != "fp8":
            raise ValueError(f"unknown matrix format {w[0]!r}")
        return dequant_fp8_block(w[1], w[2])
    return dequant(*w)


def expert_ffn(xrows: np.ndarray, weights) -> np.ndarray:
    """SwiGLU expert on float64 rows [n][H]: silu(x Wg^T) * (x Wu^T), then times Wd^T -> [n][H]."""
    wg = dequant_matrix(weights["gate"])       # [I][H]
    wu = dequant_matrix(weights["up"])         # [I][H]
    wd = dequant_matrix(weights["down"])       # [H][I]
    g = xrows @ wg.T
    u = xrows @ wu.T
    h = silu(g) * u
    return h @ wd.T


def moe_forward(x_bits, w_router, bias, experts, top_k: int, n_shared: int, routed_scale: float = 1.0):
    """The whole layer.  ``experts[g]`` -> dict(gate=(codes, scales), up=..., down=...);
    groups 0..E-1 are routed experts, group E the shared expert when ``n_shared`` is 1.
    ``routed_scale`` multiplies the weighted sum of the routed experts' outputs.

    Returns a dict with y (float64 [T][H]), logits (float64), l32, idx, w,
    counts, offsets, perm.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    t_count = x_bits.shape[0]
    n_exp = np.asarray(w_router).shape[0]
    logits = router_logits(x_bits, w_router, bias)
    idx, w, l32 = select_experts(logits, top_k)
    counts, offsets, perm = group_rows(idx, n_exp)
    x = bf16_bits_to_f64(x_bits)
    y = np.zeros((t_count, x.shape[1]), dtype=np.float64)
    for e in range(n_exp):                      # expert-major: each expert decoded once
        rows = perm[offsets[e]:offsets[e + 1]]
        if rows.size == 0:
            continue
        tok = rows // top_k
        slot = rows % top_k
        ye = expert_ffn(x[tok], experts[e])
        y[tok] += w[tok, slot][:, None] * ye     # a token meets an expert at most once
    y *= routed_scale
    if n_shared:
        y += expert_ffn(x, experts[n_exp])
    return dict(y=y, logits=logits, l32=l32, idx=idx, w=w, counts=counts,
                offsets=offsets, perm=perm)


def screen_near_ties(x_bits, w_router, bias, top_k: int, margin: float = 1e-4) -> np.ndarray:
    """True for tokens whose top min(k+1, E) float64 scores have an adjacent gap below ``margin``.

    Such tokens have a top-k set or order that rounding could flip; the
    generators redraw them so that expert choices are unique on both sides.
    """
    l = router_logits(x_bits, w_router, bias)
    m = min(top_k + 1, l.shape[1])
    top = -np.sort(-l, axis=1)[:, :m]
    if m < 2:
        return np.zeros(l.shape[0], dtype=bool)
    return (top[:, :-1] - top[:, 1:] < margin).any(axis=1)
