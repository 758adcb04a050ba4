"""Planted mistakes in the oracle must each make at least one pin fail.

Each mutant below swaps one piece of the float64 oracle for a plausibly wrong
version (a dropped term, a wrong sign, a swapped index or operand, an off-by-one
in the format) and runs every pin of ``test_oracle_pins.py`` against it.  A mutant
that no pin notices would mean the pins do not constrain that part of the oracle.
Everything here runs on the CPU and touches nothing but the oracle.
"""
import contextlib
import inspect

import numpy as np
import pytest

import oracle
import oracle.fp4 as ofp4
import oracle.chain as ochain
import oracle.fp8 as ofp8
import oracle.moe as omoe
import test_oracle_pins as pins

ORIG = {
    "dequant": ofp4.dequant,
    "e8m0_value": ofp4.e8m0_value,
    "select_experts": omoe.select_experts,
    "group_rows": omoe.group_rows,
    "router_logits": omoe.router_logits,
    "expert_ffn": omoe.expert_ffn,
    "moe_forward": omoe.moe_forward,
    "silu": omoe.silu,
    "bf16_bits_to_f64": omoe.bf16_bits_to_f64,
    "dequant_fp8_block": ofp8.dequant_fp8_block,
    "rms_norm": ochain.rms_norm,
    "f64_to_bf16_bits": ochain.f64_to_bf16_bits,
    "chain_forward": ochain.chain_forward,
}


@contextlib.contextmanager
def patched(name, value, modules=(ofp4, ofp8, omoe, ochain, oracle)):
    """Replace `name` in every oracle namespace that holds it (package re-exports included)."""
    saved = [(m, getattr(m, name)) for m in modules if hasattr(m, name)]
    try:
        for m, _ in saved:
            setattr(m, name, value)
        yield
    finally:
        for m, v in saved:
            setattr(m, name, v)


def _dequant_nibbles_swapped(codes, scales):
    codes = np.asarray(codes, dtype=np.uint8)
    swapped = ((codes & 0x0F) << 4) | (codes >> 4)
    return ORIG["dequant"](swapped.astype(np.uint8), scales)


def _dequant_scale_block_16(codes, scales):
    v = ORIG["dequant"](codes, np.zeros_like(np.asarray(scales)) + 127)  # values, unscaled
    s = ofp4.E8M0_VALUES[np.asarray(scales, dtype=np.uint8)]
    k = v.shape[1]
    block = (np.arange(k) // 16) % s.shape[1]   # scale j read as covering 16 values, wrapping
    with np.errstate(invalid="ignore"):
        return v * s[:, block]


def _select_full_softmax(logits, k):
    idx, _, l32 = ORIG["select_experts"](logits, k)
    l = l32.astype(np.float64)
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return idx, np.take_along_axis(p, idx.astype(np.int64), axis=1), l32


def _select_ties_high(logits, k):
    l32 = np.asarray(logits, dtype=np.float64).astype(np.float32)
    t, e = l32.shape
    ids = np.broadcast_to(np.arange(e)[::-1], (t, e))
    order = np.lexsort((ids, -l32.astype(np.float64)), axis=-1)
    idx = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(l32, idx, axis=1).astype(np.float64)
    p = np.exp(sel - sel[:, :1])
    return idx, p / p.sum(axis=1, keepdims=True), l32


def _select_unit_weights(logits, k):
    idx, w, l32 = ORIG["select_experts"](logits, k)
    return idx, np.ones_like(w), l32


def _group_unstable(idx, n_experts):
    counts, offsets, perm = ORIG["group_rows"](idx, n_experts)
    perm = perm.copy()
    for e in range(n_experts):
        perm[offsets[e]:offsets[e + 1]] = perm[offsets[e]:offsets[e + 1]][::-1]
    return counts, offsets, perm


def _router_no_bias(x_bits, w_router, bias=None):
    return ORIG["router_logits"](x_bits, w_router, None)


def _ffn_gate_up_swapped(xrows, weights):
    return ORIG["expert_ffn"](xrows, dict(gate=weights["up"], up=weights["gate"], down=weights["down"]))


def _forward_no_shared(x_bits, w_router, bias, experts, top_k, n_shared, routed_scale=1.0):
    return ORIG["moe_forward"](x_bits, w_router, bias, experts, top_k, 0, routed_scale)


def _forward_scale_ignored(x_bits, w_router, bias, experts, top_k, n_shared, routed_scale=1.0):
    return ORIG["moe_forward"](x_bits, w_router, bias, experts, top_k, n_shared)


def _forward_scale_on_shared_too(x_bits, w_router, bias, experts, top_k, n_shared, routed_scale=1.0):
    out = ORIG["moe_forward"](x_bits, w_router, bias, experts, top_k, n_shared)
    out["y"] = out["y"] * routed_scale
    return out


def _bf16_shift15(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 15
    return b.view(np.float32).astype(np.float64)


def _fp8_blocks_of_64(codes, scales):
    codes = np.asarray(codes, np.uint8)
    s = np.asarray(scales, np.float32).astype(np.float64)
    r = np.minimum(np.arange(codes.shape[0]) // 64, s.shape[0] - 1)
    c = np.minimum(np.arange(codes.shape[1]) // 64, s.shape[1] - 1)
    return ofp8.E4M3_VALUES[codes] * s[r[:, None], c[None, :]]


def _fp8_scales_transposed(codes, scales):
    s = np.asarray(scales, np.float32)
    return ORIG["dequant_fp8_block"](codes, s.T if s.shape[0] == s.shape[1] else s[::-1, ::-1])


def _rms_sum_not_mean(h, gamma, eps=1e-6):
    h = np.asarray(h, np.float64)
    return h / np.sqrt(np.sum(h * h, axis=-1, keepdims=True) + eps) * np.asarray(gamma, np.float64)


def _rms_eps_outside(h, gamma, eps=1e-6):
    h = np.asarray(h, np.float64)
    return h / (np.sqrt(np.mean(h * h, axis=-1, keepdims=True)) + eps) * np.asarray(gamma, np.float64)


def _rms_no_gamma(h, gamma, eps=1e-6):
    return ORIG["rms_norm"](h, np.ones(np.asarray(h).shape[-1]), eps)


def _bf16_truncate(v):
    b = np.asarray(v, np.float64).astype(np.float32).view(np.uint32) >> np.uint32(16)
    return b.astype(np.uint16)


def _chain_no_residual(h_in, gammas, routers, biases, experts, top_k, n_shared, eps=1e-6, routed_scale=1.0):
    h = np.asarray(h_in, np.float64)
    xs, ys, routes = [], [], []
    for l in range(len(routers)):
        x = ochain.norm_input(h, gammas[l], eps)
        out = omoe.moe_forward(x, routers[l], biases[l], experts[l], top_k, n_shared, routed_scale)
        h = out["y"]                                   # the residual dropped
        xs.append(x), ys.append(out["y"]), routes.append(out)
    return dict(x=xs, y=ys, route=routes, h=h)


def _chain_gamma_shifted(h_in, gammas, routers, biases, experts, top_k, n_shared, eps=1e-6, routed_scale=1.0):
    shifted = list(gammas[1:]) + list(gammas[:1])
    return ORIG["chain_forward"](h_in, shifted, routers, biases, experts, top_k, n_shared, eps, routed_scale)


def _chain_norm_skipped(h_in, gammas, routers, biases, experts, top_k, n_shared, eps=1e-6, routed_scale=1.0):
    with patched("norm_input", lambda h, g, e=1e-6: ochain.f64_to_bf16_bits(np.asarray(h) * np.asarray(g))):
        return ORIG["chain_forward"](h_in, gammas, routers, biases, experts, top_k, n_shared, eps, routed_scale)


MUTANTS = {
    "nibble order swapped": [("dequant", _dequant_nibbles_swapped)],
    "scale blocks of 16": [("dequant", _dequant_scale_block_16)],
    "e8m0 off by one": [("E8M0_VALUES", ofp4.E8M0_VALUES * 2.0),
                        ("e8m0_value", lambda s: 2.0 * ORIG["e8m0_value"](s))],
    "e2m1 mantissa weight": [("E2M1_VALUES", np.where(np.arange(16) & 1,
                                                      ofp4.E2M1_VALUES * 1.125, ofp4.E2M1_VALUES))],
    "silu sign": [("silu", lambda z: np.asarray(z, np.float64) / (1.0 + np.exp(np.asarray(z, np.float64))))],
    "softmax over all experts": [("select_experts", _select_full_softmax)],
    "ties to higher index": [("select_experts", _select_ties_high)],
    "routing weights dropped": [("select_experts", _select_unit_weights)],
    "grouping not stable": [("group_rows", _group_unstable)],
    "router bias ignored": [("router_logits", _router_no_bias)],
    "gate and up swapped": [("expert_ffn", _ffn_gate_up_swapped)],
    "shared expert dropped": [("moe_forward", _forward_no_shared)],
    "routed scale ignored": [("moe_forward", _forward_scale_ignored)],
    "routed scale on the shared expert too": [("moe_forward", _forward_scale_on_shared_too)],
    "bf16 decode shifted": [("bf16_bits_to_f64", _bf16_shift15)],
    "e4m3 exponent bias 8": [("E4M3_VALUES", ofp8.E4M3_VALUES / 2)],
    "e4m3 subnormals flushed": [("E4M3_VALUES", np.where((np.arange(256) & 0x78) == 0, 0.0, ofp8.E4M3_VALUES))],
    "fp8 scale blocks of 64": [("dequant_fp8_block", _fp8_blocks_of_64)],
    "fp8 scale grid transposed": [("dequant_fp8_block", _fp8_scales_transposed)],
    "rms norm over the sum, not the mean": [("rms_norm", _rms_sum_not_mean)],
    "rms norm eps outside the root": [("rms_norm", _rms_eps_outside)],
    "rms norm gamma dropped": [("rms_norm", _rms_no_gamma)],
    "bf16 rounding truncates": [("f64_to_bf16_bits", _bf16_truncate)],
    "chain residual dropped": [("chain_forward", _chain_no_residual)],
    "chain gamma of the next layer": [("chain_forward", _chain_gamma_shifted)],
    "chain norm skipped": [("chain_forward", _chain_norm_skipped)],
}


def _pin_functions():
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if name.startswith("test_") and not inspect.signature(fn).parameters:
            out.append((name, fn))
    return out


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant):
    caught = []
    with contextlib.ExitStack() as stack:
        for name, value in MUTANTS[mutant]:
            stack.enter_context(patched(name, value))
        for name, fn in _pin_functions():
            try:
                fn()
            except Exception:  # an assertion, or the mutant breaking a shape
                caught.append(name)
    assert caught, f"no pin notices the mutant '{mutant}'"


def test_unmutated_oracle_passes_every_pin():
    for name, fn in _pin_functions():
        fn()
