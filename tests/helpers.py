"""Shared test helpers: golden-file readers, screened input batches, hand-built expert weights."""
from __future__ import annotations

import os

import numpy as np

import moe_synth as synth
import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def screened_tokens(wl, w_router, bias, layer=0, step=0, margin=1e-4, max_attempts=64):
    """Token batch (bf16 bits) with every near-tie token redrawn from the next attempt's stream."""
    wl = synth.workload(wl)
    x = synth.tokens(wl, layer=layer, step=step, attempt=0)
    bad = oracle.screen_near_ties(x, w_router, bias, wl.top_k, margin)
    attempt = 1
    while bad.any():
        if attempt > max_attempts:
            raise RuntimeError("could not screen near-ties")
        repl = synth.tokens(wl, layer=layer, step=step, attempt=attempt, count=int(bad.sum()))
        x = x.copy()
        x[bad] = repl
        bad = oracle.screen_near_ties(x, w_router, bias, wl.top_k, margin)
        attempt += 1
    return x


def _put_code(codes_row, k, code):
    """Set nibble k of a row of code bytes (low nibble = even element)."""
    b = codes_row[k // 2]
    codes_row[k // 2] = (b & 0xF0) | code if k % 2 == 0 else (b & 0x0F) | (code << 4)


def identity_experts(hidden, inter, n_experts, n_shared, sigma):
    """Hand-built groups whose FFN has a closed form.

    gate = selector with value 1 (gate[i][i] = 1), up = selector with value 2
    (up[i][i] = 2), down[h][h] = 2^-sigma[g] for h < I, zero elsewhere.  Then for
    h < I: f_g(x)_h = 2^-sigma[g] * silu(x_h) * 2 x_h, and f_g(x)_h = 0 for h >= I.
    """
    assert inter <= hidden
    groups = []
    for g in range(n_experts + n_shared):
        gate_c = np.zeros((inter, hidden // 2), np.uint8)
        up_c = np.zeros((inter, hidden // 2), np.uint8)
        for i in range(inter):
            _put_code(gate_c[i], i, 2)   # E2M1 code 2 = 1.0
            _put_code(up_c[i], i, 4)     # E2M1 code 4 = 2.0
        gate_s = np.full((inter, hidden // 32), 127, np.uint8)
        up_s = np.full((inter, hidden // 32), 127, np.uint8)
        down_c = np.zeros((hidden, inter // 2), np.uint8)
        down_s = np.full((hidden, inter // 32), 127, np.uint8)
        for h in range(inter):
            _put_code(down_c[h], h, 2)
            down_s[h, h // 32] = 127 - sigma[g]
        groups.append(dict(gate=(gate_c, gate_s), up=(up_c, up_s), down=(down_c, down_s)))
    return groups


def random_experts(rng, hidden, inter, groups, scale_lo=123, scale_hi=127):
    out = []
    for _ in range(groups):
        d = {}
        for mat, (n, k) in (("gate", (inter, hidden)), ("up", (inter, hidden)), ("down", (hidden, inter))):
            d[mat] = (rng.integers(0, 256, (n, k // 2), dtype=np.uint8),
                      rng.integers(scale_lo, scale_hi + 1, (n, k // 32), dtype=np.uint8))
        out.append(d)
    return out
