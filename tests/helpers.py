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


def random_fp8_shared(rng, hidden, inter, code_hi=0x7E, scale_exp=-7):
    """A random FP8 shared expert, dict mat -> (codes [N][K] uint8, float32 scales
    [ceil(N/128)][ceil(K/128)]): codes uniform on the finite E4M3 patterns with magnitude code
    at most ``code_hi`` (0x7E = 448), scales (0.5 + U) * 2^scale_exp."""
    out = {}
    for mat, (n, k) in (("gate", (inter, hidden)), ("up", (inter, hidden)), ("down", (hidden, inter))):
        mag = rng.integers(0, code_hi + 1, (n, k), dtype=np.uint8)
        sign = rng.integers(0, 2, (n, k), dtype=np.uint8) << 7
        sc = ((0.5 + rng.random((-(-n // 128), -(-k // 128)))) * 2.0 ** scale_exp).astype(np.float32)
        out[mat] = (mag | sign, sc)
    return out


def identity_fp8_shared(hidden, inter, down_scale=0.75):
    """FP8 shared expert with a closed form: gate = selector of 1.0 (E4M3 0x38), up = selector of
    2.0 (0x40), down = selector of 1.0 with every down block scale ``down_scale``; it adds
    down_scale * silu(x_i) * 2 x_i for i < I."""
    g = np.zeros((inter, hidden), np.uint8)
    u = np.zeros((inter, hidden), np.uint8)
    d = np.zeros((hidden, inter), np.uint8)
    for i in range(inter):
        g[i, i], u[i, i], d[i, i] = 0x38, 0x40, 0x38
    one = lambda n, k: np.ones((-(-n // 128), -(-k // 128)), np.float32)
    return dict(gate=(g, one(inter, hidden)), up=(u, one(inter, hidden)),
                down=(d, np.full((-(-hidden // 128), -(-inter // 128)), down_scale, np.float32)))


def as_oracle_fp8(shared):
    """dict mat -> (codes, scales) as the oracle's tagged FP8 triples."""
    return {mat: ("fp8", np.asarray(c), np.asarray(s)) for mat, (c, s) in shared.items()}
