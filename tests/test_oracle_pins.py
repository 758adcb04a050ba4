"""Pins of the CPU oracle to facts outside itself: golden values, closed forms, brute force, invariants."""
import itertools
import math

import numpy as np
import pytest
import torch

import moe_synth as synth
import oracle
from oracle.fp4 import E8M0_VALUES
from oracle.moe import bf16_bits_to_f64
from helpers import golden_lines, identity_experts, random_experts


def _float(tok):
    return float(tok)


# --------------------------------------------------------------------- codec


def test_e2m1_codebook_matches_golden():
    rows = [line.split() for line in golden_lines("e2m1_codebook.txt")]
    assert len(rows) == 16
    for code, val in rows:
        got = oracle.e2m1_value(int(code))
        want = float(val)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)
    assert np.array_equal(oracle.E2M1_VALUES, [float(v) for _, v in rows])


def test_e2m1_table_facts_from_the_pages():
    # 16 float32 entries fill 64 bytes; doubled values are integers.
    assert oracle.E2M1_VALUES.astype(np.float32).nbytes == 64
    doubled = 2 * oracle.E2M1_VALUES
    assert np.array_equal(doubled, np.round(doubled))
    assert set(np.abs(doubled).astype(int)) == {0, 1, 2, 3, 4, 6, 8, 12}
    # codes 8..15 are the negatives of codes 0..7 (code 8 is -0)
    assert np.array_equal(oracle.E2M1_VALUES[8:], -oracle.E2M1_VALUES[:8])
    assert math.copysign(1, oracle.E2M1_VALUES[8]) == -1


def test_e8m0_closed_form_and_edges():
    for s in range(1, 255):
        assert oracle.e8m0_value(s) == math.ldexp(1.0, s - 127)
    assert oracle.e8m0_value(0) == 0.0 and math.copysign(1, oracle.e8m0_value(0)) == 1
    assert oracle.e8m0_value(255) == math.inf
    assert oracle.e8m0_value(127) == 1.0
    assert np.array_equal(E8M0_VALUES[123:128], [1 / 16, 1 / 8, 1 / 4, 1 / 2, 1])


def _read_blocks():
    lines = list(golden_lines("fp4_block_example.txt"))
    out = []
    for i in range(0, len(lines), 3):
        codes = bytes.fromhex("".join(lines[i].split()[1:]))
        scale = int(lines[i + 1].split()[1])
        vals = [float(v) for v in lines[i + 2].split()[1:]]
        out.append((np.frombuffer(codes, np.uint8), scale, np.array(vals)))
    return out


def test_dequant_hand_worked_blocks():
    blocks = _read_blocks()
    assert len(blocks) == 4
    for codes, scale, want in blocks:
        got = oracle.dequant(codes[None, :], np.array([[scale]], np.uint8))[0]
        assert got.shape == (32,)
        np.testing.assert_array_equal(got, want)
        finite = np.isfinite(want)
        assert np.array_equal(np.signbit(got[finite]), np.signbit(want[finite]))


def test_nibble_order_low_first():
    got = oracle.dequant(np.array([[0x21] + [0] * 15], np.uint8), np.array([[127]], np.uint8))[0]
    assert got[0] == 0.5 and got[1] == 1.0 and not got[2:].any()


def test_dequant_matches_scalar_loops():
    rng = np.random.default_rng(3)
    n, k = 5, 96
    codes = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = rng.integers(100, 140, (n, k // 32), dtype=np.uint8)
    got = oracle.dequant(codes, scales)
    for r in range(n):
        for c in range(k):
            byte = int(codes[r, c // 2])
            nib = byte & 15 if c % 2 == 0 else byte >> 4
            want = oracle.e2m1_value(nib) * math.ldexp(1.0, int(scales[r, c // 32]) - 127)
            assert got[r, c] == want


# --------------------------------------------------------------------- router


def test_bf16_decode_examples():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F80], np.uint16)
    got = bf16_bits_to_f64(bits)
    assert list(got[:3]) == [1.0, -1.0, 3.140625]
    assert got[3] == 0 and np.signbit(got[4]) and got[5] == np.inf


def test_router_logits_bruteforce_small():
    rng = np.random.default_rng(0)
    t, e, h = 3, 5, 64
    x = synth.f32_to_bf16_bits(rng.standard_normal((t, h)).astype(np.float32))
    w = rng.standard_normal((e, h)).astype(np.float32)
    b = rng.standard_normal(e).astype(np.float32)
    got = oracle.router_logits(x, w, b)
    xf = bf16_bits_to_f64(x)
    for i in range(t):
        for j in range(e):
            acc = math.fsum(float(xf[i, q]) * float(w[j, q]) for q in range(h)) + float(b[j])
            assert abs(got[i, j] - acc) <= 1e-12 * (1 + abs(acc))


def test_router_closed_form_weights():
    # W_r[e] = ln(c_e) * onehot(e): with x = all ones the scores are ln(c_e), so the top-3
    # weights are c_j / sum(c) for the three largest c.
    c = np.array([1.0, 4.0, 2.0, 0.5, 3.0, 0.25])
    e, h = len(c), 32
    w = np.zeros((e, h), np.float32)
    for i in range(e):
        w[i, i] = np.log(c[i])
    x = np.full((1, h), 0x3F80, np.uint16)       # 1.0 in bf16
    idx, wt, _ = oracle.select_experts(oracle.router_logits(x, w), 3)
    assert idx.tolist() == [[1, 4, 2]]
    np.testing.assert_allclose(wt[0], [4 / 9, 3 / 9, 2 / 9], rtol=1e-6)
    assert abs(wt.sum() - 1) < 1e-15


def test_bias_shifts_selection():
    w = np.zeros((4, 32), np.float32)
    x = np.zeros((1, 32), np.uint16)
    b = np.array([0.0, -1.0, 2.0, 1.0], np.float32)
    idx, wt, _ = oracle.select_experts(oracle.router_logits(x, w, b), 2)
    assert idx.tolist() == [[2, 3]]
    np.testing.assert_allclose(wt[0], [math.e / (math.e + 1), 1 / (math.e + 1)], rtol=1e-7)


def test_topk_ties_go_to_lower_index():
    logits = np.array([[1.0, 3.0, 3.0, 0.0, 3.0, -0.0]])
    idx, wt, _ = oracle.select_experts(logits, 4)
    assert idx.tolist() == [[1, 2, 4, 0]]
    logits = np.array([[-0.0, 0.0, -1.0]])
    assert oracle.select_experts(logits, 2)[0].tolist() == [[0, 1]]


def test_top2_bruteforce_over_pairs_tiny_workload():
    wl = synth.WORKLOADS["tiny"]
    wr = synth.router_weights(wl)
    x = synth.tokens(wl)
    logits = oracle.router_logits(x, wr, None)
    idx, _, l32 = oracle.select_experts(logits, 2)
    for t in range(wl.tokens):
        winners = [p for p in itertools.combinations(range(wl.experts), 2)
                   if min(l32[t, list(p)]) > max(np.delete(l32[t], list(p)))]
        assert len(winners) == 1
        a, b = winners[0]
        want = [a, b] if l32[t, a] > l32[t, b] else [b, a]
        assert idx[t].tolist() == want


def test_softmax_is_renormalised_full_softmax():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((7, 16))
    idx, wt, l32 = oracle.select_experts(logits, 5)
    full = np.exp(l32.astype(np.float64))
    full /= full.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(full, idx, axis=1)
    np.testing.assert_allclose(wt, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13)


# --------------------------------------------------------------------- grouping


def test_grouping_hand_worked_example():
    lines = {l.split()[0]: [int(v) for v in l.split()[1:]] for l in golden_lines("grouping_example.txt")}
    idx = np.array(lines["idx"]).reshape(3, 2)
    counts, offsets, perm = oracle.group_rows(idx, 3)
    assert counts.tolist() == lines["counts"]
    assert offsets.tolist() == lines["offsets"]
    assert perm.tolist() == lines["perm"]


def test_grouping_invariants_random():
    rng = np.random.default_rng(7)
    t, e, k = 300, 40, 6
    idx = np.stack([rng.choice(e, k, replace=False) for _ in range(t)])
    counts, offsets, perm = oracle.group_rows(idx, e)
    assert counts.sum() == t * k
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(np.sort(perm), np.arange(t * k))
    for x in range(e):
        rows = perm[offsets[x]:offsets[x + 1]]
        assert np.all(idx.reshape(-1)[rows] == x)
        assert np.all(np.diff(rows // k) > 0)


# --------------------------------------------------------------------- experts and layer


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    l3 = math.log(3.0)
    assert abs(oracle.silu(l3) - 0.75 * l3) < 1e-15
    assert abs(oracle.silu(-l3) + 0.25 * l3) < 1e-15
    z = np.linspace(-30, 30, 61)
    np.testing.assert_allclose(oracle.silu(z) - oracle.silu(-z), z, atol=1e-13)
    assert oracle.silu(-1000.0) == 0.0 and oracle.silu(1000.0) == 1000.0


def _identity_setup(hidden=128, inter=64, experts=6, k=2, tokens=5, seed=0):
    rng = np.random.default_rng(seed)
    sigma = [g + 1 for g in range(experts)] + [0]
    groups = identity_experts(hidden, inter, experts, 1, sigma)
    wr = (0.3 * rng.standard_normal((experts, hidden))).astype(np.float32)
    x = synth.f32_to_bf16_bits(rng.standard_normal((tokens, hidden)).astype(np.float32))
    return groups, wr, x, sigma


def test_identity_experts_closed_form():
    _identity_closed_form(1.0)


def test_routed_scale_closed_form():
    # the routed scale multiplies the routed experts' weighted sum; the shared expert keeps weight 1
    _identity_closed_form(2.5)


def _identity_closed_form(routed_scale):
    hidden, inter, experts, k = 128, 64, 6, 2
    groups, wr, x, sigma = _identity_setup(hidden, inter, experts, k)
    out = oracle.moe_forward(x, wr, None, groups, k, 1, routed_scale=routed_scale)
    xf = bf16_bits_to_f64(x)
    for t in range(x.shape[0]):
        coef = 2.0 ** -sigma[experts]  # shared expert
        for j in range(k):
            coef += routed_scale * out["w"][t, j] * 2.0 ** -sigma[out["idx"][t, j]]
        for h in range(hidden):
            v = xf[t, h]
            want = coef * (v / (1 + math.exp(-v))) * 2 * v if h < inter else 0.0
            assert abs(out["y"][t, h] - want) <= 1e-13 * (1 + abs(want)), (t, h)


def test_topk_equal_to_all_experts_is_dense_mixture():
    rng = np.random.default_rng(5)
    hidden, inter, e = 64, 32, 5
    groups = random_experts(rng, hidden, inter, e + 1)
    wr = (0.05 * rng.standard_normal((e, hidden))).astype(np.float32)
    b = rng.standard_normal(e).astype(np.float32)
    x = synth.f32_to_bf16_bits(rng.standard_normal((4, hidden)).astype(np.float32))
    out = oracle.moe_forward(x, wr, b, groups, e, 1)
    xf = bf16_bits_to_f64(x)
    l32 = (xf @ wr.astype(np.float64).T + b).astype(np.float32).astype(np.float64)
    p = np.exp(l32 - l32.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dense = np.zeros_like(xf)
    for g in range(e + 1):
        wg = oracle.dequant(*groups[g]["gate"])
        wu = oracle.dequant(*groups[g]["up"])
        wd = oracle.dequant(*groups[g]["down"])
        a = np.einsum("th,ih->ti", xf, wg)
        u = np.einsum("th,ih->ti", xf, wu)
        f = np.einsum("ti,hi->th", a / (1 + np.exp(-a)) * u, wd)
        dense += f if g == e else p[:, g:g + 1] * f
    np.testing.assert_allclose(out["y"], dense, rtol=1e-10, atol=1e-9 * np.abs(dense).max())


def test_batch_equals_single_token():
    rng = np.random.default_rng(11)
    hidden, inter, e, k = 64, 32, 8, 3
    groups = random_experts(rng, hidden, inter, e + 1)
    wr = (0.1 * rng.standard_normal((e, hidden))).astype(np.float32)
    x = synth.f32_to_bf16_bits(rng.standard_normal((6, hidden)).astype(np.float32))
    full = oracle.moe_forward(x, wr, None, groups, k, 1)
    for t in range(6):
        one = oracle.moe_forward(x[t:t + 1], wr, None, groups, k, 1)
        assert np.array_equal(one["idx"][0], full["idx"][t])
        np.testing.assert_allclose(one["y"][0], full["y"][t], rtol=1e-12, atol=1e-9)


def test_no_shared_expert_and_zero_scale_blocks():
    rng = np.random.default_rng(2)
    hidden, inter, e, k = 64, 32, 4, 2
    groups = random_experts(rng, hidden, inter, e)
    for g in groups:
        g["down"][1][:] = 0                     # s=0 -> every down weight is +-0
    wr = (0.1 * rng.standard_normal((e, hidden))).astype(np.float32)
    x = synth.f32_to_bf16_bits(rng.standard_normal((3, hidden)).astype(np.float32))
    out = oracle.moe_forward(x, wr, None, groups, k, 0)
    assert not out["y"].any()


# --------------------------------------------------------------------- generator + screen


def test_screen_removes_near_ties():
    from helpers import screened_tokens
    wl = synth.custom_workload("screen", 256, 64, 6, 1, 128, 256)
    wr = synth.router_weights(wl)
    x0 = synth.tokens(wl)
    x = screened_tokens(wl, wr, None, margin=2e-3)      # wide margin: forces redraws
    assert oracle.screen_near_ties(x0, wr, None, 6, 2e-3).any()
    assert not oracle.screen_near_ties(x, wr, None, 6, 2e-3).any()
    l = np.sort(oracle.router_logits(x, wr, None), axis=1)[:, ::-1][:, :7]
    assert (np.diff(-l, axis=1) >= 2e-3).all()


def test_zipf_bias_makes_hot_experts():
    wl = synth.WORKLOADS["prefill_t4096_zipf"]
    b = synth.router_bias(wl)
    assert b[0] == 0 and abs(b[1] + 1.1 * math.log(2)) < 1e-6
    wr = synth.router_weights(wl)
    x = synth.tokens(wl)
    idx, _, _ = oracle.select_experts(oracle.router_logits(x, wr, b), wl.top_k)
    counts = np.bincount(idx.reshape(-1), minlength=wl.experts)
    assert counts.max() > 0.10 * idx.size
    assert (counts == 0).sum() > 10


# ------------------------------------------------------------- FP8 (E4M3, 128 x 128 blocks)
# "Add DeepSeek V4 Flash CPU inference with NVMe expert streaming" (PR #165, the question on V4
# sizes): dense tensors are FP8 E4M3 with 128x128 block scales; the shared expert may be stored so.


def test_e4m3_closed_form_and_edges():
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        v = oracle.e4m3_value(c)
        if e == 15 and m == 7:
            assert math.isnan(v)
            continue
        want = (-1) ** s * (m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
        assert v == want and math.copysign(1, v) == math.copysign(1, want), c
    vals = oracle.E4M3_VALUES
    assert vals[0x38] == 1.0 and vals[0xB8] == -1.0
    assert vals[0x7E] == 448.0 and np.nanmax(vals) == 448.0      # largest finite, no infinity
    assert vals[0x01] == 2.0 ** -9 and vals[0x08] == 2.0 ** -6    # smallest subnormal, smallest normal
    assert np.isnan(vals[[0x7F, 0xFF]]).all() and np.isnan(vals).sum() == 2
    assert math.copysign(1, vals[0x80]) == -1 and vals[0x80] == 0
    np.testing.assert_array_equal(vals[128:], -vals[:128])


def test_e4m3_matches_torch_float8_e4m3fn():
    # an independent decoder: torch's float8_e4m3fn dtype (the same OCP E4M3 "fn" encoding)
    import torch
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = oracle.E4M3_VALUES
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(mine[ok], ref[ok])
    np.testing.assert_array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def test_fp8_block_dequant_hand_worked():
    lines = list(golden_lines("fp8_block_example.txt"))
    scales = np.array([float(v) for v in lines[0].split()[1:]], np.float32).reshape(2, 2)
    codes = np.zeros((130, 256), np.uint8)
    entries = []
    for line in lines[1:]:
        r, c, code, val = line.split("#")[0].split()
        entries.append((int(r), int(c), int(code, 16), float(val)))
        codes[int(r), int(c)] = int(code, 16)
    out = oracle.dequant_fp8_block(codes, scales)
    for r, c, _, val in entries:
        assert out[r, c] == val and math.copysign(1, out[r, c]) == math.copysign(1, val), (r, c, out[r, c], val)
    # every other element is +0 (code 0) whatever its block's scale
    mask = np.ones_like(codes, bool)
    for r, c, _, _ in entries:
        mask[r, c] = False
    assert (out[mask] == 0).all()


def test_fp8_shared_identity_expert_closed_form():
    # FP4 identity routed experts (as above) with an FP8 shared expert: gate = selector of 1.0,
    # up = selector of 2.0, down = selector of 1.0, and down's block scale 0.75 (not a power of
    # two), so the shared expert adds 0.75 * silu(x_i) * 2 x_i for i < I.
    hidden, inter, experts, k = 128, 64, 6, 2
    groups, wr, x, sigma = _identity_setup(hidden, inter, experts, k)
    one, two = 0x38, 0x40
    g = np.zeros((inter, hidden), np.uint8)
    u = np.zeros((inter, hidden), np.uint8)
    d = np.zeros((hidden, inter), np.uint8)
    for i in range(inter):
        g[i, i], u[i, i], d[i, i] = one, two, one
    sg = np.ones((1, 1), np.float32)
    groups[experts] = dict(gate=oracle.Fp8Matrix(g, sg), up=("fp8", u, sg),
                           down=oracle.Fp8Matrix(d, np.full((1, 1), 0.75, np.float32)))
    out = oracle.moe_forward(x, wr, None, groups, k, 1)
    xf = bf16_bits_to_f64(x)
    for t in range(x.shape[0]):
        coef = 0.75
        for j in range(k):
            coef += out["w"][t, j] * 2.0 ** -sigma[out["idx"][t, j]]
        for h in range(hidden):
            v = xf[t, h]
            want = coef * (v / (1 + math.exp(-v))) * 2 * v if h < inter else 0.0
            assert abs(out["y"][t, h] - want) <= 1e-13 * (1 + abs(want)), (t, h)


# ---------------------------------------------------------------- chained decode (oracle/chain.py)
# The inter-layer step is a reading (pre-norm residual with RMSNorm, eps 1e-6): the pages run the
# MoE stage per layer ("feat(v4/cuda): the CUDA tier wired into the DeepSeek V4 engine", PR #1055,
# "What it is") without defining the join.  Pins: torch's own conversions and rms_norm, hand-worked
# values, and closed forms of whole chains.


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(50000) * 3, rng.standard_normal(2000) * 1e-38,
                        rng.standard_normal(2000) * 1e38]).astype(np.float32)
    x = np.concatenate([x, np.float32([0.0, -0.0, np.inf, -np.inf, 3.3e38, -3.39e38])])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.f64_to_bf16_bits(x.astype(np.float64)), want)


def test_bf16_rounding_hand_cases():
    cases = [(1.0, 0x3F80), (1 + 2.0 ** -8, 0x3F80),        # tie -> even (down)
             (1 + 3 * 2.0 ** -8, 0x3F82),                     # tie -> even (up)
             (1 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),            # just past the tie: float64 decides
             (255.5, 0x4380),                                 # tie rounds up into the next binade (256)
             (-2.5, 0xC020), (2.0 ** -133, 0x0001), (2.0 ** -134, 0x0000), (3 * 2.0 ** -134, 0x0002),
             (float("nan"), 0x7FC0), (2.0 ** 128, 0x7F80)]
    for v, bits in cases:
        assert int(oracle.f64_to_bf16_bits(np.float64(v))) == bits, (v, hex(bits))


def test_rms_norm_hand_worked():
    # h = (3, 4): mean of squares 12.5; gamma = (2, 1/2)
    got = oracle.rms_norm(np.array([[3.0, 4.0]]), np.array([2.0, 0.5]), eps=0.0)
    np.testing.assert_allclose(got, [[6 / math.sqrt(12.5), 2 / math.sqrt(12.5)]], rtol=1e-15)
    got = oracle.rms_norm(np.array([[3.0, 4.0]]), np.ones(2), eps=0.5)     # eps inside the root
    np.testing.assert_allclose(got, [[3 / math.sqrt(13.0), 4 / math.sqrt(13.0)]], rtol=1e-15)
    assert (oracle.rms_norm(np.zeros((1, 64)), np.ones(64)) == 0).all()     # eps keeps 0 finite
    c = oracle.rms_norm(np.full((1, 32), -0.25), np.ones(32), eps=oracle.RMS_EPS)
    np.testing.assert_allclose(c, -0.25 / math.sqrt(0.0625 + 1e-6), rtol=1e-15)
    assert oracle.RMS_EPS == 1e-6


def test_rms_norm_matches_torch():
    rng = np.random.default_rng(12)
    h = rng.standard_normal((5, 96)) * 1e3
    g = 1 + 0.1 * rng.standard_normal(96)
    want = torch.nn.functional.rms_norm(torch.from_numpy(h), (96,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rms_norm(h, g), want, rtol=1e-14)


def _zero_experts(hidden, inter, groups):
    z = lambda n, k: (np.zeros((n, k // 2), np.uint8), np.full((n, k // 32), 127, np.uint8))
    return [dict(gate=z(inter, hidden), up=z(inter, hidden), down=z(hidden, inter)) for _ in range(groups)]


def test_chain_with_zero_experts_keeps_the_residual():
    # every expert is zero, so each y_l = 0: h_L = h_0 and x_l = bf16(RMSNorm(h_0) * gamma_l), each
    # layer with its own gamma
    rng = np.random.default_rng(13)
    hidden, inter, e, k, layers = 64, 32, 4, 2, 3
    h0 = rng.standard_normal((3, hidden))
    gammas = [1 + 0.1 * rng.standard_normal(hidden) for _ in range(layers)]
    routers = [(0.1 * rng.standard_normal((e, hidden))).astype(np.float32) for _ in range(layers)]
    out = oracle.chain_forward(h0, gammas, routers, [None] * layers, [_zero_experts(hidden, inter, e + 1)] * layers,
                               k, 1)
    np.testing.assert_array_equal(out["h"], h0)
    for l in range(layers):
        want = torch.nn.functional.rms_norm(torch.from_numpy(h0), (hidden,), torch.from_numpy(gammas[l]),
                                            eps=1e-6).numpy()
        np.testing.assert_array_equal(out["x"][l], oracle.f64_to_bf16_bits(want))
        assert (out["y"][l] == 0).all()


def test_chain_identity_experts_closed_form():
    # two layers of identity experts (closed form of each layer as in the single-layer pin): the
    # residual after layer l is h_l + y_l with y_l[h] = c_l * silu(x_h) * 2 x_h for h < I, 0 above
    hidden, inter, experts, k = 128, 64, 6, 2
    groups, wr, _, sigma = _identity_setup(hidden, inter, experts, k)
    rng = np.random.default_rng(14)
    h0 = rng.standard_normal((4, hidden))
    gammas = [np.ones(hidden), 1 + 0.1 * rng.standard_normal(hidden)]
    out = oracle.chain_forward(h0, gammas, [wr, wr], [None, None], [groups, groups], k, 1)
    h = h0.copy()
    for l in range(2):
        want_x = oracle.f64_to_bf16_bits(torch.nn.functional.rms_norm(
            torch.from_numpy(h), (hidden,), torch.from_numpy(gammas[l]), eps=1e-6).numpy())
        np.testing.assert_array_equal(out["x"][l], want_x)
        xf = bf16_bits_to_f64(want_x)
        r = out["route"][l]
        coef = 2.0 ** -sigma[experts] + (r["w"] * 2.0 ** -np.array(sigma)[r["idx"]]).sum(axis=1)
        y = np.zeros_like(h)
        v = xf[:, :inter]
        y[:, :inter] = coef[:, None] * (v / (1 + np.exp(-v))) * 2 * v
        np.testing.assert_allclose(out["y"][l], y, rtol=1e-13, atol=1e-300)
        h = h + y
    np.testing.assert_allclose(out["h"], h, rtol=1e-13)
