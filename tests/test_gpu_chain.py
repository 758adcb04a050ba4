"""GPU parity of the chained decode: the join step (residual add + RMSNorm + bf16) and whole chains
of MoE layers recorded into one HIP graph, checked step by step on the GPU's own intermediate values
(teacher forcing) against the float64 oracle, and graph replays against the same calls made eagerly.

The join is a reading of the pages (they run the MoE stage per layer and leave the join open): a
pre-norm residual stream, x_l = bf16(RMSNorm(h_l) * gamma_l), h_{l+1} = h_l + y_l, eps 1e-6.
"""
import numpy as np
import pytest
import torch

import moe_synth as synth
import oracle
from helpers import random_experts
from gpu_util import (U32, check_bf16_near, check_chain_teacher_forced, check_device_weights, make_layer,
                      oracle_outputs, pack_weights, require_gpu, say, stack_groups, x_to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ------------------------------------------------------------------------------- the join step


@pytest.mark.parametrize("tokens,hidden", [(1, 4096), (5, 96), (8, 7168), (3, 4), (2, 8196)])
def test_residual_rmsnorm_step(tokens, hidden):
    from fp4_routed_expert_moe_amd import residual_rmsnorm
    rng = np.random.default_rng(tokens * 1000 + hidden)
    h = (rng.standard_normal((tokens, hidden)) * 3).astype(np.float32)
    y = (rng.standard_normal((tokens, hidden)) * 1e4).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(hidden)).astype(np.float32)
    hd, yd, gd = _t(h), _t(y), _t(g)
    out = torch.empty_like(hd)
    x = torch.empty((tokens, hidden), dtype=torch.int16, device="cuda")
    residual_rmsnorm(hd, yd, out, gd, 1e-6, x)
    torch.cuda.synchronize()
    want_h = (h + y).astype(np.float32)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), want_h.view(np.uint32))
    check_bf16_near(x.cpu().numpy(), oracle.rms_norm(want_h.astype(np.float64), g), what="x")
    # in place (h_dst = h_src), the norm alone (no y), and no weight (all ones)
    residual_rmsnorm(hd, yd, hd, None, 1e-6, x)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(hd.cpu().numpy().view(np.uint32), want_h.view(np.uint32))
    check_bf16_near(x.cpu().numpy(), oracle.rms_norm(want_h.astype(np.float64), np.ones(hidden)), what="x in place")
    x2 = torch.empty_like(x)
    residual_rmsnorm(_t(h), None, None, gd, 1e-6, x2)
    torch.cuda.synchronize()
    check_bf16_near(x2.cpu().numpy(), oracle.rms_norm(h.astype(np.float64), g), what="x without y")


def test_residual_rmsnorm_edge_rows():
    # a zero row (eps keeps it finite: x = 0), a row of one repeated value, a row whose squares
    # approach the float32 range (sum of squares 2.6e36), and a row far below eps
    from fp4_routed_expert_moe_amd import residual_rmsnorm
    hidden = 256
    h = np.zeros((4, hidden), np.float32)
    h[1] = -0.25
    h[2] = np.linspace(-1e17, 1e17, hidden, dtype=np.float32)
    h[3] = np.linspace(-1e-8, 2e-8, hidden, dtype=np.float32)
    x = torch.empty((4, hidden), dtype=torch.int16, device="cuda")
    residual_rmsnorm(_t(h), None, None, None, 1e-6, x)
    torch.cuda.synchronize()
    got = x.cpu().numpy()
    assert (got[0] == 0).all()
    check_bf16_near(got, oracle.rms_norm(h.astype(np.float64), np.ones(hidden)), what="edge rows")


def test_residual_rmsnorm_bound_is_tight_enough_to_fail():
    # the comparison is not vacuous: x from a norm with eps outside the root, or over the row sum,
    # or without the weight, fails it
    rng = np.random.default_rng(3)
    h = rng.standard_normal((4, 512))
    g = 1 + 0.1 * rng.standard_normal(512)
    ms = np.mean(h * h, axis=1, keepdims=True)
    for wrong in (h / (np.sqrt(ms) + 1e-3) * g, h / np.sqrt(ms * 512) * g, h / np.sqrt(ms + 1e-6)):
        with pytest.raises(AssertionError):
            check_bf16_near(oracle.f64_to_bf16_bits(wrong), oracle.rms_norm(h, g))
    assert 64 * U32 < 2.0 ** -12


# ------------------------------------------------------------------------------- small chains


def _small_chain(seed, n_layers, hidden=256, experts=8, top_k=2, inter=128, shared=1):
    rng = np.random.default_rng(seed)
    layers, refs = [], []
    for _ in range(n_layers):
        groups = random_experts(rng, hidden, inter, experts + shared)
        wr = (0.05 * rng.standard_normal((experts, hidden))).astype(np.float32)
        layers.append(make_layer(wr, stack_groups(groups), top_k, shared))
        refs.append((groups, wr))
    gammas = [(1 + 0.1 * rng.standard_normal(hidden)).astype(np.float32) for _ in range(n_layers)]
    return layers, refs, gammas


# 16 tokens: the largest batch whose join runs inside the routing launch; 17: the join kernel
@pytest.mark.parametrize("n_layers,tokens", [(1, 3), (3, 5), (2, 16), (2, 17), (4, 40)])
def test_small_chain_teacher_forced(n_layers, tokens):
    from fp4_routed_expert_moe_amd import MoeChain
    layers, refs, gammas = _small_chain(20 + n_layers, n_layers)
    ch = MoeChain(layers, tokens, residual=True, norm_weight=[_t(g) for g in gammas], routes=True)
    h_in = np.random.default_rng(7).standard_normal((tokens, 256)).astype(np.float32)
    ch.h_in.copy_(_t(h_in))
    ch.run()
    torch.cuda.synchronize()
    x = ch.x.cpu().numpy().view(np.uint16)
    y = ch.y.cpu().numpy()
    routes = [{k: v.cpu().numpy() for k, v in r.items()} for r in ch.routes]
    y_refs = [oracle.moe_forward(x[l], refs[l][1], None, refs[l][0], 2, 1)["y"] for l in range(n_layers)]
    compared, across = check_chain_teacher_forced(x, y, ch.h_out.cpu().numpy(), routes, h_in, gammas,
                                                  [r[1] for r in refs], [None] * n_layers, y_refs, 2)
    say(f"[chain L={n_layers} T={tokens}] {compared} token-layers compared, {across} bf16 values across a boundary")
    assert compared >= n_layers * tokens - 2


def test_chain_graph_replays_match_eager_calls():
    # the graph, replayed three times with eager library work and synchronisations in between, gives
    # bit for bit what the same calls give eagerly, and a new h_in changes every replay's result
    from fp4_routed_expert_moe_amd import MoeChain, residual_rmsnorm
    n, t = 4, 6
    layers, _, gammas = _small_chain(31, n)
    gd = [_t(g) for g in gammas]
    ch = MoeChain(layers, t, residual=True, norm_weight=gd)
    rng = np.random.default_rng(8)

    def eager(h_in):
        hd = _t(h_in)
        h = torch.empty_like(hd)
        xs, ys = [], []
        for l in range(n):
            x = torch.empty((t, 256), dtype=torch.int16, device="cuda")
            if l == 0:
                residual_rmsnorm(hd, None, None, gd[0], 1e-6, x)
            else:
                residual_rmsnorm(hd if l == 1 else h, ys[-1], h, gd[l], 1e-6, x)
            ys.append(layers[l].forward(x))
            xs.append(x)
        residual_rmsnorm(hd if n == 1 else h, ys[-1], h, None, 1e-6, None)
        torch.cuda.synchronize()
        return torch.stack(xs).cpu(), torch.stack(ys).cpu(), h.cpu()

    for rep in range(3):
        h_in = rng.standard_normal((t, 256)).astype(np.float32) * (rep + 1)
        want = eager(h_in)
        ch.h_in.copy_(_t(h_in))
        ch.run()
        torch.cuda.synchronize()
        assert torch.equal(ch.x.cpu(), want[0]), rep
        assert torch.equal(ch.y.cpu().view(torch.int32), want[1].view(torch.int32)), rep
        assert torch.equal(ch.h_out.cpu().view(torch.int32), want[2].view(torch.int32)), rep
        ch.run()                           # a second replay on the same input: the same bits
        torch.cuda.synchronize()
        assert torch.equal(ch.h_out.cpu().view(torch.int32), want[2].view(torch.int32)), rep
        _ = layers[0].forward(x_to_device(np.zeros((3, 256), np.uint16)))   # eager work between replays
        torch.cuda.synchronize()


def test_stacked_chain_equals_independent_forwards():
    # without the residual the graph runs each layer on the input the caller wrote into x
    from fp4_routed_expert_moe_amd import MoeChain
    n, t = 5, 4
    layers, _, _ = _small_chain(41, n)
    ch = MoeChain(layers, t, residual=False, routes=True)
    xs = [synth.f32_to_bf16_bits(np.random.default_rng(l).standard_normal((t, 256)).astype(np.float32))
          for l in range(n)]
    for l in range(n):
        ch.x[l].copy_(x_to_device(xs[l]))
    for _ in range(2):
        ch.run()
        torch.cuda.synchronize()
        for l in range(n):
            want = layers[l].forward(x_to_device(xs[l]))
            torch.cuda.synchronize()
            assert torch.equal(ch.y[l].view(torch.int32), want.view(torch.int32)), l


def test_chain_with_fp8_shared_and_gemm_path():
    # layers with an FP8 shared expert, 40 tokens on the grouped-GEMM path
    from fp4_routed_expert_moe_amd import MoeChain
    from helpers import as_oracle_fp8, random_fp8_shared
    rng = np.random.default_rng(51)
    hidden, experts, k, inter, n, t = 256, 8, 2, 128, 2, 40
    layers, refs = [], []
    for _ in range(n):
        groups = random_experts(rng, hidden, inter, experts)
        sh = random_fp8_shared(rng, hidden, inter)
        wr = (0.05 * rng.standard_normal((experts, hidden))).astype(np.float32)
        layers.append(make_layer(wr, stack_groups(groups), k, 1, path="gemm", shared_fp8=sh))
        refs.append((list(groups) + [as_oracle_fp8(sh)], wr))
    gammas = [(1 + 0.1 * rng.standard_normal(hidden)).astype(np.float32) for _ in range(n)]
    ch = MoeChain(layers, t, residual=True, norm_weight=[_t(g) for g in gammas], routes=True)
    h_in = rng.standard_normal((t, hidden)).astype(np.float32)
    ch.h_in.copy_(_t(h_in))
    ch.run()
    torch.cuda.synchronize()
    x = ch.x.cpu().numpy().view(np.uint16)
    y_refs = [oracle.moe_forward(x[l], refs[l][1], None, refs[l][0], k, 1)["y"] for l in range(n)]
    routes = [{kk: v.cpu().numpy() for kk, v in r.items()} for r in ch.routes]
    check_chain_teacher_forced(x, ch.y.cpu().numpy(), ch.h_out.cpu().numpy(), routes, h_in, gammas,
                               [r[1] for r in refs], [None] * n, y_refs, k, what="fp8 chain")


# ------------------------------------------------------------------------------- full size


def test_chained_decode_16_layers_full_size():
    # one token through 16 V4 Flash MoE layers (55 GB of FP4 experts resident), teacher-forced:
    # every layer's input, routing, output and the residual checked against the oracle
    from fp4_routed_expert_moe_amd import MoeChain
    wl = synth.WORKLOADS["chained_decode_16l"]
    layers, keep, routers, gammas = [], [], [], []
    for l in range(wl.layers):
        weights = synth.layer_weights(wl, l, device="cuda")
        if l == wl.layers - 1:
            check_device_weights(wl, l, weights, [5])
        packed = pack_weights(weights)
        del weights
        wr = synth.router_weights(wl, l)
        layers.append(make_layer(wr, None, wl.top_k, wl.shared, packed=packed))
        keep.append(packed)
        routers.append(wr)
        gammas.append(synth.norm_weight(wl, l))
    torch.cuda.synchronize()
    say("[chained] 16 layers resident")
    ch = MoeChain(layers, wl.tokens, residual=True, norm_weight=[_t(g) for g in gammas], routes=True)
    for step in (0, 1):
        h_in = synth.residual_input(wl, step=step)
        ch.h_in.copy_(_t(h_in))
        ch.run()
        torch.cuda.synchronize()
        x = ch.x.cpu().numpy().view(np.uint16)
        y = ch.y.cpu().numpy()
        routes = [{k: v.cpu().numpy() for k, v in r.items()} for r in ch.routes]
        say(f"[chained] step {step}: oracle on 16 layers")
        y_refs = oracle_outputs([(wl, l, x[l], routers[l], None, wl.top_k, wl.shared) for l in range(wl.layers)])
        compared, across = check_chain_teacher_forced(x, y, ch.h_out.cpu().numpy(), routes, h_in, gammas, routers,
                                                      [None] * wl.layers, y_refs, wl.top_k, what=f"chained step {step}")
        say(f"[chained] step {step}: {compared} of 16 layer inputs compared, {across} bf16 values across a boundary")
        assert compared >= 15
