"""GPU parity of the shared expert stored in FP8 E4M3 with float32 128 x 128 block scales, and of the
routed scale, against the float64 oracle on the same inputs.

The routed experts stay FP4; the shared expert's matrices are FP8 (the V4 checkpoints' dense format,
"Add DeepSeek V4 Flash CPU inference with NVMe expert streaming", PR #165, the question on V4
sizes).  Routing must match bit for bit; outputs within the layer's output tolerance.
"""
import numpy as np
import pytest
import torch

import moe_synth as synth
import oracle
from helpers import as_oracle_fp8, identity_experts, identity_fp8_shared, random_experts, random_fp8_shared, \
    screened_tokens
from gpu_util import (check_device_weights, check_outputs, check_routing, make_layer, oracle_routing,
                      oracle_sampled, require_gpu, run_layer, sample_tokens, say, stack_groups)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("shape", [(1, 128, 128), (1, 2048, 4096), (1, 4096, 2048), (3, 384, 256)])
def test_pack_fp8_is_the_block_transpose(shape):
    from fp4_routed_expert_moe_amd import pack_fp8
    g, n, k = shape
    codes = np.random.default_rng(n * 7 + k).integers(0, 256, (g, n, k), dtype=np.uint8)
    got = pack_fp8(torch.from_numpy(codes).cuda()).cpu().numpy()
    want = codes.reshape(g, n, k // 128, 128).transpose(0, 2, 1, 3)   # [G][K/128][N][128]
    np.testing.assert_array_equal(got, want)


def _fp8_case(seed, hidden, experts, top_k, inter, tokens, bias=False):
    rng = np.random.default_rng(seed)
    groups = random_experts(rng, hidden, inter, experts)
    shared = random_fp8_shared(rng, hidden, inter)
    wr = (0.02 * rng.standard_normal((experts, hidden))).astype(np.float32)
    b = rng.standard_normal(experts).astype(np.float32) if bias else None
    wl = synth.custom_workload(f"fp8case{seed}", hidden, experts, top_k, 1, inter, tokens, shared_fp8=True)
    x = screened_tokens(wl, wr, b)
    return groups, shared, wr, b, x


def _check_fp8(groups, shared, wr, b, x, top_k, routed_scale=1.0, paths=("gemv", "gemm"), what=""):
    ref = oracle.moe_forward(x, wr, b, list(groups) + [as_oracle_fp8(shared)], top_k, 1, routed_scale)
    weights = stack_groups(groups)
    outs = {}
    for path in paths:
        layer = make_layer(wr, weights, top_k, 1, b, path, shared_fp8=shared, routed_scale=routed_scale)
        got = run_layer(layer, x)
        check_routing(got, ref, x, wr, b)
        check_outputs(got["y"], ref["y"], f"{what} path={path}")
        outs[path] = got
    return outs


@pytest.mark.parametrize("case", [
    # (seed, H, E, k, I, T, routed_scale)  H and I multiples of 128
    (21, 256, 8, 2, 128, 16, 1.0),
    (22, 512, 16, 4, 256, 100, 2.5),     # several 64-row tiles with a ragged tail, scaled routed sum
    (23, 384, 32, 6, 384, 129, 1.0),     # three 128-blocks on each axis
    (24, 1024, 64, 8, 512, 33, 0.5),
    (25, 128, 4, 2, 128, 1, 1.0),        # one token, one block
    (26, 256, 16, 4, 256, 700, 1.7),     # eleven 64-row tiles of the shared expert in the GEMM path
    (27, 256, 8, 2, 256, 2080, 1.0),     # ~520 rows an expert and 33 FP8 shared M-tiles
])
def test_fp8_shared_random_shapes_both_paths(case):
    seed, hidden, experts, k, inter, tokens, rs = case
    groups, shared, wr, b, x = _fp8_case(seed, hidden, experts, k, inter, tokens, bias=seed % 2 == 0)
    _check_fp8(groups, shared, wr, b, x, k, rs, what=f"fp8 case{case}")


def test_fp8_shared_identity_closed_form_on_gpu():
    # FP4 identity routed experts and an FP8 identity shared expert whose down block scale is 0.75:
    # y_h = (0.75 + sum_j w_j 2^-sigma_j) * silu(x_h) * 2 x_h for h < I, 0 elsewhere
    hidden, inter, experts, k = 256, 128, 6, 2
    rng = np.random.default_rng(0)
    sigma = [g + 1 for g in range(experts)]
    groups = identity_experts(hidden, inter, experts, 0, sigma)
    shared = identity_fp8_shared(hidden, inter, 0.75)
    wr = (0.3 * rng.standard_normal((experts, hidden))).astype(np.float32)
    wl = synth.custom_workload("ident8", hidden, experts, k, 1, inter, 5, shared_fp8=True)
    x = screened_tokens(wl, wr, None)
    outs = _check_fp8(groups, shared, wr, None, x, k, what="identity fp8")
    from oracle.moe import bf16_bits_to_f64
    xf = bf16_bits_to_f64(x)
    for got in outs.values():
        coef = 0.75 + (got["weight"] * 2.0 ** -np.array(sigma)[got["idx"]]).sum(axis=1)
        want = np.zeros_like(xf)
        v = xf[:, :inter]
        want[:, :inter] = coef[:, None] * (v / (1 + np.exp(-v))) * 2 * v
        check_outputs(got["y"], want, "identity fp8 closed form")
        assert (got["y"][:, inter:] == 0).all()


@pytest.mark.parametrize("routed_scale", [0.25, 2.5])
def test_routed_scale_with_fp4_shared_both_paths(routed_scale):
    rng = np.random.default_rng(31)
    hidden, experts, k, inter = 256, 16, 4, 128
    groups = random_experts(rng, hidden, inter, experts + 1)
    wr = (0.02 * rng.standard_normal((experts, hidden))).astype(np.float32)
    wl = synth.custom_workload("rscale", hidden, experts, k, 1, inter, 90)
    x = screened_tokens(wl, wr, None)
    ref = oracle.moe_forward(x, wr, None, groups, k, 1, routed_scale)
    weights = stack_groups(groups)
    for path in ("gemv", "gemm"):
        got = run_layer(make_layer(wr, weights, k, 1, None, path, routed_scale=routed_scale), x)
        check_routing(got, ref, x, wr, None)
        check_outputs(got["y"], ref["y"], f"routed_scale={routed_scale} path={path}")


def test_fp8_layer_rejects_bad_shapes():
    from fp4_routed_expert_moe_amd import MoeError
    rng = np.random.default_rng(5)
    hidden, experts, k, inter = 256, 8, 2, 96                # I not a multiple of 128
    groups = random_experts(rng, hidden, inter, experts)
    wr = (0.02 * rng.standard_normal((experts, hidden))).astype(np.float32)
    shared = {m: (torch.zeros((n, kk), dtype=torch.uint8), torch.ones((-(-n // 128), -(-kk // 128))))
              for m, (n, kk) in (("gate", (inter, hidden)), ("up", (inter, hidden)), ("down", (hidden, inter)))}
    with pytest.raises((MoeError, ValueError)):
        make_layer(wr, stack_groups(groups), k, 1, shared_fp8=shared)


@pytest.mark.parametrize("path", ["auto", "gemm"])
def test_decode_fp8_shared_full_size(path):
    # V4 Flash decode shape (H 4096, 256 experts, I 2048, top-6, 8 tokens) with the shared expert in
    # FP8; every token checked against the oracle
    wl = synth.WORKLOADS["decode_t8_fp8shared"]
    say(f"[{wl.name}] generating weights on the GPU")
    weights = synth.layer_weights(wl, 0, device="cuda")
    shared = synth.shared_fp8_weights(wl, 0, device="cuda")
    torch.cuda.synchronize()
    check_device_weights(wl, 0, weights, [0, 97, wl.experts - 1])
    for mat in synth.MATRICES:
        c, s = synth.shared_fp8_matrix(wl, 0, mat)
        assert torch.equal(shared[mat][0].cpu(), c) and torch.equal(shared[mat][1].cpu(), s), mat
    wr = synth.router_weights(wl, 0)
    x = screened_tokens(wl, wr, None)
    layer = make_layer(wr, weights, wl.top_k, wl.shared, None, path, shared_fp8=shared)
    got = run_layer(layer, x)
    ref_route = oracle_routing(x, wr, None, wl.top_k)
    check_routing(got, ref_route, x, wr, None)
    tokens = np.arange(x.shape[0])
    say(f"[{wl.name}] oracle on {len(tokens)} tokens")
    ref_y = oracle_sampled(wl, 0, x, wr, None, tokens, ref_route["idx"])
    check_outputs(got["y"], ref_y, f"{wl.name} path={path}")


def test_prefill_fp8_shared_sampled():
    # 512 tokens at the V4 Flash shapes with an FP8 shared expert: the GEMM path's shared M-tiles
    wl = synth.custom_workload("prefill_t512_fp8shared", 4096, 256, 6, 1, 2048, 512, shared_fp8=True)
    weights = synth.layer_weights(wl, 0, device="cuda")
    shared = synth.shared_fp8_weights(wl, 0, device="cuda")
    wr = synth.router_weights(wl, 0)
    x = screened_tokens(wl, wr, None)
    layer = make_layer(wr, weights, wl.top_k, wl.shared, None, shared_fp8=shared)
    got = run_layer(layer, x)
    ref_route = oracle_routing(x, wr, None, wl.top_k)
    check_routing(got, ref_route, x, wr, None)
    sample = sample_tokens(got, wl.top_k, spread=40)
    say(f"[{wl.name}] oracle on {len(sample)} sampled tokens")
    ref_y = oracle_sampled(wl, 0, x, wr, None, sample, ref_route["idx"])
    check_outputs(got["y"][sample], ref_y, wl.name)
