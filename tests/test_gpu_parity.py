"""GPU parity: the HIP layer against the float64 oracle on the same seeded inputs.

Routing (idx, counts, offsets, perm) must match bit for bit; weights within the bound that the
rounding chain of the router kernel that ran gives (gpu_util.weight_tolerance; a bf16-rounded
router breaks it, tests/test_tolerance_cpu.py); outputs within rel-L2 5e-3 and
max|dy| <= 2e-2 * rms(y_ref).
"""
import numpy as np
import pytest
import torch

import moe_synth as synth
import oracle
from helpers import random_experts, screened_tokens, identity_experts
from gpu_util import (check_device_weights, check_outputs, check_routing, kernel_layout_scales, make_layer,
                      oracle_routing, oracle_sampled, pack_weights, require_gpu, run_layer,
                      sample_tokens, say, stack_groups, x_to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _random_case(seed, hidden, experts, top_k, shared, inter, tokens, bias=False, scale_lo=123, scale_hi=127):
    rng = np.random.default_rng(seed)
    groups = random_experts(rng, hidden, inter, experts + shared, scale_lo, scale_hi)
    wr = (0.02 * rng.standard_normal((experts, hidden))).astype(np.float32)
    b = (rng.standard_normal(experts)).astype(np.float32) if bias else None
    wl = synth.custom_workload(f"case{seed}", hidden, experts, top_k, shared, inter, tokens)
    x = screened_tokens(wl, wr, b)
    return groups, wr, b, x


def _check_case(groups, wr, b, x, top_k, shared, paths=("gemv", "gemm"), what=""):
    ref = oracle.moe_forward(x, wr, b, groups, top_k, shared)
    weights = stack_groups(groups)
    outs = {}
    for path in paths:
        layer = make_layer(wr, weights, top_k, shared, b, path)
        got = run_layer(layer, x)
        check_routing(got, ref, x, wr, b)
        check_outputs(got["y"], ref["y"], f"{what} path={path}")
        outs[path] = got
    return outs


# ------------------------------------------------------------------------------- pack


@pytest.mark.parametrize("shape", [(3, 64, 256), (2, 100, 96), (1, 4096, 2048), (5, 7, 32), (2, 130, 4160)])
def test_pack_is_the_block_transpose(shape):
    from fp4_routed_expert_moe_amd import pack_fp4
    g, n, k = shape
    rng = np.random.default_rng(n + k)
    codes = rng.integers(0, 256, (g, n, k // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (g, n, k // 32), dtype=np.uint8)
    scales[:, 0, 0] = 0
    pc, ps = pack_fp4(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda())
    torch.cuda.synchronize()
    # a block whose scale byte is 0 (+0) is all zeros: its 16 code bytes are written as zeros
    blocks = codes.reshape(g, n, k // 32, 16) * (scales != 0)[..., None]
    want_c = blocks.transpose(0, 2, 1, 3)
    np.testing.assert_array_equal(pc.cpu().numpy(), want_c)
    np.testing.assert_array_equal(ps.cpu().numpy(), kernel_layout_scales(scales))


# ------------------------------------------------------------------------------- tiny


def test_tiny_workload_both_paths():
    wl = synth.WORKLOADS["tiny"]
    weights = synth.layer_weights(wl, 0, device="cuda")
    check_device_weights(wl, 0, weights, range(wl.groups))
    wr = synth.router_weights(wl)
    x = screened_tokens(wl, wr, None)
    ref = oracle.moe_forward(x, wr, None, synth.LazyExperts(wl, 0, cache=wl.groups), wl.top_k, wl.shared)
    for path in ("auto", "gemv", "gemm"):
        got = run_layer(make_layer(wr, weights, wl.top_k, wl.shared, None, path), x)
        check_routing(got, ref, x, wr)
        check_outputs(got["y"], ref["y"], f"tiny path={path}")


def test_identity_experts_closed_form_on_gpu():
    hidden, inter, experts, k = 128, 64, 6, 2
    rng = np.random.default_rng(0)
    sigma = [g + 1 for g in range(experts)] + [0]
    groups = identity_experts(hidden, inter, experts, 1, sigma)
    wr = (0.3 * rng.standard_normal((experts, hidden))).astype(np.float32)
    wl = synth.custom_workload("ident", hidden, experts, k, 1, inter, 5)
    x = screened_tokens(wl, wr, None)
    _check_case(groups, wr, None, x, k, 1, what="identity")


@pytest.mark.parametrize("case", [
    # (seed, H, E, k, S, I, T)  multi-tile, ragged tails, several routing chunks
    (1, 512, 16, 4, 1, 256, 100),
    (2, 256, 32, 6, 1, 128, 129),
    (3, 96, 5, 2, 1, 32, 7),        # H, I not multiples of 64; E < 64
    (4, 1024, 64, 8, 0, 512, 33),   # no shared expert
    (5, 288, 70, 3, 1, 160, 65),    # E not a multiple of 64
    (7, 128, 1024, 8, 1, 64, 8),    # the layer's expert limit, routed in one launch
    (8, 160, 1000, 4, 1, 96, 40),   # near the limit, chunked routing (T*E past one workgroup's LDS)
    (10, 64, 2, 1, 1, 32, 64),      # two experts, top-1, the one-launch routing's token limit
    (11, 256, 16, 4, 0, 128, 8),    # decode batch without a shared expert
    (12, 128, 8, 8, 1, 64, 4),      # decode batch routed to every expert
    (13, 96, 256, 2, 1, 32, 2048),  # router GEMM through LDS, hidden-axis slices of one 32-value step
    (14, 224, 256, 3, 1, 64, 2048), # router GEMM through LDS, slices of 32 and 64 values
    (15, 320, 8, 3, 1, 160, 2100),  # ~790 rows an expert: a dozen M-tiles each, ragged last tiles, K tails
    (16, 256, 12, 5, 0, 288, 2049), # no shared expert; a group's last M-tile short
    (17, 64, 1, 1, 1, 32, 5),       # a single routed expert (every weight 1.0)
    (18, 160, 3, 3, 1, 96, 130),    # k = E = 3 through the router GEMM, H and I not multiples of 128
])
def test_random_shapes_both_paths(case):
    seed, hidden, experts, k, shared, inter, tokens = case
    groups, wr, b, x = _random_case(seed, hidden, experts, k, shared, inter, tokens, bias=seed % 2 == 0)
    _check_case(groups, wr, b, x, k, shared, what=f"case{case}")


def test_top_k_equals_all_experts():
    groups, wr, b, x = _random_case(6, 128, 8, 8, 1, 64, 20)
    _check_case(groups, wr, b, x, 8, 1, what="k=E")


def test_every_token_on_one_expert():
    rng = np.random.default_rng(8)
    hidden, experts, k, inter, tokens = 256, 16, 2, 128, 150
    groups = random_experts(rng, hidden, inter, experts + 1)
    wr = (0.02 * rng.standard_normal((experts, hidden))).astype(np.float32)
    b = np.zeros(experts, np.float32)
    b[11] = 50.0                                     # expert 11 always first
    wl = synth.custom_workload("onehot", hidden, experts, k, 1, inter, tokens)
    x = screened_tokens(wl, wr, b)
    outs = _check_case(groups, wr, b, x, k, 1, what="hot expert")
    assert outs["gemm"]["counts"][11] == tokens


def test_zero_and_extreme_scales():
    # s=0 blocks next to non-zero ones, over a wide scale range (2^-17 .. 2^9), on both paths
    # under the standard gate.  The GEMV path carries x exactly and h with 12 significant bits
    # (three FP8 terms), so it is also held to rel-L2 1e-4; the GEMM path rounds h to 8 bits
    # (two terms, bf16's precision).
    groups, wr, b, x = _random_case(9, 256, 8, 2, 1, 128, 24, scale_lo=110, scale_hi=136)
    for g in groups[::2]:
        g["gate"][1][:, 0] = 0
        g["down"][1][5, :] = 0
    outs = _check_case(groups, wr, b, x, 2, 1, what="scales 110..136")
    ref = oracle.moe_forward(x, wr, b, groups, 2, 1)["y"]
    d = outs["gemv"]["y"].astype(np.float64) - ref
    assert np.linalg.norm(d) <= 1e-4 * np.linalg.norm(ref)


# ------------------------------------------------------------------------- e8m0 edges
# An e8m0 byte s is the float with bit pattern s << 23 ("DeepSeek V4: the CUDA kernels, as a tier
# rather than an engine", PR #772, the note on the MXFP4 decode): s = 0 is +0, s = 255 is +inf.


def test_e8m0_zero_scale_blocks_are_exact_zeros():
    # Every block of every expert at s = 0: all weights are +0, so y is +0 bit for bit.  Then only
    # the down matrices at s = 0, with gate/up normal: h is large (~1e3), so reading byte 0 as
    # 2^-127 instead of +0 would leave values around 1e-33 in y; +0 leaves exact zeros.
    for what in ("all", "down"):
        groups, wr, b, x = _random_case(21, 256, 8, 2, 1, 128, 24)
        for g in groups:
            for mat in (("gate", "up", "down") if what == "all" else ("down",)):
                g[mat][1][:] = 0
        ref = oracle.moe_forward(x, wr, b, groups, 2, 1)
        assert (ref["y"] == 0).all()
        weights = stack_groups(groups)
        for path in ("gemv", "gemm"):
            got = run_layer(make_layer(wr, weights, 2, 1, b, path), x)
            check_routing(got, ref, x, wr, b)
            nz = np.count_nonzero(got["y"].view(np.uint32))
            assert nz == 0, f"{what}/{path}: {nz} outputs are not +0 (max |y| {np.abs(got['y']).max():.3e})"


def test_e8m0_255_scale_blocks_are_non_finite_where_the_oracle_is():
    # One s = 255 (+inf) block in a gate row of routed expert 3 (every output of its tokens turns
    # non-finite through h) and one in a down row of expert 5 (one output column of its tokens).
    groups, wr, b, x = _random_case(22, 256, 8, 2, 1, 128, 24)
    groups[3]["gate"][1][7, 2] = 255
    groups[5]["down"][1][100, 1] = 255
    ref = oracle.moe_forward(x, wr, b, groups, 2, 1)
    bad_ref = ~np.isfinite(ref["y"])
    assert bad_ref.any() and not bad_ref.all()
    weights = stack_groups(groups)
    for path in ("gemv", "gemm"):
        got = run_layer(make_layer(wr, weights, 2, 1, b, path), x)
        check_routing(got, ref, x, wr, b)
        bad = ~np.isfinite(got["y"])
        mism = np.argwhere(bad != bad_ref)
        assert mism.size == 0, f"{path}: non-finite positions differ at {mism[:6].tolist()}"
        ok = ~bad_ref.any(axis=1)                      # tokens with no non-finite output
        check_outputs(got["y"][ok], ref["y"][ok], f"finite tokens path={path}")


# --------------------------------------------------------------- router switch


@pytest.mark.parametrize("experts,limit", [(256, 32), (64, 64)])
def test_router_switch_keeps_routing(experts, limit):
    # Batches up to `limit` tokens are scored by the one-launch FMA router, one more by the
    # matrix-core router (T*E > 8192 scores, or T > 64).  Both must route every token exactly as
    # the oracle does; a token's output differs between the two only by rounding.
    groups, wr, b, x = _random_case(23 + experts, 512, experts, 4, 1, 256, limit + 1)
    weights = stack_groups(groups)
    ref_all = oracle.moe_forward(x, wr, b, groups, 4, 1)
    for path in ("gemv", "gemm"):
        layer = make_layer(wr, weights, 4, 1, b, path)
        big = run_layer(layer, x)
        small = run_layer(layer, x[:limit])
        check_routing(big, ref_all, x, wr, b)
        ref_small = oracle.moe_forward(x[:limit], wr, b, groups, 4, 1)
        check_routing(small, ref_small, x[:limit], wr, b)
        np.testing.assert_array_equal(small["idx"], big["idx"][:limit])
        check_outputs(big["y"], ref_all["y"], f"T={limit + 1} path={path}")
        check_outputs(small["y"], ref_small["y"], f"T={limit} path={path}")
        for t in (0, limit // 2, limit - 1):
            one = run_layer(layer, x[t:t + 1])
            np.testing.assert_array_equal(one["idx"][0], big["idx"][t])
            np.testing.assert_array_equal(one["y"][0], small["y"][t])   # same router: same bits


def test_single_token_and_batch_equals_single():
    groups, wr, b, x = _random_case(10, 512, 32, 4, 1, 256, 12)
    weights = stack_groups(groups)
    for path in ("gemv", "gemm"):
        layer = make_layer(wr, weights, 4, 1, b, path)
        full = run_layer(layer, x)
        for t in (0, 5, 11):
            one = run_layer(layer, x[t:t + 1])
            np.testing.assert_array_equal(one["idx"][0], full["idx"][t])
            np.testing.assert_array_equal(one["y"][0], full["y"][t])


def test_zero_tokens_is_a_noop():
    groups, wr, b, x = _random_case(11, 128, 8, 2, 1, 64, 4)
    layer = make_layer(wr, stack_groups(groups), 2, 1, b)
    y = torch.full((0, 128), 7.0, device="cuda")
    out = layer.forward(torch.empty((0, 128), dtype=torch.int16, device="cuda"), y=y,
                        workspace=layer.workspace(1))
    torch.cuda.synchronize()
    assert out.shape == (0, 128)


def test_route_call_matches_forward_routing():
    groups, wr, b, x = _random_case(12, 256, 32, 6, 1, 128, 200)
    layer = make_layer(wr, stack_groups(groups), 6, 1, b)
    xd = x_to_device(x)
    r1 = layer.route(xd)
    r2 = layer.route_buffers(xd.shape[0])
    layer.forward(xd, route=r2)
    torch.cuda.synchronize()
    for k in r1:
        assert torch.equal(r1[k], r2[k]), k


def test_deterministic_repeat():
    groups, wr, b, x = _random_case(13, 512, 16, 4, 1, 256, 80)
    layer = make_layer(wr, stack_groups(groups), 4, 1, b, "gemm")
    a = run_layer(layer, x)
    c = run_layer(layer, x)
    np.testing.assert_array_equal(a["y"], c["y"])


def test_workspace_reuse_across_sizes_and_paths():
    # The control words in the workspace must be back at zero after every call, whatever
    # mix of fused (T <= 64) and chunked routing, GEMV and GEMM paths used it before.
    groups, wr, b, x = _random_case(15, 256, 32, 4, 1, 128, 150)
    weights = stack_groups(groups)
    gemv = make_layer(wr, weights, 4, 1, b, "gemv")
    gemm = make_layer(wr, weights, 4, 1, b, "gemm")
    ws = gemv.workspace(150)
    fresh = {}
    for t in (8, 150, 64, 65):
        fresh[("gemv", t)] = run_layer(gemv, x[:t])
        fresh[("gemm", t)] = run_layer(gemm, x[:t])
    for rep in range(2):
        for t in (8, 150, 1, 64, 65, 8):
            for name, layer in (("gemv", gemv), ("gemm", gemm)):
                got = run_layer(layer, x[:t], workspace=ws)
                ref = fresh.get((name, t)) or run_layer(layer, x[:t])
                np.testing.assert_array_equal(got["y"], ref["y"])
                np.testing.assert_array_equal(got["perm"], ref["perm"])


def test_workspace_errors():
    from fp4_routed_expert_moe_amd import MoeError
    groups, wr, b, x = _random_case(14, 128, 8, 2, 1, 64, 10)
    layer = make_layer(wr, stack_groups(groups), 2, 1, b)
    xd = x_to_device(x)
    small = torch.empty(layer.workspace_bytes(10) - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(MoeError) as ei:
        layer.forward(xd, workspace=small)
    assert ei.value.status == 3
    assert layer.workspace_bytes(10) <= layer.workspace_bytes(11)


# ------------------------------------------------------------------ full-size workloads


def _full_size(name, layer_index=0, spread=48):
    wl = synth.WORKLOADS[name]
    say(f"[{name}] generating weights on the GPU")
    weights = synth.layer_weights(wl, layer_index, device="cuda")
    torch.cuda.synchronize()
    check_device_weights(wl, layer_index, weights, [0, 97, wl.experts])
    wr = synth.router_weights(wl, layer_index)
    b = synth.router_bias(wl)
    x = screened_tokens(wl, wr, b, layer=layer_index)
    layer = make_layer(wr, weights, wl.top_k, wl.shared, b)
    say(f"[{name}] GPU forward T={x.shape[0]}")
    got = run_layer(layer, x)
    ref_route = oracle_routing(x, wr, b, wl.top_k)
    check_routing(got, ref_route, x, wr, b)
    sample = sample_tokens(got, wl.top_k, spread=spread)
    say(f"[{name}] oracle on {len(sample)} sampled tokens")
    ref_y = oracle_sampled(wl, layer_index, x, wr, b, sample, ref_route["idx"])
    check_outputs(got["y"][sample], ref_y, name)
    return got, layer, x, sample


def test_decode_batch_full_size():
    _, _, x, sample = _full_size("decode_t8")
    assert len(sample) == x.shape[0]


def test_prefill_512_full_size():
    _, _, _, sample = _full_size("prefill_t512")
    assert len(sample) >= 64


def test_prefill_4096_zipf_full_size():
    got, _, _, sample = _full_size("prefill_t4096_zipf")
    assert got["counts"].max() > 0.10 * got["idx"].size
    assert len(sample) >= 64


def test_decode_pro_scale_full_size():
    # DeepSeek V4 Pro scale: hidden 7168 (56 K steps of 128), 384 experts (top-k over 6 keys
    # per lane), 9 GB of FP4 experts; every token's output checked
    _, _, x, sample = _full_size("decode_pro_t8")
    assert len(sample) == x.shape[0]


def test_prefill_pro_scale_full_size():
    # V4 Pro scale through the grouped GEMM: 512 tokens, hidden 7168, 384 experts (router GEMM over
    # six 64-expert tiles, top-k over 8 keys per lane); outputs of 16 spread tokens plus the
    # first, last and M-tile-boundary rows of the three busiest experts
    got, _, x, sample = _full_size("prefill_pro_t512", spread=16)
    assert len(sample) >= 16 and got["counts"].sum() == x.shape[0] * 6


def test_stacked_decode_16_layers():
    wl = synth.WORKLOADS["stacked_decode_16l"]
    layers, routers = [], []
    for l in range(wl.layers):
        weights = synth.layer_weights(wl, l, device="cuda")
        if l == wl.layers - 1:
            check_device_weights(wl, l, weights, [3])
        packed = pack_weights(weights)
        del weights                                   # keep only the kernel layout resident
        wr = synth.router_weights(wl, l)
        layers.append((make_layer(wr, None, wl.top_k, wl.shared, packed=packed), packed))
        routers.append(wr)
    torch.cuda.synchronize()
    say("[stacked] 16 layers resident")
    steps = wl.steps
    xs = {}
    ws = layers[0][0].workspace(1)
    ys, routes = {}, {}
    for s in range(steps):
        for l in range(wl.layers):
            x = screened_tokens(wl, routers[l], None, layer=l, step=s)
            xs[(s, l)] = x
            layer = layers[l][0]
            r = layer.route_buffers(1)
            ys[(s, l)] = layer.forward(x_to_device(x), workspace=ws, route=r)
            routes[(s, l)] = r
        if s % 64 == 0:
            say(f"[stacked] step {s}")
    torch.cuda.synchronize()
    for (s, l), r in routes.items():
        ref = oracle_routing(xs[(s, l)], routers[l], None, wl.top_k)
        got = {k: v.cpu().numpy() for k, v in r.items()}
        check_routing(got, ref, xs[(s, l)], routers[l])
    # 16 (step, layer) calls, one per layer, steps spread over the run
    calls = [(17 * l, l) for l in range(wl.layers)]
    from gpu_util import oracle_outputs
    refs = oracle_outputs([(wl, l, xs[(s, l)], routers[l], None, wl.top_k, wl.shared) for s, l in calls])
    for (s, l), ref in zip(calls, refs):
        check_outputs(ys[(s, l)].cpu().numpy(), ref, f"stacked step={s} layer={l}")
