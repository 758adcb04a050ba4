"""moe_forward_noalloc (the workspace in the library's per-device scratch array) gives what
moe_forward with a caller workspace gives, bit for bit, call after call, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_outputs, check_routing, make_layer, require_gpu, stack_groups, x_to_device
from helpers import random_experts, screened_tokens
import moe_synth as synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _case(seed, hidden, experts, top_k, inter, tokens):
    rng = np.random.default_rng(seed)
    groups = random_experts(rng, hidden, inter, experts + 1)
    wr = (0.02 * rng.standard_normal((experts, hidden))).astype(np.float32)
    wl = synth.custom_workload(f"noalloc{seed}", hidden, experts, top_k, 1, inter, tokens)
    return groups, wr, screened_tokens(wl, wr, None)


def _both(layer, x, with_route):
    xd = x_to_device(x)
    t = xd.shape[0]
    r_ref = layer.route_buffers(t) if with_route else None
    y_ref = layer.forward(xd, route=r_ref)
    r_na = layer.route_buffers(t) if with_route else None
    y_na = torch.full((t, layer.hidden), float("nan"), device="cuda")
    layer.forward_noalloc(xd, y_na, route=r_na)
    torch.cuda.synchronize()
    assert torch.equal(y_na.view(torch.int32), y_ref.view(torch.int32)), "outputs differ from moe_forward"
    if with_route:
        for k in r_ref:
            assert torch.equal(r_na[k], r_ref[k]), k
    return y_na.cpu().numpy(), ({k: v.cpu().numpy() for k, v in r_na.items()} if with_route else None)


def test_noalloc_matches_forward_on_consecutive_calls():
    groups, wr, x = _case(31, 512, 32, 4, 256, 100)
    layer = make_layer(wr, stack_groups(groups), 4, 1)
    # 100 tokens (grouped GEMM, chunked routing), then 7 (GEMV, one-launch routing) in the same
    # scratch, then 100 again: nothing left over from an earlier call may change a result
    for t, with_route in ((100, True), (7, False), (7, True), (100, False)):
        y, r = _both(layer, x[:t], with_route)
        ref = oracle.moe_forward(x[:t], wr, None, groups, 4, 1)
        if r is not None:
            check_routing(r, ref, x[:t], wr)
        check_outputs(y, ref["y"], f"noalloc T={t}")


def test_noalloc_rejects_batches_beyond_the_scratch():
    from fp4_routed_expert_moe_amd import MoeError, _lib
    groups, wr, x = _case(32, 256, 8, 2, 128, 16)
    layer = make_layer(wr, stack_groups(groups), 2, 1)
    t = 16
    while layer.workspace_bytes(t) <= _lib.MOE_NOALLOC_SCRATCH_BYTES:
        t *= 2
    xd = torch.zeros((t, 256), dtype=torch.int16, device="cuda")
    y = torch.full((t, 256), 7.0, device="cuda")
    with pytest.raises(MoeError) as ei:
        layer.forward_noalloc(xd, y)
    assert ei.value.status == _lib.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "a rejected call must enqueue nothing"
    # the largest batch that fits still runs
    lo = t // 2
    while lo + 1 < t:
        mid = (lo + t) // 2
        lo, t = (mid, t) if layer.workspace_bytes(mid) <= _lib.MOE_NOALLOC_SCRATCH_BYTES else (lo, mid)
    xs = np.ascontiguousarray(np.resize(x, (lo, 256)))
    y_na, _ = _both(layer, xs, False)
    assert np.isfinite(y_na).all()
