"""CPU checks of the GPU-test harness's derived tolerances (no GPU needed)."""
import numpy as np

import moe_synth as synth
import oracle
from oracle.moe import bf16_bits_to_f64
from gpu_util import U32, kernel_layout_scales, weight_tolerance


def test_weight_tolerance_follows_the_summation_bound():
    wl = synth.WORKLOADS["tiny"]
    wr = synth.router_weights(wl)
    x = synth.tokens(wl)
    idx, _, _ = oracle.select_experts(oracle.router_logits(x, wr, None), wl.top_k)
    tol = weight_tolerance(x, wr, None, idx)
    assert tol.shape == (x.shape[0],) and np.isfinite(tol).all() and (tol > 1e-6).all()
    # doubling the weights doubles the score-magnitude part of the bound
    tol2 = weight_tolerance(x, 2 * wr, None, idx)
    np.testing.assert_allclose(tol2 - 1e-6, 2 * (tol - 1e-6), rtol=1e-12)
    # the bound is n * u * S with n = 2 * (3H/32) + 64 (+1 for the oracle's own rounding)
    s = np.abs(bf16_bits_to_f64(x)) @ np.abs(wr.astype(np.float64)).T
    n = 2 * (3 * wl.hidden // 32) + 64 + 1
    want = 2 * n * U32 * np.take_along_axis(s, idx.astype(np.int64), axis=1).max(axis=1) + 1e-6
    np.testing.assert_allclose(tol, want, rtol=1e-12)


def test_kernel_scale_layout_by_hand():
    """One entry spelled out: row 64*1 + 16*2 + 5 = 101, block 4*1 + 3 = 7."""
    s = np.zeros((1, 130, 12), dtype=np.uint8)
    s[0, 101, 7] = 9
    lay = kernel_layout_scales(s)
    assert lay.shape == (1, 3, 3, 16, 4, 4) and lay.sum() == 9 and lay[0, 1, 1, 5, 3, 2] == 9
