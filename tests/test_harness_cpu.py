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
    idx, w_ref, _ = oracle.select_experts(oracle.router_logits(x, wr, None), wl.top_k)
    tol = weight_tolerance(x, wr, None, idx, w_ref)
    assert tol.shape == idx.shape and np.isfinite(tol).all() and (tol > 0).all()
    # the score part: w_j (dl_j + sum_i w_i dl_i) * 1.01 with dl = (gamma_n + 1e-12) S + u |l|
    xf = bf16_bits_to_f64(x)
    s = np.abs(xf) @ np.abs(wr.astype(np.float64)).T
    l = xf @ wr.astype(np.float64).T
    n = 8 * 1 + 11                                  # one 512-value step per quarter at H=256
    g = n * U32 / (1 - n * U32)
    dl = np.take_along_axis((g + 1e-12) * s + U32 * np.abs(l), idx.astype(np.int64), axis=1)
    ls = np.take_along_axis(l, idx.astype(np.int64), axis=1)
    want = (w_ref * (dl + (w_ref * dl).sum(axis=1, keepdims=True)) * 1.01
            + w_ref * (np.abs(ls - ls[:, :1]) + wl.top_k + 12) * U32 + 1e-9)
    np.testing.assert_allclose(tol, want, rtol=1e-12)


def test_kernel_scale_layout_by_hand():
    """One entry spelled out: row 64*1 + 16*2 + 5 = 101, block 4*1 + 3 = 7."""
    s = np.zeros((1, 130, 12), dtype=np.uint8)
    s[0, 101, 7] = 9
    lay = kernel_layout_scales(s)
    assert lay.shape == (1, 3, 3, 16, 4, 4) and lay.sum() == 9 and lay[0, 1, 1, 5, 3, 2] == 9
