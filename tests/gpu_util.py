"""Helpers for the GPU parity tests: build layers on the device, run them, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import moe_synth as synth
import oracle
from oracle.moe import bf16_bits_to_f64

REL_L2_TOL = 5e-3          # relative L2 error of y
MAX_ABS_OVER_RMS_TOL = 2e-2  # max |dy| relative to rms(y_ref)
U32 = 2.0 ** -24            # unit roundoff of fp32


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def require_gpu():
    import fp4_routed_expert_moe_amd as m
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    m.load_library()
    ok, arch = m.device_supported(0)
    assert ok, f"device 0 is {arch}, not gfx950"


def stack_groups(groups, device="cuda"):
    """List of per-group dicts (numpy codes/scales) -> dict mat -> (codes, scales) device tensors."""
    out = {}
    for mat in synth.MATRICES:
        c = np.stack([g[mat][0] for g in groups])
        s = np.stack([g[mat][1] for g in groups])
        out[mat] = (torch.from_numpy(c).to(device).contiguous(), torch.from_numpy(s).to(device).contiguous())
    return out


def pack_weights(weights):
    """Checkpoint-layout device weights -> kernel layout, through the library's pack call."""
    from fp4_routed_expert_moe_amd import pack_fp4
    return {mat: pack_fp4(*weights[mat]) for mat in synth.MATRICES}


def make_layer(w_router, weights, top_k, n_shared, bias=None, path="auto", packed=None):
    """Layer over checkpoint-layout device weights (packed here unless `packed` is given)."""
    from fp4_routed_expert_moe_amd import MoeLayer
    wr = torch.from_numpy(np.ascontiguousarray(w_router, dtype=np.float32)).cuda()
    b = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias, dtype=np.float32)).cuda()
    pk = packed if packed is not None else pack_weights(weights)
    layer = MoeLayer(wr, pk["gate"], pk["up"], pk["down"], top_k, n_shared, b, path)
    return layer


def x_to_device(x_bits):
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda()


def run_layer(layer, x_bits, workspace=None):
    """Forward with the routing written out, and again without it: a call whose caller reads
    no routing builds only the tables its expert kernels use (for small batches), and must
    give the same output bit for bit."""
    x = x_to_device(x_bits)
    route = layer.route_buffers(x.shape[0])
    y = layer.forward(x, workspace=workspace, route=route)
    y_lean = layer.forward(x, workspace=workspace)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y_lean.view(torch.int32)), "output differs without routing outputs"
    out = {k: v.cpu().numpy() for k, v in route.items()}
    out["y"] = y.cpu().numpy()
    return out


def kernel_layout_scales(scales):
    """The kernel scale layout written out: [G][K/128][N/64][16 m][4 q][4 j] holds the scale of
    row 64t + 16j + m, block 4i + q, zero-padded past the matrix."""
    g, n, kb = scales.shape
    ki, nt = -(-kb // 4), -(-n // 64)
    padded = np.zeros((g, nt * 64, ki * 4), dtype=np.uint8)
    padded[:, :n, :kb] = scales
    # row 64t + 16j + m -> (t, j, m); block 4i + q -> (i, q)
    six = padded.reshape(g, nt, 4, 16, ki, 4)           # [g][t][j][m][i][q]
    return six.transpose(0, 4, 1, 3, 5, 2)              # [g][i][t][m][q][j]


def weight_tolerance(x_bits, w_router, bias, idx):
    """Per-token bound on |w_gpu - w_ref| from the arithmetic (not fitted to results).

    A GPU score is an fp32 sum of the H products x_h * W[e,h] (+ b_e) in some fixed order.  The
    longest chain of fp32 roundings is the matrix-core router's: one per MFMA step for each of
    the three bf16 terms of W (3H/32), plus the reduction tail; bound it by n = 2*(3H/32) + 64.
    Every partial sum is at most S = sum_h |x_h W[e,h]| + |b_e|, so |dl| <= n * u * S (Higham's
    gamma_n bound), and the oracle's rounding of its float64 score to fp32 adds u * |l|.  A
    softmax weight moves by at most 2 * max_j |dl_j| (d w_j / d l_i = w_j (delta_ij - w_i)),
    and the fp32 exp and divide add a few ulps (1e-6 covers them).
    """
    x = bf16_bits_to_f64(x_bits)
    w = np.asarray(w_router, dtype=np.float64)
    h = w.shape[1]
    s = np.abs(x) @ np.abs(w).T                       # [T][E]
    if bias is not None:
        s = s + np.abs(np.asarray(bias, dtype=np.float64))
    n = 2 * (3 * h // 32) + 64
    dl = np.take_along_axis(s, np.asarray(idx, dtype=np.int64), axis=1).max(axis=1) * (n + 1) * U32
    return 2.0 * dl + 1e-6                            # [T]


def check_routing(got, ref, x_bits, w_router, bias=None):
    np.testing.assert_array_equal(got["idx"], ref["idx"])
    np.testing.assert_array_equal(got["counts"], ref["counts"])
    np.testing.assert_array_equal(got["offsets"], ref["offsets"])
    np.testing.assert_array_equal(got["perm"], ref["perm"])
    tol = weight_tolerance(x_bits, w_router, bias, ref["idx"])
    err = np.abs(np.asarray(got["weight"], dtype=np.float64) - ref["w"]).max(axis=1)
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, f"routing weights off for tokens {bad[:8]}: err {err[bad[:8]]} > tol {tol[bad[:8]]}"


def output_error(y, y_ref):
    y = np.asarray(y, dtype=np.float64)
    d = y - y_ref
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    nref = float(np.linalg.norm(y_ref))
    return dict(rel_l2=float(np.linalg.norm(d)) / nref if nref else float(np.linalg.norm(d)),
                max_abs=float(np.abs(d).max()) if d.size else 0.0, rms_ref=rms,
                max_over_rms=float(np.abs(d).max()) / rms if rms else float(np.abs(d).max()),
                max_ref=float(np.abs(y_ref).max()) if d.size else 0.0)


def check_outputs(y, y_ref, what=""):
    if y_ref.size == 0:
        return {}
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    e = output_error(y, y_ref)
    say(f"  {what}: rel_l2={e['rel_l2']:.3e} max_abs={e['max_abs']:.3e} "
        f"max/rms={e['max_over_rms']:.3e} rms_ref={e['rms_ref']:.3e}")
    if e["rms_ref"] == 0:
        assert e["max_abs"] == 0
        return e
    assert e["rel_l2"] <= REL_L2_TOL, e
    assert e["max_over_rms"] <= MAX_ABS_OVER_RMS_TOL, e
    return e


def oracle_routing(x_bits, w_router, bias, top_k):
    logits = oracle.router_logits(x_bits, w_router, bias)
    idx, w, _ = oracle.select_experts(logits, top_k)
    counts, offsets, perm = oracle.group_rows(idx, np.asarray(w_router).shape[0])
    return dict(idx=idx, w=w, counts=counts, offsets=offsets, perm=perm)


def check_device_weights(wl, layer, weights, groups):
    """Device-generated weights equal the host generator's bytes for the given groups."""
    for g in groups:
        for mat in synth.MATRICES:
            c, s = synth.expert_matrix(wl, layer, mat, g)
            assert torch.equal(weights[mat][0][g].cpu(), c), (mat, g)
            assert torch.equal(weights[mat][1][g].cpu(), s), (mat, g)
