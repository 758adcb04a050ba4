"""Helpers for the GPU parity tests: build layers on the device, run them, compare with the oracle."""
from __future__ import annotations

import concurrent.futures
import multiprocessing
import os
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


def pack_shared_fp8(shared):
    """FP8 shared expert, dict mat -> (codes [N][K], float32 scales) on the host or the device ->
    the kernel layout (codes through the library's pack call), as MoeLayer's ``shared_fp8``."""
    from fp4_routed_expert_moe_amd import pack_fp8
    out = {}
    for mat in synth.MATRICES:
        c, sc = shared[mat]
        c = torch.as_tensor(np.asarray(c) if not torch.is_tensor(c) else c).cuda().contiguous()
        sc = torch.as_tensor(np.asarray(sc) if not torch.is_tensor(sc) else sc).cuda().contiguous()
        out[mat] = (pack_fp8(c[None])[0], sc)
    return out


def make_layer(w_router, weights, top_k, n_shared, bias=None, path="auto", packed=None, shared_fp8=None,
               routed_scale=1.0):
    """Layer over checkpoint-layout device weights (packed here unless `packed` is given); with
    ``shared_fp8`` (see ``pack_shared_fp8``) the FP4 weights hold the routed experts only."""
    from fp4_routed_expert_moe_amd import MoeLayer
    wr = torch.from_numpy(np.ascontiguousarray(w_router, dtype=np.float32)).cuda()
    b = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias, dtype=np.float32)).cuda()
    pk = packed if packed is not None else pack_weights(weights)
    f8 = None if shared_fp8 is None else pack_shared_fp8(shared_fp8)
    layer = MoeLayer(wr, pk["gate"], pk["up"], pk["down"], top_k, n_shared, b, path, shared_fp8=f8,
                     routed_scale=routed_scale)
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


def router_chain(tokens, experts, hidden):
    """Which router kernel scores a batch of `tokens`, and the longest rounding chain of a score.

    The library's dispatch rule (route.hip, route_fused / router_slices): batches with
    T <= 64 and T*E <= 8192 are scored by the one-launch FMA router, larger ones by the
    matrix-core router cut into `slices` hidden-axis slices.  Chains, in fp32 roundings a
    product can pass before the score is final:
    * FMA router: one per FMA of the lane (8 per 512 values of a quarter of H), four DPP adds
      and three lane-total adds, three quarter adds, the bias: 8*ceil(H/2048) + 11, each a
      round-to-nearest (unit u = 2^-24).
    * matrix-core router: the step's MFMA (32 exact products from zero, any internal order:
      at most 31), one add per 32-value step of the longest slice, the low-term add, one per
      slice in the top-k's sum, the bias.  Counted at 2u each, which also covers a matrix
      core that truncates.  The low bf16 terms of W_r (at most 2^-7 of |W_r|) add a chain of
      31 + 2*steps of their own.
    """
    if tokens <= 64 and tokens * experts <= 8192:
        return dict(kind="fused", n=8 * -(-hidden // 2048) + 11, unit=U32, lo_n=0)
    tiles = -(-tokens // 64) * -(-experts // 64)
    ks = min(max(-(-512 // tiles), 1), 16, hidden // 32)
    steps = -(-(hidden // 32) // ks)
    return dict(kind="gemm", slices=ks, n=31 + steps + 1 + ks + 1, unit=2 * U32, lo_n=31 + 2 * steps)


def weight_tolerance(x_bits, w_router, bias, idx, w_ref=None, tokens_per_call=None):
    """Bound on |w_gpu - w_ref| for each selected (token, slot), [T][k], from the arithmetic of
    the router kernel that scored the batch (router_chain), not fitted to results.

    Score error: every product x_h*W[e,h] and the bias pass at most n roundings of relative
    size `unit`, so |dl_e| <= gamma_n * S_e with S_e = sum_h |x_h W[e,h]| + |b_e| (Higham's
    bound for any summation order of that height), plus the low-term chain, plus u*|l_e| for
    the oracle's own rounding of its float64 score to fp32.
    Weight error: w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) moves by w_j (dl_j - sum_i w_i
    dl_i) to first order, so |dw_j| <= w_j (|dl_j| + sum_i w_i |dl_i|); the kernel's own fp32
    exp, sum and divide add w_j (|l_j - l_0| + k + 12) u.
    """
    x = bf16_bits_to_f64(x_bits)
    w = np.asarray(w_router, dtype=np.float64)
    t_count, hidden = x.shape
    experts = w.shape[0]
    idx = np.asarray(idx, dtype=np.int64)
    k = idx.shape[1]
    ch = router_chain(tokens_per_call or t_count, experts, hidden)
    s = np.abs(x) @ np.abs(w).T                        # [T][E]
    l = x @ w.T
    if bias is not None:
        bb = np.asarray(bias, dtype=np.float64)
        s = s + np.abs(bb)
        l = l + bb
    n, unit = ch["n"], ch["unit"]
    gamma = n * unit / (1.0 - n * unit)
    lo = ch["lo_n"] * unit * 2.0 ** -7 * 1.01
    dl_all = (gamma + lo + 1e-12) * s + U32 * np.abs(l)
    dl = np.take_along_axis(dl_all, idx, axis=1)      # [T][k]
    ls = np.take_along_axis(l, idx, axis=1)
    if w_ref is None:
        p = np.exp(ls - ls[:, :1])
        w_ref = p / p.sum(axis=1, keepdims=True)
    w_ref = np.asarray(w_ref, dtype=np.float64)
    first = w_ref * (dl + (w_ref * dl).sum(axis=1, keepdims=True)) * 1.01
    own = w_ref * (np.abs(ls - ls[:, :1]) + k + 12) * U32
    return first + own + 1e-9


def check_routing(got, ref, x_bits, w_router, bias=None, tokens_per_call=None):
    np.testing.assert_array_equal(got["idx"], ref["idx"])
    np.testing.assert_array_equal(got["counts"], ref["counts"])
    np.testing.assert_array_equal(got["offsets"], ref["offsets"])
    np.testing.assert_array_equal(got["perm"], ref["perm"])
    check_weights(got["weight"], ref, x_bits, w_router, bias, tokens_per_call)


def check_weights(weight, ref, x_bits, w_router, bias=None, tokens_per_call=None):
    tol = weight_tolerance(x_bits, w_router, bias, ref["idx"], ref["w"], tokens_per_call)
    err = np.abs(np.asarray(weight, dtype=np.float64) - ref["w"])
    bad = np.argwhere(err > tol)
    assert bad.size == 0, (f"routing weights off at (token, slot) {bad[:8].tolist()}: "
                           f"err {err[tuple(bad[:8].T)]} > tol {tol[tuple(bad[:8].T)]}")


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


# ---- the oracle on many sampled tokens, in parallel host processes -------------------------
# The float64 oracle decodes each expert it meets (about 1 s per expert at H=4096, I=2048), so
# full-size checks run it in worker processes (spawned: the parent has a HIP context), each on
# a chunk of the sampled tokens whose routed experts overlap.
_POOL = None


def oracle_workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _one_thread():
    # each worker runs numpy on one core: the pool, not BLAS threads, spreads the work
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)
    torch.set_num_threads(1)


def _pool():
    global _POOL
    if _POOL is None:
        _POOL = concurrent.futures.ProcessPoolExecutor(oracle_workers(), initializer=_one_thread,
                                                       mp_context=multiprocessing.get_context("spawn"))
    return _POOL


def _oracle_job(args):
    wl, layer, x_bits, w_router, bias, top_k, shared = args[:7]
    routed_scale = args[7] if len(args) > 7 else 1.0
    return oracle.moe_forward(x_bits, w_router, bias, synth.LazyExperts(wl, layer, cache=2), top_k, shared,
                              routed_scale)["y"]


def oracle_outputs(jobs):
    """y of oracle.moe_forward for each job (wl, layer, x_bits, w_router, bias, top_k, shared
    [, routed_scale]); the experts are the workload's seeded ones."""
    return list(_pool().map(_oracle_job, jobs))


def oracle_sampled(wl, layer, x_bits, w_router, bias, tokens, idx, routed_scale=1.0):
    """Oracle outputs [len(tokens)][H] of the given tokens of one layer call, computed in chunks
    of tokens grouped by their first expert (so a chunk decodes fewer distinct experts)."""
    tokens = np.asarray(tokens)
    order = tokens[np.argsort(np.asarray(idx)[tokens, 0], kind="stable")]
    n = min(len(order), 2 * oracle_workers())
    chunks = [c for c in np.array_split(order, n) if len(c)]
    ys = oracle_outputs([(wl, layer, np.ascontiguousarray(x_bits[c]), w_router, bias, wl.top_k, wl.shared,
                          routed_scale) for c in chunks])
    out = {}
    for c, y in zip(chunks, ys):
        for t, row in zip(c, y):
            out[int(t)] = row
    return np.stack([out[int(t)] for t in tokens])


def sample_tokens(got, top_k, spread=48, hot=3, per_hot=8):
    """Tokens whose outputs a full-size test checks: `spread` evenly over the batch, and in each of
    the `hot` experts with the most rows, the tokens of its first and last grouped rows, the last
    row of its first 64-row M-tile, the first row of its last (partial) M-tile, and `per_hot`
    rows spread in between."""
    t_count = got["idx"].shape[0]
    picks = set(np.linspace(0, t_count - 1, min(spread, t_count)).astype(int).tolist())
    counts, offsets, perm = got["counts"], got["offsets"], got["perm"]
    for e in np.argsort(-counts, kind="stable")[:hot]:
        rows = perm[offsets[e]:offsets[e + 1]] // top_k
        n = len(rows)
        if n == 0:
            continue
        last_tile = 64 * ((n - 1) // 64)
        at = {0, min(63, n - 1), last_tile, n - 1} | set(np.linspace(0, n - 1, per_hot).astype(int).tolist())
        picks |= {int(rows[i]) for i in at}
    return np.array(sorted(picks))


# ---- chained decode -------------------------------------------------------------------------
NORM_REL = 64 * U32   # relative bound of the join kernel's fp32 RMSNorm value before its bf16 rounding


def check_bf16_near(got_bits, ref, rel=NORM_REL, what=""):
    """Each bf16 pattern in ``got_bits`` must be the round-to-nearest-even of some value within
    relative distance ``rel`` of the float64 ``ref``: the rounding of ``ref`` itself, or, when
    ``ref`` lies that close to a rounding boundary, its neighbour across it."""
    got = np.asarray(got_bits).view(np.uint16)
    ref = np.asarray(ref, dtype=np.float64)
    ok = ((got == oracle.f64_to_bf16_bits(ref)) | (got == oracle.f64_to_bf16_bits(ref * (1 - rel)))
          | (got == oracle.f64_to_bf16_bits(ref * (1 + rel))))
    bad = np.argwhere(~ok)
    assert bad.size == 0, (f"{what}: {len(bad)} bf16 values off, first at {bad[:4].tolist()}: "
                           f"got {got[tuple(bad[:4].T)]}, ref {ref[tuple(bad[:4].T)]}")
    return int((got != oracle.f64_to_bf16_bits(ref)).sum())   # values on the far side of a boundary


def check_routing_screened(got, ref, x_bits, w_router, bias, top_k):
    """Routing of a computed (not screened) input: tokens whose top-(k+1) float64 scores hold a gap
    under 1e-4 may order differently at any precision, so only the other tokens' experts and
    weights are compared; with no such token the whole grouping must match too.  Returns the
    mask of compared tokens."""
    near = oracle.screen_near_ties(x_bits, w_router, bias, top_k)
    keep = ~near
    if not near.any():
        check_routing(got, ref, x_bits, w_router, bias)
        return keep
    np.testing.assert_array_equal(got["idx"][keep], ref["idx"][keep])
    tol = weight_tolerance(x_bits, w_router, bias, ref["idx"], ref["w"])
    assert (np.abs(got["weight"][keep] - ref["w"][keep]) <= tol[keep]).all()
    assert int(got["counts"].sum()) == got["idx"].size
    return keep


def check_chain_teacher_forced(x_gpu, y_gpu, h_out, routes, h_in, gammas, routers, biases, y_refs, top_k,
                               eps=1e-6, what="chain"):
    """Every step of a GPU chain checked on the GPU's own inputs to that step:
    the residual h_{l+1} = fl32(h_l + y_l) bit for bit (h_L against h_out), each layer input x_l
    against the float64 RMSNorm of the GPU's h_l (check_bf16_near), each layer's routing of x_l
    against the oracle's (check_routing_screened), and y_l against ``y_refs[l]``, the oracle layer
    on the GPU's x_l.  Returns (compared tokens, bf16 values across a boundary)."""
    h = np.asarray(h_in, dtype=np.float32)
    compared, across = 0, 0
    for l in range(len(routers)):
        ref_x = oracle.rms_norm(h.astype(np.float64), gammas[l], eps)
        across += check_bf16_near(x_gpu[l], ref_x, what=f"{what} x[{l}]")
        xb = np.ascontiguousarray(x_gpu[l]).view(np.uint16)
        keep = np.ones(xb.shape[0], bool)
        if routes is not None:
            ref_r = oracle_routing(xb, routers[l], biases[l], top_k)
            keep = check_routing_screened(routes[l], ref_r, xb, routers[l], biases[l], top_k)
        check_outputs(y_gpu[l][keep], y_refs[l][keep], f"{what} y[{l}]")
        compared += int(keep.sum())
        h = (h + np.asarray(y_gpu[l], dtype=np.float32)).astype(np.float32)   # one fp32 rounding per add
    np.testing.assert_array_equal(np.asarray(h_out).view(np.uint32), h.view(np.uint32))
    return compared, across
