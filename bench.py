#!/usr/bin/env python3
"""Throughput of the routed FP4-expert MoE layer on one MI355X.

A step is one full layer call (router, top-k, grouping, gate/up with FP4 dequant and
SwiGLU, down projection, shared expert, combine) on one batch of synthetic tokens.
Default workload: the decode batch at DeepSeek V4 Flash expert shapes (H=4096, E=256,
top-6, 1 shared expert, I=2048, 8 tokens).  Steps rotate over 16 independent layers'
weights (55 GB resident) and 64 token batches, so no layer's weights are still in the
256 MB last-level cache when it runs again.

Prints one JSON line.  Besides tokens/s it reports:
* ``roofline``: the dominant kernel against its roof.  ``achieved`` = algorithmic bytes
  (or flops) per launch / the kernel's mean duration, timed with HIP events recorded on
  the stream the library launches it on.  ``traffic`` = HBM bytes per launch from the
  committed hardware-counter summary of the same kernel and workload (profiles/), or
  null when the kernel's sources changed since those counters were taken.
* ``cpu_baseline``: the float64 CPU oracle on a bounded sample of the same workload.

``--pmc-summary FETCH_DIR WRITE_DIR`` instead digests two rocprofv3 ``--pmc`` runs of
this script (FETCH_SIZE, then WRITE_SIZE, both with ``--copy-probe-mib``) into the
markdown summary that ``traffic`` is read from.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "fp4_routed_expert_moe_amd", "csrc")

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0

# Sources each timed kernel is compiled from: a change to any of them voids its counters.
KERNEL_SOURCES = {
    "gemv_gateup": ("gemv.hip", "common.h"),
    "gemv_down": ("gemv.hip", "common.h"),
    "gemm_gateup": ("gemm.hip", "common.h"),
    "gemm_down": ("gemm.hip", "common.h"),
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default=None,
                   help="measure only this workload (default: decode_t8 as the headline, plus a 'workloads' "
                        "object with the other workloads, the expert-bank one included)")
    p.add_argument("--no-workloads", action="store_true", help="headline only")
    p.add_argument("--mfma-summary", metavar="DIR", help="summarise a rocprofv3 --pmc run of MFMA counters")
    p.add_argument("--stats-summary", metavar="DIR", help="summarise a rocprofv3 --kernel-trace --stats run")
    p.add_argument("--layers", type=int, default=16, help="independent weight sets rotated per step")
    p.add_argument("--batches", type=int, default=64)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="the CPU oracle runs batches of the workload until this much time is spent")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="run one plain device copy of this many MiB before the steps (a known-size "
                        "reference for hardware byte counters)")
    p.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="summarise two rocprofv3 --pmc runs of this script instead of benchmarking")
    p.add_argument("--pmc-log", help="the stdout of the FETCH_SIZE run (its JSON line)")
    p.add_argument("--pmc-command", default="", help="command line recorded in the summary")
    return p.parse_args()


def expert_bytes(wl):
    """Bytes of one FP4 expert: (whole expert, gate+up, down)."""
    h, i = wl.hidden, wl.inter
    per_matrix = i * h // 2 + i * h // 32
    return 3 * per_matrix, 2 * per_matrix, per_matrix


def shared_bytes(wl):
    """Bytes of the shared expert in its stored format: (whole expert, gate+up, down)."""
    if not wl.shared:
        return 0, 0, 0
    if not wl.shared_fp8:
        return expert_bytes(wl)
    h, i = wl.hidden, wl.inter
    per_matrix = i * h + 4 * (-(-i // 128)) * (-(-h // 128))   # e4m3 codes + float32 block scales
    return 3 * per_matrix, 2 * per_matrix, per_matrix


def sources_digest(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, ()):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def traffic_record(kernel, workload):
    """HBM bytes per launch of `kernel` at `workload` from the committed counter summary, or
    None if there is none or the kernel's sources changed since it was taken."""
    for path in sorted(glob.glob(os.path.join(PROFILES, "*hbm_traffic*.md"))):
        with open(path) as f:
            m = re.search(r"```json\n(.*?)\n```", f.read(), re.S)
        if not m:
            continue
        rec = json.loads(m.group(1))
        if rec.get("workload") != workload:
            continue
        k = rec.get("kernels", {}).get(kernel)
        if k and k.get("sources") == sources_digest(kernel):
            return k["traffic_bytes_per_launch"]
    return None


EXTRA_WORKLOADS = ("decode_t8_fp8shared", "prefill_t512", "prefill_t4096_zipf", "stacked_decode_16l",
                   "chained_decode_16l", "decode_pro_t8", "prefill_pro_t512")
# per extra workload: (steps, warm-up steps, weight sets rotated, token batches rotated).  A
# prefill call's 3.4 GB of weights is far beyond the 256 MB last-level cache, so two weight sets
# and four token batches suffice there; the stacked workload is 16 layers by definition.
EXTRA_SHAPE = {"decode_t8_fp8shared": (200, 20, 16, 64), "prefill_t512": (50, 5, 2, 4),
               "prefill_t4096_zipf": (50, 5, 2, 4), "stacked_decode_16l": (100, 10, 16, 64),
               "chained_decode_16l": (100, 10, 16, 64),
               # V4 Pro scale: 8.9 GB of experts per layer, so six weight sets (53 GB) for decode
               "decode_pro_t8": (200, 20, 6, 64), "prefill_pro_t512": (50, 5, 2, 4)}


# Partial-residency expert bank workloads: the named layer workload with its experts in pinned host
# memory, served through an HBM bank of n_slots expert slots refilled `group` experts at a time.
# name -> (layer workload, steps, warm-up steps, n_slots, group, token batches rotated)
BANK_WORKLOADS = {"prefill_t512_bank64": ("prefill_t512", 10, 2, 64, 16, 4)}
PCIE_PEAK_GBPS = 64.0   # PCIe 5.0 x16, one direction (the MI355X host link)


def progress(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.pmc_summary:
        return pmc_summary(args)
    if args.mfma_summary:
        return mfma_summary(args)
    if args.stats_summary:
        return stats_summary(args)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the library has no "
              "multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch

    import moe_synth as synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload in BANK_WORKLOADS:
        print(json.dumps(measure_bank(args.workload)), flush=True)
        return
    headline = args.workload or "decode_t8"
    wl = synth.WORKLOADS[headline]
    res = measure(wl, args.steps, args.warmup, args.layers, args.batches, args.copy_probe_mib)
    extra = {}
    if args.workload is None and not args.no_workloads:
        for name in EXTRA_WORKLOADS:
            steps, warm, nl, nb = EXTRA_SHAPE[name]
            r = measure(synth.WORKLOADS[name], steps, warm, nl, nb, 0)
            extra[name] = {k: r[k] for k in ("value", "unit", "ms_per_step", "step_us_events", "steps", "warmup",
                                             "config",
                                             "weight_GBps", "weight_frac_hbm", "tflops",
                                             "tflops_frac_bf16", "active_groups_per_call", "layer_calls_per_step",
                                             "roofline", "kernels")}
        for name in BANK_WORKLOADS:
            extra[name] = measure_bank(name)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args, synth)
        progress("cpu baseline done")
    out = {
        "metric": "MoE layer tokens/s; decode FP4 weight GB/s & prefill TFLOPS vs MI355X peak",
        "value": res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16xfp4->fp32",
        "dtype_note": ("x bf16 enters the block-scaled matrix cores exactly, as two e4m3 terms; weights e2m1 "
                       "codes with e8m0 scales as stored; fp32 accumulation and output; SwiGLU h carried as three "
                       "e4m3 terms (12 bits) in decode, two (8 bits, bf16's precision) in prefill"),
        "data": "synthetic (seeded; random-init weights at the workload's DeepSeek V4 expert shapes)",
    }
    out.update({k: res[k] for k in ("step_us_events", "config", "weight_GBps", "weight_frac_hbm", "tflops",
                                    "tflops_frac_bf16",
                                    "active_groups_per_call", "layer_calls_per_step", "roofline", "kernels")})
    out["cpu_baseline"] = cpu
    if extra:
        out["workloads"] = extra
    if args.copy_probe_mib:
        out["copy_probe_mib"] = args.copy_probe_mib
    print(json.dumps(out), flush=True)


def measure(wl, steps, warmup, layers_rotated, batches, copy_probe_mib):
    """Time `steps` steps of one workload (after `warmup` untimed ones) and its kernels."""
    import numpy as np
    import torch

    import moe_synth as synth
    import fp4_routed_expert_moe_amd as moe

    dev = torch.device("cuda:0")
    nl = max(1, min(layers_rotated, wl.layers if wl.layers > 1 else layers_rotated))
    layers, keep = [], []
    for l in range(nl):
        raw = synth.layer_weights(wl, l, device=dev)          # checkpoint layout
        w = {m: moe.pack_fp4(*raw[m]) for m in synth.MATRICES}  # kernel layout, packed once
        del raw
        f8 = None
        if wl.shared_fp8:
            f8 = {}
            for m, (c, sc) in synth.shared_fp8_weights(wl, l, device=dev).items():
                f8[m] = (moe.pack_fp8(c[None])[0], sc)
        wr = torch.from_numpy(synth.router_weights(wl, l)).to(dev)
        b = synth.router_bias(wl)
        bt = None if b is None else torch.from_numpy(b).to(dev)
        layers.append(moe.MoeLayer(wr, w["gate"], w["up"], w["down"], wl.top_k, wl.shared, bt, shared_fp8=f8))
        keep.append((w, f8, wr, bt))
    torch.cuda.synchronize()
    progress(f"{wl.name}: {nl} weight set(s) resident")
    nb = batches
    xs = torch.stack([torch.from_numpy(synth.tokens(wl, layer=0, step=s).view(np.int16)) for s in range(nb)]).to(dev)
    T = wl.tokens
    ws = layers[0].workspace(T)
    y = torch.empty((T, wl.hidden), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    # A step is one pass of the layer.  Stacked decode runs its L layers one after another per step
    # (call i of the run uses layer i % nl and token batch i % nb); chained decode runs them as one
    # token's residual stream (RMSNorm between layers), from residual input h_0 = batch s % nb.
    # Both replay the step from a HIP graph the library records (moe_chain_*): one launch per step.
    # The per-kernel event timing pass runs the same kernels from eager calls (the graph carries
    # no timing events).
    L = wl.layers if wl.layers > 1 else 1
    chains, hs, gammas = [], None, None
    if wl.chained:
        hs = torch.stack([torch.from_numpy(synth.residual_input(wl, step=s)) for s in range(nb)]).to(dev)
        gammas = [torch.from_numpy(synth.norm_weight(wl, l)).to(dev) for l in range(nl)]
        chains.append(moe.MoeChain(layers, T, residual=True, norm_weight=gammas))
    elif L > 1:
        period_steps = int(np.lcm(nl, nb)) // L if int(np.lcm(nl, nb)) % L == 0 else None
        if period_steps is None or nl != L:
            raise ValueError("stacked decode: the layer/batch rotation must repeat after whole steps")
        for p in range(period_steps):
            ch = moe.MoeChain(layers, T, residual=False)
            for l in range(L):
                ch.x[l].copy_(xs[(p * L + l) % nb])
            chains.append(ch)
        torch.cuda.synchronize()

    def step(s):
        if wl.chained:
            chains[0].h_in.copy_(hs[s % nb])
            chains[0].run(torch.cuda.current_stream())
        elif chains:
            chains[s % len(chains)].run(torch.cuda.current_stream())
        else:
            layers[s % nl].forward(xs[s % nb], workspace=ws, y=y)

    ye = torch.empty((L, T, wl.hidden), dtype=torch.float32, device=dev)
    xe = torch.empty((L, T, wl.hidden), dtype=torch.int16, device=dev)
    he = torch.empty((T, wl.hidden), dtype=torch.float32, device=dev)

    def eager_step(s):
        """The step's kernels from eager library calls (for the per-kernel event timing)."""
        if not wl.chained:
            for c in range(s * L, (s + 1) * L):
                layers[c % nl].forward(xs[c % nb], workspace=ws, y=y)
            return
        h0 = hs[s % nb]
        for l in range(L):
            if l == 0:
                moe.residual_rmsnorm(h0, None, None, gammas[0], 1e-6, xe[0])
            else:
                moe.residual_rmsnorm(h0 if l == 1 else he, ye[l - 1], he, gammas[l], 1e-6, xe[l])
            layers[l].forward(xe[l], workspace=ws, y=ye[l])
        moe.residual_rmsnorm(h0 if L == 1 else he, ye[L - 1], he, None, 1e-6, None)

    if copy_probe_mib:
        src = torch.empty(copy_probe_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # active experts of every (layer, batch) pair a step can meet (outside the timed region)
    period = int(np.lcm(nl, nb))
    active = {}
    if wl.chained:
        # the layers' inputs come from the chain itself: route what an eager pass computes
        for b in range(min(nb, steps)):
            eager_step(b)
            for l in range(L):
                r = layers[l].route(xe[l], workspace=ws)
                active[(l, b)] = r["counts"]
    else:
        for c in range(min(period, steps * L)):
            r = layers[c % nl].route(xs[c % nb], workspace=ws)
            active[(c % nl, c % nb)] = r["counts"]
    torch.cuda.synchronize()
    active = {k: int((v > 0).sum().item()) for k, v in active.items()}

    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        step(s)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / steps
    tokens_per_s = steps * T / elapsed
    progress(f"{wl.name}: {steps} timed steps, {ms_per_step:.4f} ms per step")

    # the spread of single steps: HIP events around each of up to 100 more steps on the launch
    # stream (outside the timed region above)
    n_ev = min(steps, 100)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    for i, (e0, e1) in enumerate(evs):
        e0.record()
        step(steps + i)
        e1.record()
    torch.cuda.synchronize()
    step_us = np.array([1e3 * e0.elapsed_time(e1) for e0, e1 in evs])
    step_pct = {"p10": float(np.percentile(step_us, 10)), "p50": float(np.percentile(step_us, 50)),
                "p90": float(np.percentile(step_us, 90)), "steps": n_ev}

    # per-kernel HIP-event timing over a second pass of the same steps
    moe.timing_reset()
    moe.timing_enable(True)
    for s in range(steps):
        eager_step(s)
    torch.cuda.synchronize()
    kt = moe.timing_read()
    moe.timing_enable(False)

    e_all, e_gu, e_dn = expert_bytes(wl)
    s_all, s_gu, s_dn = shared_bytes(wl)
    if wl.chained:
        routed_per_call = [active[(l, s % nb)] for s in range(steps) for l in range(L)]
    else:
        routed_per_call = [active[(c % nl, c % nb)] for c in range(steps * L)]
    routed = float(np.mean(routed_per_call))
    groups = routed + wl.shared
    weight_bytes_step = L * (routed * e_all + s_all)   # weight bytes of the active groups
    flops_step = L * 2.0 * T * (wl.top_k + wl.shared) * 3 * wl.hidden * wl.inter
    # the dominant kernel and its algorithmic work per launch
    # (gate/up weight bytes of the groups it reads; gate/up flops).  The grouped GEMM is priced
    # against the roof its arithmetic intensity reaches first: MFMA above the ridge
    # (bf16 peak / HBM peak flop per byte), HBM below it.  The decode gate/up launch reads the
    # shared expert in either format (an FP8 one as extra tiles of the same launch); the grouped
    # GEMM gives an FP8 shared expert launches of its own.
    gu_bytes = routed * e_gu + s_gu
    gu_bytes_gemm = routed * e_gu + (0 if wl.shared_fp8 else s_gu)
    gu_flops = 2.0 * T * (wl.top_k + (0 if wl.shared_fp8 else wl.shared)) * 2 * wl.hidden * wl.inter
    if "gemv_gateup" in kt:
        dom, work, bound = "gemv_gateup", gu_bytes, "hbm"
    elif gu_flops / gu_bytes_gemm >= BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9):
        dom, work, bound = "gemm_gateup", gu_flops, "mfma"
    else:
        dom, work, bound = "gemm_gateup", gu_bytes_gemm, "hbm"
    launches, total_ms = kt.get(dom, (0, 0.0))
    avg_s = total_ms * 1e-3 / launches if launches else float("nan")
    if bound == "hbm":
        roof = dict(bound="hbm", achieved=work / avg_s / 1e9, peak=HBM_PEAK_GBPS, unit="GB/s")
    else:
        roof = dict(bound="mfma", achieved=work / avg_s / 1e12, peak=BF16_PEAK_TFLOPS, unit="TFLOP/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic_record(dom, wl.name)
    roof["kernel"] = dom
    roof["avg_launch_us"] = avg_s * 1e6
    roof["algorithmic_per_launch"] = work
    roof["algorithmic_unit"] = "bytes" if bound == "hbm" else "flops"
    roof["algorithmic_bytes_per_launch"] = gu_bytes if dom == "gemv_gateup" else gu_bytes_gemm
    kernels = {k: dict(launches=v[0], avg_us=1e3 * v[1] / max(v[0], 1)) for k, v in kt.items()}
    res = {
        "value": tokens_per_s, "unit": "tokens/s", "ms_per_step": ms_per_step, "steps": steps, "warmup": warmup,
        "step_us_events": step_pct,
        "config": {"workload": wl.name, "hidden": wl.hidden, "experts": wl.experts, "top_k": wl.top_k,
                   "shared": wl.shared, "shared_format": "fp8_e4m3_128x128" if wl.shared_fp8 else "fp4_e2m1_e8m0_32",
                   "inter": wl.inter, "tokens": T, "layers_rotated": nl,
                   "batches_rotated": nb, "parallelism": "single GPU",
                   "launch": "hip_graph_per_step" if chains else "eager_per_call",
                   **({"join": "residual + RMSNorm (eps 1e-6) between layers"} if wl.chained else {})},
        "weight_GBps": weight_bytes_step / (ms_per_step * 1e-3) / 1e9,
        "weight_frac_hbm": weight_bytes_step / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "tflops": flops_step / (ms_per_step * 1e-3) / 1e12,
        "tflops_frac_bf16": flops_step / (ms_per_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "active_groups_per_call": groups,
        "layer_calls_per_step": L,
        "roofline": roof,
        "kernels": kernels,
    }
    for ch in chains:
        ch.close()
    del layers, keep, xs, ws, y, chains
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def measure_bank(name):
    """Time whole layer calls served through a partial-residency expert bank (uploads included)."""
    import numpy as np
    import torch

    import moe_synth as synth
    import fp4_routed_expert_moe_amd as moe

    base, steps, warmup, n_slots, group, nb = BANK_WORKLOADS[name]
    wl = synth.WORKLOADS[base]
    dev = torch.device("cuda:0")
    raw = synth.layer_weights(wl, 0, device=dev)
    host = {}
    for m in synth.MATRICES:
        c, sc = moe.pack_fp4(*raw[m])
        hc = torch.empty(c.shape, dtype=torch.uint8, pin_memory=True)
        hs = torch.empty(sc.shape, dtype=torch.uint8, pin_memory=True)
        hc.copy_(c)
        hs.copy_(sc)
        host[m] = (hc, hs)
    torch.cuda.synchronize()
    del raw, c, sc
    torch.cuda.empty_cache()
    wr = torch.from_numpy(synth.router_weights(wl, 0)).to(dev)
    b = synth.router_bias(wl)
    bt = None if b is None else torch.from_numpy(b).to(dev)
    layer = moe.MoeLayer(wr, host["gate"], host["up"], host["down"], wl.top_k, wl.shared, bt, "gemm",
                         host_weights=True)
    bank = moe.MoeBank(layer, n_slots, group)
    xs = torch.stack([torch.from_numpy(synth.tokens(wl, layer=0, step=s).view(np.int16)) for s in range(nb)]).to(dev)
    T = wl.tokens
    ws = layer.workspace(T)
    y = torch.empty((T, wl.hidden), dtype=torch.float32, device=dev)
    progress(f"{name}: {sum(t.numel() for p in host.values() for t in p) / 1e9:.2f} GB of experts in pinned host "
             f"memory, bank of {n_slots} slots")
    for s in range(warmup):
        bank.forward(xs[s % nb], workspace=ws, y=y)
    torch.cuda.synchronize()
    st0 = bank.stats()
    t0 = time.perf_counter()
    for s in range(steps):
        bank.forward(xs[s % nb], workspace=ws, y=y)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    st1 = bank.stats()
    up_bytes = st1["bytes_uploaded"] - st0["bytes_uploaded"]
    ms = 1e3 * elapsed / steps
    progress(f"{name}: {steps} timed steps, {ms:.3f} ms per step")
    res = {"value": steps * T / elapsed, "unit": "tokens/s", "ms_per_step": ms, "steps": steps, "warmup": warmup,
           "config": {"workload": name, "layer_workload": base, "tokens": T, "bank_slots": n_slots,
                      "refill_group": group, "expert_bytes_host": sum(t.numel() for p in host.values() for t in p),
                      "bank_bytes": n_slots * sum(t[0].numel() for p in host.values() for t in p),
                      "launch": "moe_bank_forward per call (blocks on the routing counts)"},
           "h2d_GBps": up_bytes / elapsed / 1e9, "h2d_frac_pcie": up_bytes / elapsed / 1e9 / PCIE_PEAK_GBPS,
           "uploads_per_call": (st1["uploads"] - st0["uploads"]) / steps,
           "resident_hits_per_call": (st1["resident_hits"] - st0["resident_hits"]) / steps,
           "refill_groups_per_call": (st1["refill_groups"] - st0["refill_groups"]) / steps,
           "bound": "pcie (uploads of the experts not resident)"}
    bank.close()
    del layer, host, xs, ws, y
    torch.cuda.synchronize()
    return res


def _cpu_batch(wl, b, synth):
    """Token batch `b` of the workload (layer 0) and the expert weights its routing needs."""
    import oracle
    t_batch = min(wl.tokens, 8)
    wr = synth.router_weights(wl, 0)
    bias = synth.router_bias(wl)
    x = synth.tokens(wl, layer=0, step=b)[:t_batch]
    idx, _, _ = oracle.select_experts(oracle.router_logits(x, wr, bias), wl.top_k)
    needed = sorted(set(idx.reshape(-1).tolist()) | ({wl.experts} if wl.shared else set()))
    lazy = synth.LazyExperts(wl, 0, cache=len(needed) + 1)
    return x, wr, bias, {g: lazy[g] for g in needed}


class _Pre:
    def __init__(self, experts):
        self.experts = experts

    def __getitem__(self, g):
        return self.experts[g]


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits
    import torch
    threadpool_limits(1)
    torch.set_num_threads(1)


def _cpu_job(wl, b):
    """One all-cores oracle job: prepare batch b's weights (untimed), run the oracle on it with
    one numpy thread; returns (tokens, start, end) of the oracle run."""
    import moe_synth as synth
    import oracle
    x, wr, bias, experts = _cpu_batch(wl, b, synth)
    t0 = time.time()
    oracle.moe_forward(x, wr, bias, _Pre(experts), wl.top_k, wl.shared)
    return x.shape[0], t0, time.time()


def cpu_baseline(wl, args, synth):
    """The float64 CPU oracle on whole batches of the same workload (layer 0, 8 tokens each).

    One thread: batches one after another until half of ``--cpu-seconds`` of oracle time is
    spent.  All cores: one worker process per core of this process's CPU set (at most 16, the
    host share of one GPU), each running the oracle on its own batches with one numpy thread,
    timed from the first oracle start to the last oracle end.  Weight generation is outside
    both timed regions."""
    import multiprocessing

    from threadpoolctl import threadpool_limits

    import oracle

    total_t, total_s, batches = 0, 0.0, 0
    while batches < 16 and (batches == 0 or total_s < args.cpu_seconds / 2):
        x, wr, bias, experts = _cpu_batch(wl, batches, synth)
        with threadpool_limits(limits=1):          # the oracle as it stands: numpy, one thread
            t0 = time.perf_counter()
            oracle.moe_forward(x, wr, bias, _Pre(experts), wl.top_k, wl.shared)
            total_s += time.perf_counter() - t0
        total_t += x.shape[0]
        batches += 1
    one = total_t / total_s
    per_batch_s = total_s / batches
    progress(f"cpu baseline: one thread {one:.3g} tokens/s over {batches} batch(es)")

    affinity = len(os.sched_getaffinity(0))
    workers = max(1, min(16, affinity))
    # batches per worker so the parallel phase lasts about half of --cpu-seconds
    per_worker = max(1, min(8, int(round(args.cpu_seconds / 2 / per_batch_s))))
    import concurrent.futures
    res = []
    with concurrent.futures.ProcessPoolExecutor(workers, initializer=_cpu_worker_init,
                                                mp_context=multiprocessing.get_context("spawn")) as pool:
        futs = [pool.submit(_cpu_job, wl, 100 + j) for j in range(workers * per_worker)]
        for f in concurrent.futures.as_completed(futs, timeout=300):
            res.append(f.result())
            progress(f"cpu baseline: {len(res)} of {len(futs)} all-cores batches done")
    toks = sum(r[0] for r in res)
    wall = max(r[2] for r in res) - min(r[1] for r in res)
    L = wl.layers if wl.layers > 1 else 1  # a token of the stacked workload passes L layers
    per_layer = f"; a token passes {L} layers of the same cost" if L > 1 else ""
    return {"value": toks / wall / L, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": (f"{workers} worker processes, {per_worker} batch(es) each, of {min(wl.tokens, 8)} tokens of "
                       f"{wl.name} layer 0, one numpy thread each, {wall:.1f} s wall{per_layer}"),
            "host_cpus_in_affinity": affinity,
            "single_thread": {"value": one / L, "unit": "tokens/s", "cores": 1,
                              "sample": f"{batches} batch(es) one after another, {total_s:.1f} s of oracle time"}}


# ---------------------------------------------------------------------------------------
# Hardware-counter summary (FETCH_SIZE / WRITE_SIZE per dispatch, calibrated on a copy)
# ---------------------------------------------------------------------------------------

def _short_name(full):
    """Kernel symbol -> the name its launches are timed under (the grouped GEMM template is
    one symbol for gate/up and down)."""
    m = re.match(r"(?:void )?moe::(\w+?)(?:_kernel)?\b(<\w+)?", full)
    if not m:
        return None
    if m.group(1) == "gemm_f8f4":
        return "gemm_gateup" if m.group(2) == "<true" else "gemm_down"
    return m.group(1)


def _read_pmc(directory):
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def pmc_summary(args):
    fetch = _read_pmc(args.pmc_summary[0])
    write = _read_pmc(args.pmc_summary[1])
    run = {}
    if args.pmc_log:
        with open(args.pmc_log) as f:
            for line in f:
                if line.startswith("{"):
                    run = json.loads(line)
    probe = (run.get("copy_probe_mib") or 512) << 20

    def calib(rows):
        # the copy probe is the largest plain device copy of the run
        cp = [float(r["Counter_Value"]) for r in rows if r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer")]
        return probe / (max(cp) * 1024.0)

    ff, fw = calib(fetch), calib(write)

    def per_kernel(rows):
        acc = {}
        for r in rows:
            n = _short_name(r["Kernel_Name"])
            if n:
                acc.setdefault(n, []).append(float(r["Counter_Value"]))
        return acc

    kf, kw = per_kernel(fetch), per_kernel(write)
    wl = run.get("config", {}).get("workload", "decode_t8")
    roof = run.get("roofline", {})
    kernels = {}
    lines = []
    for n in sorted(kf):
        f_kib = sum(kf[n]) / len(kf[n])
        w_kib = sum(kw.get(n, [0.0])) / max(len(kw.get(n, [])), 1)
        tb = (f_kib * ff + w_kib * fw) * 1024.0
        rec = {"dispatches": len(kf[n]), "fetch_kib": f_kib, "write_kib": w_kib, "traffic_bytes_per_launch": tb}
        if n in KERNEL_SOURCES:
            rec["sources"] = sources_digest(n)
        if n == roof.get("kernel"):
            rec["algorithmic_bytes_per_launch"] = roof.get("algorithmic_bytes_per_launch",
                                                          roof.get("algorithmic_per_launch"))
        kernels[n] = rec
        alg = rec.get("algorithmic_bytes_per_launch")
        ratio = f"{tb / alg:.3f}" if alg else "-"
        lines.append(f"| {n} | {len(kf[n])} | {f_kib:,.0f} | {w_kib:,.0f} | {tb / 1e6:,.1f} | {ratio} |")
    rec = {"workload": wl, "fetch_factor": ff, "write_factor": fw, "kernels": kernels}
    print(f"# HBM traffic per dispatch: {wl}\n")
    print("Commands (repository root on the GPU box, `cd /tmp && export TMPDIR=/tmp` first):\n")
    print("```\n" + (args.pmc_command or "(not recorded)") + "\n```\n")
    print(f"Calibration: a {probe >> 20} MiB device copy (`__amd_rocclr_copyBuffer`) reads "
          f"FETCH_SIZE x {ff:.3f} and WRITE_SIZE x {fw:.3f} of its true byte counts; those factors scale "
          "every kernel's counters below.\n")
    print("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | traffic MB / launch | traffic / algorithmic |")
    print("|---|---|---|---|---|---|")
    print("\n".join(lines))
    print("\n`sources` is a digest of the files the kernel is built from; `bench.py` reports `traffic` only "
          "while it matches.\n")
    print("```json\n" + json.dumps(rec, indent=None) + "\n```")


def mfma_summary(args):
    """Per-kernel means of an MFMA counter pass (MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES over
    GRBM_GUI_ACTIVE x SIMDs, and the F8 / F6F4 MFMA op counts, 512 flops each) as markdown."""
    rows = _read_pmc(args.mfma_summary)
    run = {}
    if args.pmc_log:
        with open(args.pmc_log) as f:
            for line in f:
                if line.startswith("{"):
                    run = json.loads(line)
    acc = {}
    for r in rows:
        n = _short_name(r["Kernel_Name"])
        if n:
            acc.setdefault(n, {}).setdefault(r.get("Counter_Name", "value"), []).append(float(r["Counter_Value"]))
    cfg = run.get("config", {})
    wl = cfg.get("workload", "?")
    print(f"# MFMA counters per dispatch: {wl}\n")
    print("Command (repository root on the GPU box, `cd /tmp && export TMPDIR=/tmp` first):\n")
    print("```\n" + (args.pmc_command or "(not recorded)") + "\n```\n")
    print("| kernel | dispatches | MfmaUtil % | F8 MFMA flops (x512 ops) | F6F4 MFMA flops | "
          "algorithmic flops / launch |")
    print("|---|---|---|---|---|---|")
    recs = {}
    t, kk, ss, h, i = (cfg.get(k, 0) for k in ("tokens", "top_k", "shared", "hidden", "inter"))
    alg = {"gemm_gateup": 2.0 * t * (kk + ss) * 2 * h * i, "gemm_down": 2.0 * t * (kk + ss) * h * i}
    for n in sorted(acc):
        c = acc[n]
        mean = {k: sum(v) / len(v) for k, v in c.items()}
        nd = max(len(v) for v in c.values())
        util = mean.get("MfmaUtil")
        f8 = mean.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0) * 512
        f6 = mean.get("SQ_INSTS_VALU_MFMA_MOPS_F6F4", 0.0) * 512
        recs[n] = {"dispatches": nd, "mfma_util_pct": util, "f8_flops": f8, "f6f4_flops": f6,
                   "algorithmic_flops": alg.get(n)}
        print(f"| {n} | {nd} | {util if util is None else f'{util:.1f}'} | {f8:.4g} | {f6:.4g} | "
              f"{alg.get(n, float('nan')):.4g} |")
    print("\n```json\n" + json.dumps({"workload": wl, "kernels": recs}) + "\n```")


def stats_summary(args):
    """The library's kernels from a rocprofv3 --kernel-trace --stats run (k_kernel_stats.csv), and
    the run's own JSON line, as markdown."""
    files = glob.glob(os.path.join(args.stats_summary, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {args.stats_summary}")
    run = {}
    if args.pmc_log:
        with open(args.pmc_log) as f:
            for line in f:
                if line.startswith("{"):
                    run = json.loads(line)
    cfg = run.get("config", {})
    print(f"# rocprofv3 kernel stats: {cfg.get('workload', '?')}\n")
    print("Command (`cd /tmp && export TMPDIR=/tmp` first):\n")
    print("```\n" + (args.pmc_command or "(not recorded)") + "\n```\n")
    print("| kernel | calls | average (us) | min (us) | max (us) | total (ms) |")
    print("|---|---|---|---|---|---|")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += [r for r in csv.DictReader(fh)
                     if r["Name"].replace("(anonymous namespace)::", "").split("(")[0].split("<")[0].strip().split()[-1]
                     .startswith("moe::")]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").replace("moe::", "")
        print(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
              f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['TotalDurationNs']) / 1e6:.2f} |")
    if run:
        keep = {k: run.get(k) for k in ("value", "unit", "ms_per_step", "steps", "warmup")}
        keep["kernels_event_timed"] = run.get("kernels")
        print("\nThe run's own line (steps timed without the profiler's per-dispatch records are faster):\n")
        print("```json\n" + json.dumps(keep) + "\n```")


if __name__ == "__main__":
    main()
