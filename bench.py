#!/usr/bin/env python3
"""Throughput of the routed FP4-expert MoE layer on one MI355X.

A step is one full layer call (router, top-k, grouping, gate/up with FP4 dequant and
SwiGLU, down projection, shared expert, combine) on one batch of synthetic tokens.
Default workload: the decode batch at DeepSeek V4 Flash expert shapes (H=4096, E=256,
top-6, 1 shared expert, I=2048, 8 tokens).  Steps rotate over 16 independent layers'
weights (55 GB resident) and 64 token batches, so no layer's weights are still in the
256 MB last-level cache when it runs again.

Prints one JSON line (rank 0).  Also reports the dominant kernel against its roofline
(HIP-event timing of every launch inside the library, on the launching stream) and the
CPU oracle's throughput on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode_t8")
    p.add_argument("--layers", type=int, default=16, help="independent weight sets rotated per step")
    p.add_argument("--batches", type=int, default=64)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=0, help="0 = one batch (capped at 8 tokens)")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="run one plain device copy of this many MiB before the steps (a known-size "
                        "reference for hardware byte counters)")
    return p.parse_args()


def expert_bytes(wl):
    h, i = wl.hidden, wl.inter
    per_matrix = i * h // 2 + i * h // 32
    return 3 * per_matrix, 2 * per_matrix, per_matrix  # whole expert, gate+up, down


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this build has no "
              "multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import moe_synth as synth
    import fp4_routed_expert_moe_amd as moe

    wl = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nl = max(1, min(args.layers, wl.layers if wl.layers > 1 else args.layers))
    layers, keep = [], []
    for l in range(nl):
        raw = synth.layer_weights(wl, l, device=dev)          # checkpoint layout
        w = {m: moe.pack_fp4(*raw[m]) for m in synth.MATRICES}  # kernel layout, packed once
        del raw
        wr = torch.from_numpy(synth.router_weights(wl, l)).to(dev)
        b = synth.router_bias(wl)
        bt = None if b is None else torch.from_numpy(b).to(dev)
        layers.append(moe.MoeLayer(wr, w["gate"], w["up"], w["down"], wl.top_k, wl.shared, bt))
        keep.append((w, wr, bt))
    nb = args.batches
    xs = torch.stack([torch.from_numpy(synth.tokens(wl, layer=0, step=s).view(np.int16)) for s in range(nb)]).to(dev)
    T = wl.tokens
    ws = layers[0].workspace(T)
    y = torch.empty((T, wl.hidden), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(s):
        layers[s % nl].forward(xs[s % nb], workspace=ws, y=y)

    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # active experts of every (layer, batch) pair a step can meet (outside the timed region)
    period = int(np.lcm(nl, nb))
    active = {}
    for s in range(min(period, args.steps)):
        r = layers[s % nl].route(xs[s % nb], workspace=ws)
        active[(s % nl, s % nb)] = r["counts"]
    torch.cuda.synchronize()
    active = {k: int((v > 0).sum().item()) for k, v in active.items()}

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(s)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    tokens_per_s = args.steps * T / elapsed

    # per-kernel HIP-event timing over a second pass of the same steps
    moe.timing_reset()
    moe.timing_enable(True)
    for s in range(args.steps):
        step(s)
    torch.cuda.synchronize()
    kt = moe.timing_read()
    moe.timing_enable(False)

    e_all, e_gu, e_dn = expert_bytes(wl)
    groups_per_step = [active[(s % nl, s % nb)] + wl.shared for s in range(args.steps)]
    fp4_bytes_step = float(np.mean(groups_per_step)) * e_all
    flops_step = 2.0 * T * (wl.top_k + wl.shared) * 3 * wl.hidden * wl.inter
    gemv = "gemv_gateup" in kt
    dom = "gemv_gateup" if gemv else "gemm_gateup"
    launches, total_ms = kt.get(dom, (0, 0.0))
    avg_ms = total_ms / launches if launches else float("nan")
    if gemv:
        roof = dict(bound="hbm", achieved=float(np.mean(groups_per_step)) * e_gu / (avg_ms * 1e-3) / 1e9,
                    peak=HBM_PEAK_GBPS, unit="GB/s")
    else:
        fl = 2.0 * T * (wl.top_k + wl.shared) * 2 * wl.hidden * wl.inter
        roof = dict(bound="mfma", achieved=fl / (avg_ms * 1e-3) / 1e12, peak=BF16_PEAK_TFLOPS, unit="TFLOP/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = dom
    roof["avg_launch_us"] = avg_ms * 1e3
    roof["algorithmic_bytes_per_launch"] = float(np.mean(groups_per_step)) * e_gu if gemv else None

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args, synth)

    kernels = {k: dict(launches=v[0], avg_us=1e3 * v[1] / max(v[0], 1)) for k, v in kt.items()}
    out = {
        "metric": "MoE layer tokens/s; decode FP4 weight GB/s & prefill TFLOPS vs MI355X peak",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4(e2m1,e8m0/32) weights; bf16 activations; fp32 accumulate",
        "data": "synthetic (seeded; random-init weights at DeepSeek V4 Flash expert shapes)",
        "config": {"workload": wl.name, "hidden": wl.hidden, "experts": wl.experts, "top_k": wl.top_k,
                   "shared": wl.shared, "inter": wl.inter, "tokens": T, "layers_rotated": nl,
                   "batches_rotated": nb, "parallelism": "single GPU"},
        "fp4_weight_GBps": fp4_bytes_step / (ms_per_step * 1e-3) / 1e9,
        "fp4_weight_frac_hbm": fp4_bytes_step / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "tflops": flops_step / (ms_per_step * 1e-3) / 1e12,
        "active_groups_per_step": float(np.mean(groups_per_step)),
        "roofline": roof,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(wl, args, synth):
    """The float64 CPU oracle on one batch of the same workload (time excludes weight generation)."""
    import numpy as np

    import oracle

    t = args.cpu_sample_tokens or min(wl.tokens, 8)
    x = synth.tokens(wl, layer=0, step=0)[:t]
    wr = synth.router_weights(wl, 0)
    b = synth.router_bias(wl)
    idx, _, _ = oracle.select_experts(oracle.router_logits(x, wr, b), wl.top_k)
    needed = sorted(set(idx.reshape(-1).tolist()) | ({wl.experts} if wl.shared else set()))
    lazy = synth.LazyExperts(wl, 0, cache=len(needed) + 1)
    experts = {g: lazy[g] for g in needed}

    class Pre:
        def __getitem__(self, g):
            return experts[g]

    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):          # the oracle as it stands: numpy, one thread
        t0 = time.perf_counter()
        oracle.moe_forward(x, wr, b, Pre(), wl.top_k, wl.shared)
        dt = time.perf_counter() - t0
    cores = 1
    return {"value": t / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{t} tokens of {wl.name} layer 0 ({len(needed)} expert groups), {dt:.2f} s"}


if __name__ == "__main__":
    main()
