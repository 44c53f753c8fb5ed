#!/usr/bin/env python3
"""Benchmark of the MoE layer on one MI355X.

One step = one call of the whole layer (router, top-k, permutation, routed
SwiGLU experts, shared expert, combine) on one batch of seeded synthetic tokens,
inputs and weights already resident in HBM.  The headline workload is the
Ling-lite-shaped layer (hidden 2048, 64 experts top-6, moe_intermediate 1408,
shared width 2816, bf16) at T=4096 tokens; decode batches T=1 and T=64 of the
same layer are reported alongside.  Layer copies are rotated between steps so
that weight reads come from HBM, not from the 256 MB Infinity Cache.

Prints one JSON line (see the repository's design notes for every field).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
METRIC = "MoE-layer tokens/s at T=1/64/4096; achieved HBM GB/s & MFMA % of peak"


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="workload 1..5 (default 2: Ling-lite shape)")
    ap.add_argument("--tokens", type=int, default=4096, help="headline batch size T")
    ap.add_argument("--decode-tokens", default="1,64", help="extra decode batch sizes ('' = none)")
    ap.add_argument("--min-rotation-bytes", type=float, default=2e9,
                    help="rotate layer copies until this many weight bytes separate reuses")
    ap.add_argument("--max-copies", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=256)
    return ap.parse_args()


def gpu_copy(spec, c, ref, device):
    """Timing-only layer copy drawn on the GPU with the same distributions."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(7919 * (c + 1) + spec.seed_id)
    out = {}
    for name, t in ref.__dict__.items():
        if t is None:
            out[name] = None
        elif name in ("router_bias", "expert_bias"):
            out[name] = t                      # routing biases are shared by all copies
        elif t.dtype == torch.bfloat16 or t.dtype == torch.float32:
            out[name] = (torch.randn(t.shape, generator=g, device=device, dtype=torch.float32)
                         * spec.weight_std).to(t.dtype)
        elif t.dtype == torch.uint8:
            out[name] = torch.randint(0, 256, t.shape, generator=g, device=device,
                                      dtype=torch.int32).to(torch.uint8)
        else:                                   # fp16 scales / zero points
            out[name] = t.clone()
    return type(ref)(**out)


def algorithmic(spec, T, counts):
    """Bytes the layer must move and flops it must do for one call (routing of that call)."""
    import synth
    lb = synth.layer_bytes(spec)
    D = int((counts > 0).sum())
    k, H, I, Is, E = spec.top_k, spec.hidden, spec.moe_intermediate, spec.shared_intermediate, spec.num_experts
    byt = D * lb["expert"] + lb["shared"] + lb["router"] + T * H * 2 * lb["act"]
    byt += 4 * E if spec.use_expert_bias else 0
    flops = 2.0 * T * E * H + 6.0 * T * k * H * I + 6.0 * T * H * Is
    per_expert_up_bytes = lb["expert"] * 2 / 3
    up_bytes = D * per_expert_up_bytes + (2 * Is * H * lb["act"]) + T * H * lb["act"] + T * k * I * lb["act"]
    up_flops = 4.0 * T * k * H * I
    return dict(bytes=byt, flops=flops, D=D, up_bytes=up_bytes, up_flops=up_flops)


def run_case(moe, spec, cfg, copies, x, steps, warmup, stage_mask):
    """Time `steps` layer calls over rotating copies; returns (seconds, stage timings)."""
    import torch
    y = torch.empty_like(x)
    T = x.shape[0]
    ws = torch.empty(cfg.workspace_size(T), dtype=torch.uint8, device=x.device)
    L = len(copies)
    for i in range(warmup):
        moe.forward(x, copies[i % L], cfg, ws=ws, out=y)
    torch.cuda.synchronize()
    lib = moe.lib()
    from mixture_experts_layer_03_amd import _lib
    _lib.check(lib.moe_profile_enable(stage_mask, max(8, 8 * steps)))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        moe.forward(x, copies[i % L], cfg, ws=ws, out=y)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    import ctypes as C
    stages = {}
    for name, bit in _lib.STAGES.items():
        if stage_mask & bit:
            ms, n = C.c_float(0), C.c_int32(0)
            _lib.check(lib.moe_profile_collect(bit, C.byref(ms), C.byref(n)))
            if n.value:
                stages[name] = ms.value / n.value
    _lib.check(lib.moe_profile_disable())
    return t1 - t0, stages, y


def cpu_baseline(spec, L_host, x_host, n_tok):
    from dataclasses import fields
    import oracle.moe_oracle as om
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        cores = os.cpu_count() or 1
    tok = np.arange(min(n_tok, x_host.shape[0]))
    t0 = time.perf_counter()
    ocfg = om.OracleConfig(**{f.name: getattr(spec, f.name) for f in fields(om.OracleConfig)})
    om.forward(x_host, L_host, ocfg, tokens=tok)
    dt = time.perf_counter() - t0
    return dict(value=len(tok) / dt, unit="tokens/s", cores=int(cores), kind="oracle",
                sample=f"fp64 oracle, {len(tok)} tokens of the T={x_host.shape[0]} batch, "
                       f"same layer, {dt:.1f} s")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this layer build has no multi-GPU path "
              "(expert-parallel sharding is a design note only); use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import torch
    import synth
    import mixture_experts_layer_03_amd as moe

    spec = synth.SPECS[args.config]
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    L_host = synth.make_layer(spec)
    W0 = moe.weights_from_host(L_host, dev)
    gen_s = time.perf_counter() - t_gen
    lb = synth.layer_bytes(spec)
    layer_bytes = spec.num_experts * lb["expert"] + lb["shared"] + lb["router"]

    def copies_for(touched):
        n = int(np.ceil(args.min_rotation_bytes / max(touched, 1.0)))
        return max(1, min(args.max_copies, n))

    all_copies = [W0]

    def get_copies(n):
        while len(all_copies) < n:
            all_copies.append(gpu_copy(spec, len(all_copies), W0, dev))
        return all_copies[:n]

    cfg = moe.MoEConfig.from_object(spec)
    results = {}
    Ts = [args.tokens] + [int(t) for t in args.decode_tokens.split(",") if t.strip()]
    for T in Ts:
        x_host = synth.make_x(spec, T)
        x = moe.host_tensor_to_device(x_host, dev)
        _, (idx, wt, counts) = moe.forward(x, W0, cfg, return_routing=True)
        torch.cuda.synchronize()
        alg = algorithmic(spec, T, counts.cpu().numpy())
        ncp = copies_for(alg["bytes"])
        cps = get_copies(ncp)
        mask = moe._lib.STAGES["up"] | moe._lib.STAGES["down"]
        steps = args.steps if T == args.tokens else max(args.steps, 50)
        secs, stages, _ = run_case(moe, spec, cfg, cps, x, steps, args.warmup, mask)
        t_step = secs / steps
        results[T] = dict(T=T, copies=ncp, ms_per_step=t_step * 1e3, tokens_per_s=T / t_step,
                          hbm_gbps=alg["bytes"] / t_step / 1e9, mfma_tflops=alg["flops"] / t_step / 1e12,
                          distinct_experts=alg["D"], stage_ms=stages, alg=alg)
        results[T]["hbm_frac"] = results[T]["hbm_gbps"] / HBM_PEAK_GBPS
        results[T]["mfma_frac"] = results[T]["mfma_tflops"] / BF16_PEAK_TFLOPS
        results[T]["roofline_frac"] = max(alg["bytes"] / (HBM_PEAK_GBPS * 1e9),
                                          alg["flops"] / (BF16_PEAK_TFLOPS * 1e12)) / t_step
        if T == args.tokens:
            head_x_host = x_host

    head = results[args.tokens]
    alg = head["alg"]
    up_ms = head["stage_ms"].get("up")
    prefill = args.tokens > 64 and spec.act_dtype == "bf16"
    if up_ms:
        if prefill:
            ach = alg["up_flops"] / (up_ms * 1e-3) / 1e12
            roof = dict(bound="mfma", achieved=ach, peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                        frac=ach / BF16_PEAK_TFLOPS, traffic=None,
                        kernel="routed gate/up grouped GEMM + SwiGLU", avg_ms=up_ms)
        else:
            ach = alg["up_bytes"] / (up_ms * 1e-3) / 1e9
            roof = dict(bound="hbm", achieved=ach, peak=HBM_PEAK_GBPS, unit="GB/s",
                        frac=ach / HBM_PEAK_GBPS, traffic=None,
                        kernel="routed+shared gate/up weight streaming + SwiGLU", avg_ms=up_ms)
    else:
        roof = None

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(spec, L_host, head_x_host, args.cpu_sample_tokens)

    def brief(r):
        return {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items() if k != "alg"}

    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if spec.act_dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{spec.name} MoE layer: hidden {spec.hidden}, {spec.num_experts} experts "
                               f"top-{spec.top_k}, moe_intermediate {spec.moe_intermediate}, shared "
                               f"{spec.shared_intermediate}, {spec.score_function}, n_group {spec.n_group}, "
                               f"experts {spec.expert_dtype}; T={args.tokens}",
                   "tokens": args.tokens, "layer_gb": layer_bytes / 1e9},
        "roofline": roof,
        "cpu_baseline": cpu,
        "hbm_gbps": head["hbm_gbps"],
        "mfma_frac": head["mfma_frac"],
        "roofline_frac": head["roofline_frac"],
        "per_T": [brief(results[T]) for T in Ts],
        "gen_seconds": gen_s,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
