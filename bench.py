#!/usr/bin/env python3
"""Benchmark of the MoE layer on one MI355X.

One step = one call of the whole layer (router, top-k, permutation, routed
SwiGLU experts, shared expert, combine) on one batch of seeded synthetic tokens,
inputs and weights already resident in HBM.  The headline workload is the
Ling-lite-shaped layer (hidden 2048, 64 experts top-6, moe_intermediate 1408,
shared width 2816, bf16) at T=4096 tokens; decode batches T=1 and T=64 of the
same layer are reported alongside (eager calls and HIP-graph replays), and
per_config repeats the protocol for other workloads (by default the
Ling-2.6-flash-style layer at T=1/64/4096 and the u8 Ling-3.0-flash-style layer
at T=1/64).  Layer copies are rotated between steps so that weight reads come
from HBM, not from the 256 MB Infinity Cache.  Every batch also carries its
comparison with the fp64 oracle (routing-set mismatches, near-ties, max relative
error) and its p10/p50/p90 step times; the line carries the measured bandwidth of
a 1 GiB device copy.

Prints one JSON line (field meanings are in the repository's design notes).
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
METRIC = "MoE-layer tokens/s at T=1/64/4096; achieved HBM GB/s & MFMA % of peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
DENSE_STREAM_MAX_T = 192        # moe_dense_mlp streams up to this many tokens (include/moe.h)


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--spinup-ms", type=float, default=200.0,
                    help="untimed layer calls for this long before the warm-up steps of each batch size "
                         "(the GPU's clocks ramp over the first tens of ms of sustained load)")
    ap.add_argument("--config", type=int, default=2, help="workload 1..7 (default 2: Ling-lite shape)")
    ap.add_argument("--dense", action="store_true",
                    help="time the dense MLP in front of the MoE layers (Ling-2.6-flash layer 0: "
                         "hidden 4096, intermediate 9216) instead of a MoE workload")
    ap.add_argument("--tokens", type=int, default=4096, help="headline batch size T")
    ap.add_argument("--decode-tokens", default="1,64", help="extra decode batch sizes ('' = none)")
    ap.add_argument("--min-rotation-bytes", type=float, default=2e9,
                    help="rotate layer copies until this many weight bytes separate reuses")
    ap.add_argument("--max-copies", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a 1 GiB device copy under the profiler (reference kernel for counter scaling); "
                         "the copy's bandwidth is measured and reported in every run")
    ap.add_argument("--per-config", default="3:1,64,4096;5:1,64",
                    help="extra workloads reported in per_config, 'cfg:T,T;cfg:T' ('' = none)")
    ap.add_argument("--parity-tokens", type=int, default=256,
                    help="tokens of a batch above 64 tokens compared with the oracle (seeded sample; "
                         "batches up to 64 tokens are compared on every token)")
    ap.add_argument("--no-parity", action="store_true", help="skip the oracle comparison of each batch")
    return ap.parse_args()


def source_digest() -> str:
    """Hash of the kernel sources (counter results are valid only for this exact code)."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "mixture_experts_layer_03_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


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
    # dominant kernel (routed + shared gate/up): weights of the D experts (and, on the
    # streaming path, the shared gate/up), token rows in, SwiGLU rows out
    up_bytes = D * lb["expert"] * 2 / 3 + T * H * lb["act"] + T * k * I * lb["act"]
    up_bytes_decode = up_bytes + 2 * Is * H * lb["act"] + T * Is * lb["act"]
    up_flops = 4.0 * T * k * H * I
    return dict(bytes=byt, flops=flops, D=D, up_bytes=up_bytes, up_bytes_decode=up_bytes_decode,
                up_flops=up_flops)


def stage_times(moe, stage_mask):
    from mixture_experts_layer_03_amd import _lib
    lib = moe.lib()
    out = {}
    for name, bit in _lib.STAGES.items():
        if stage_mask & bit:
            ms, n = C.c_float(0), C.c_int32(0)
            _lib.check(lib.moe_profile_collect(bit, C.byref(ms), C.byref(n)))
            if n.value:
                out[name] = ms.value / n.value
    return out


def spin_up(call, ms):
    """Untimed calls for `ms` milliseconds of wall time, four per synchronisation.

    Measured on the MI355X (Ling-lite layer, 4096 tokens, kernel trace): the routed
    gate/up kernel took 430-460 us in the first ten calls of a run, 380 us after 30 and
    370 us after 70, and the timed step fell from 0.800 ms after 5 warm-up steps to
    0.758 ms after 50 or 100: the clocks ramp over the first tens of milliseconds of
    sustained load, so a timed loop that starts earlier measures the ramp."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(4):
            call(i)
            i += 1
        torch.cuda.synchronize()


def run_eager(moe, cfg, copies, x, steps, warmup, stage_mask, spinup_ms=0.0):
    """Time `steps` layer calls over rotating copies; then the same calls again with
    per-stage HIP events (kept out of the timed loop: recording them costs time)."""
    import torch
    from mixture_experts_layer_03_amd import _lib
    y = torch.empty_like(x)
    T = x.shape[0]
    ws = torch.empty(cfg.workspace_size(T), dtype=torch.uint8, device=x.device)
    L = len(copies)
    spin_up(lambda i: moe.forward(x, copies[i % L], cfg, ws=ws, out=y), spinup_ms)
    for i in range(warmup):
        moe.forward(x, copies[i % L], cfg, ws=ws, out=y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        moe.forward(x, copies[i % L], cfg, ws=ws, out=y)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # per-step durations for the percentiles: one event after each step on the launch
    # stream (a pass of its own; the loop above records none)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        moe.forward(x, copies[i % L], cfg, ws=ws, out=y)
        ev[i + 1].record()
    torch.cuda.synchronize()
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    _lib.check(moe.lib().moe_profile_enable(stage_mask, max(8, 16 * steps)))
    torch.cuda.synchronize()
    for i in range(steps):
        moe.forward(x, copies[i % L], cfg, ws=ws, out=y)
    torch.cuda.synchronize()
    st = stage_times(moe, stage_mask)
    _lib.check(moe.lib().moe_profile_disable())
    return t1 - t0, st, per_step


def percentile(sorted_vals, q):
    """q-th percentile (0..100) of an ascending list, by linear interpolation."""
    if not sorted_vals:
        return None
    pos = (len(sorted_vals) - 1) * q / 100.0
    lo = int(np.floor(pos))
    hi = min(lo + 1, len(sorted_vals) - 1)
    return sorted_vals[lo] + (sorted_vals[hi] - sorted_vals[lo]) * (pos - lo)


def run_graph(moe, cfg, copies, x, steps, warmup, spinup_ms=0.0):
    """HIP-graph replay: the L layer copies' calls captured back to back in one graph (as
    a model's decode step captures its layers), replayed until `steps` layer calls have
    run; returns the seconds for `steps` layer calls and whether every layer's output
    equals its eager result.  (One graph per layer call would add the runtime's per-graph
    launch cost, about 8 us on this stack, to every call.)  Like the eager loop, the
    replays first run untimed for `spinup_ms`: the capture leaves the GPU idle, and the
    clocks take tens of milliseconds of load to come back up."""
    import torch
    T = x.shape[0]
    L = len(copies)
    ys = [torch.empty_like(x) for _ in range(L)]
    wss = [torch.empty(cfg.workspace_size(T), dtype=torch.uint8, device=x.device) for _ in range(L)]
    for i in range(L):                      # eager reference outputs (and warm caches)
        moe.forward(x, copies[i], cfg, ws=wss[i], out=ys[i])
    torch.cuda.synchronize()
    ref = [y.clone() for y in ys]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(L):
                moe.forward(x, copies[i], cfg, ws=wss[i], out=ys[i])
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for y in ys:
        y.zero_()
    reps = max(1, -(-steps // L))
    for _ in range(max(1, -(-warmup // L))):
        g.replay()
    torch.cuda.synchronize()
    ok = all(torch.equal(ys[i], ref[i]) for i in range(L))
    if spinup_ms > 0:
        spin_up(lambda i: g.replay(), spinup_ms)
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * steps / (reps * L), ok


def cpu_baseline(spec, L_host, x_host, n_tok):
    """The fp64 oracle timed on the host on the first n_tok tokens of the batch; also
    returns its first pass's outputs and diagnostics (for the parity fields)."""
    from dataclasses import fields
    import oracle.moe_oracle as om
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        cores = os.cpu_count() or 1
    tok = np.arange(min(n_tok, x_host.shape[0]))
    ocfg = om.OracleConfig(**{f.name: getattr(spec, f.name) for f in fields(om.OracleConfig)})
    # repeat the token sample until about min_seconds of oracle work (bounded by max_passes)
    min_seconds, max_passes = 10.0, 20
    passes, t0 = 0, time.perf_counter()
    first = None
    while True:
        out = om.forward(x_host, L_host, ocfg, tokens=tok)
        if first is None:
            first = out
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= max_passes:
            break
    rec = dict(value=passes * len(tok) / dt, unit="tokens/s", cores=int(cores), kind="oracle",
               sample=f"fp64 oracle (NumPy/BLAS) on {len(tok)} tokens of the T={x_host.shape[0]} batch "
                      f"(same layer and routing), {passes} passes, {dt:.1f} s on {cores} threads")
    return rec, tok, first


MARGIN = 1e-5      # routing decisions closer than this to a tie may flip under rounding
Y_TOL = {"bf16": 2e-2, "f32": 1e-4}


def parity_fields(spec, L_host, x_host, y_gpu, idx_gpu, tok, oracle_out=None):
    """The GPU batch against the fp64 oracle on tokens `tok`: routing-set mismatches on
    tokens whose decision margin exceeds 1e-5, the near-tie count, masked picks, and the
    largest per-token relative error of the outputs (near-tie tokens compared with the
    oracle re-run on the GPU's own expert sets)."""
    from dataclasses import fields
    import oracle.moe_oracle as om
    ocfg = om.OracleConfig(**{f.name: getattr(spec, f.name) for f in fields(om.OracleConfig)})
    y_o, d = oracle_out if oracle_out is not None else om.forward(x_host, L_host, ocfg, tokens=tok)
    y_o = y_o.copy()
    ig = idx_gpu[tok]
    near = d["margin"] <= MARGIN
    mism = sum(int(set(ig[t].tolist()) != set(d["idx"][t].tolist())) for t in np.nonzero(~near)[0])
    if near.any():
        nz = np.nonzero(near)[0]
        y_f, _ = om.forward(x_host, L_host, ocfg, tokens=tok[nz], forced_idx=ig[nz])
        y_o[nz] = y_f
    yg = y_gpu[tok]
    rel = np.abs(yg - y_o).max(axis=1) / np.maximum(np.abs(y_o).max(axis=1), 1e-30)
    return dict(tokens=int(len(tok)), set_mismatches=int(mism), near_ties=int(near.sum()),
                masked_picks=int(d["masked_pick"].sum()), max_rel_err=float(rel.max()),
                tolerance=Y_TOL[spec.act_dtype], ok=bool(mism == 0 and rel.max() <= Y_TOL[spec.act_dtype]))


def parity_sample(T, n, seed=0):
    """Every token up to 64 (or n); beyond, the first, the last and a seeded random set."""
    if T <= max(64, n):
        return np.arange(T)
    rng = np.random.default_rng(seed + T)
    mid = rng.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, T - 1], mid]))


def copy_bandwidth(dev, nbytes=1 << 30, reps=10):
    """Device-to-device copy of nbytes (read + write bytes per second): the reference
    kernel the HBM counters are scaled with, and a measured bandwidth ceiling."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    del a, b
    torch.cuda.empty_cache()
    return 2.0 * nbytes / sec / 1e9


def recorded_traffic(kernel_key, digest, launch_div=1.0):
    """Counter-measured HBM bytes per launch, if recorded for exactly this source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != digest:
        return None
    k = rec.get("kernels", {}).get(kernel_key)
    if not k:
        return None
    return k.get("hbm_bytes_per_launch")


def bench_dense(args):
    """The dense gated MLP (moe_dense_mlp) on the Ling-2.6-flash layer-0 shape: same timing
    protocol and JSON line as the MoE workloads (eager and graph replay over rotated weight
    copies; roofline of the gate/up kernel; the oracle's gated MLP as the CPU baseline)."""
    import torch
    import synth
    import mixture_experts_layer_03_amd as moe
    from mixture_experts_layer_03_amd import _lib
    import oracle.moe_oracle as om
    spec = synth.DENSE["ling-2.6-flash-dense0"]
    H, I = spec.hidden, spec.intermediate
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    W_host = synth.make_dense(spec)
    copies = [{k: moe.host_tensor_to_device(v, dev) for k, v in W_host.items()}]
    gen_s = time.perf_counter() - t_gen
    w_bytes = 3 * I * H * 2
    ncp = max(1, min(args.max_copies, int(np.ceil(args.min_rotation_bytes / w_bytes))))
    g = torch.Generator(device=dev)
    g.manual_seed(7919 + spec.seed_id)
    while len(copies) < ncp:   # timing-only copies drawn on the GPU with the same distribution
        copies.append({k: (torch.randn(t.shape, generator=g, device=dev) * spec.weight_std).to(torch.bfloat16)
                       for k, t in copies[0].items()})
    cfg = moe.MoEConfig(hidden=H, num_experts=8, top_k=2, moe_intermediate=64, shared_intermediate=0)
    digest = source_digest()
    Ts = [args.tokens] + [int(t) for t in args.decode_tokens.split(",") if t.strip()]
    results, head_x = {}, None
    for T in Ts:
        x_host = synth.make_x(spec, T)
        x = moe.host_tensor_to_device(x_host, dev)
        if T == args.tokens:
            head_x = x_host
        y = torch.empty_like(x)
        ws = torch.empty(moe.dense_workspace_size(cfg, I, T), dtype=torch.uint8, device=dev)
        steps = args.steps if T == args.tokens else max(args.steps, 100)

        def call(i, out=y, wsp=ws):
            W = copies[i % len(copies)]
            moe.dense_mlp(x, W["gate"], W["up"], W["down"], cfg, ws=wsp, out=out)
        spin_up(call, args.spinup_ms)
        for i in range(args.warmup):
            call(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            call(i)
        torch.cuda.synchronize()
        secs = time.perf_counter() - t0
        mask = _lib.STAGES["shared_up"]   # stage events in a second, untimed pass
        _lib.check(moe.lib().moe_profile_enable(mask, max(8, 16 * steps)))
        torch.cuda.synchronize()
        for i in range(steps):
            call(i)
        torch.cuda.synchronize()
        st = stage_times(moe, mask)
        _lib.check(moe.lib().moe_profile_disable())
        t_step = secs / steps
        byt = w_bytes + 2 * T * H * 2
        fl = 6.0 * T * H * I
        r = dict(T=T, copies=len(copies), ms_per_step=t_step * 1e3, tokens_per_s=T / t_step,
                 hbm_gbps=byt / t_step / 1e9, mfma_tflops=fl / t_step / 1e12,
                 up_ms=st.get("shared_up"), path="decode" if T <= DENSE_STREAM_MAX_T else "prefill")
        r["hbm_frac"] = r["hbm_gbps"] / HBM_PEAK_GBPS
        r["mfma_frac"] = r["mfma_tflops"] / BF16_PEAK_TFLOPS
        r["roofline_frac"] = max(byt / (HBM_PEAK_GBPS * 1e9), fl / (BF16_PEAK_TFLOPS * 1e12)) / t_step
        if not args.no_graph:
            L = len(copies)
            ys = [torch.empty_like(x) for _ in range(L)]
            wss = [torch.empty_like(ws) for _ in range(L)]
            for i in range(L):
                call(i, ys[i], wss[i])
            torch.cuda.synchronize()
            ref = [t.clone() for t in ys]
            # the L copies' calls back to back in one graph, as run_graph does
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.stream(s):
                with torch.cuda.graph(gr, stream=s):
                    for i in range(L):
                        call(i, ys[i], wss[i])
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            for y in ys:
                y.zero_()
            reps = max(1, -(-steps // L))
            for _ in range(max(1, -(-args.warmup // L))):
                gr.replay()
            torch.cuda.synchronize()
            ok = all(torch.equal(ys[i], ref[i]) for i in range(L))
            if args.spinup_ms > 0:
                spin_up(lambda i: gr.replay(), args.spinup_ms)
            t0 = time.perf_counter()
            for _ in range(reps):
                gr.replay()
            torch.cuda.synchronize()
            gt = (time.perf_counter() - t0) / (reps * L)
            r.update(graph_ms_per_step=gt * 1e3, graph_tokens_per_s=T / gt,
                     graph_roofline_frac=max(byt / (HBM_PEAK_GBPS * 1e9), fl / (BF16_PEAK_TFLOPS * 1e12)) / gt,
                     graph_matches_eager=ok)
        results[T] = r
    head = results[args.tokens]
    T = args.tokens
    roof = None
    if head.get("up_ms"):
        up_s = head["up_ms"] * 1e-3
        if head["path"] == "prefill":
            ach = 4.0 * T * H * I / up_s / 1e12
            roof = dict(bound="mfma", achieved=ach, peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                        frac=ach / BF16_PEAK_TFLOPS, traffic=None, avg_ms=head["up_ms"],
                        kernel="dense gate/up GEMM + SwiGLU (copy-pipeline tiles)", algorithmic_flops=4.0 * T * H * I)
        else:
            ub = 2 * I * H * 2 + T * H * 2 + T * I * 2
            ach = ub / up_s / 1e9
            roof = dict(bound="hbm", achieved=ach, peak=HBM_PEAK_GBPS, unit="GB/s", frac=ach / HBM_PEAK_GBPS,
                        traffic=None, avg_ms=head["up_ms"], kernel="dense gate/up weight streaming + SwiGLU",
                        algorithmic_bytes=ub)
    cpu = None
    if not args.no_cpu_baseline:
        try:
            from threadpoolctl import threadpool_info
            cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
        except Exception:
            cores = os.cpu_count() or 1
        n = min(args.cpu_sample_tokens, T)
        X = om.to_f64(head_x[:n])
        Wg, Wu, Wd = (om.to_f64(W_host[k]) for k in ("gate", "up", "down"))
        passes, t0 = 0, time.perf_counter()
        while True:
            om.swiglu_mlp(X, Wg, Wu, Wd)
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= 10.0 or passes >= 20:
                break
        cpu = dict(value=passes * n / dt, unit="tokens/s", cores=int(cores), kind="oracle",
                   sample=f"fp64 oracle gated MLP (NumPy/BLAS) on {n} tokens of the T={T} batch, "
                          f"{passes} passes, {dt:.1f} s on {cores} threads")
    line = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "spinup_ms": args.spinup_ms, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{spec.name} dense gated MLP: hidden {H}, intermediate {I}; T={T}",
                   "tokens": T, "layer_gb": round(w_bytes / 1e9, 4)},
        "roofline": roof, "cpu_baseline": cpu, "hbm_gbps": head["hbm_gbps"], "mfma_frac": head["mfma_frac"],
        "roofline_frac": head["roofline_frac"],
        "per_T": [{k: (round(v, 5) if isinstance(v, float) else v) for k, v in results[t].items()} for t in Ts],
        "source_digest": digest, "gen_seconds": round(gen_s, 2),
    }
    print(json.dumps(line), flush=True)


def measure_workload(args, spec, Ts, dev, headline_T=None, cpu=False):
    """Every batch size of one workload: eager and graph-replay times (with per-step
    percentiles), the routed gate/up kernel's event-timed average, the parity fields, and
    (cpu) the oracle's host rate.  Returns (results by T, cpu_baseline record or None)."""
    import torch
    import synth
    import mixture_experts_layer_03_amd as moe
    from mixture_experts_layer_03_amd import _lib
    t_gen = time.perf_counter()
    L_host = synth.make_layer(spec)
    W0 = moe.weights_from_host(L_host, dev)
    gen_s = time.perf_counter() - t_gen
    all_copies = [W0]

    def get_copies(n):
        while len(all_copies) < n:
            all_copies.append(gpu_copy(spec, len(all_copies), W0, dev))
        return all_copies[:n]

    cfg = moe.MoEConfig.from_object(spec)
    results, cpu_rec = {}, None
    for T in Ts:
        x_host = synth.make_x(spec, T)
        x = moe.host_tensor_to_device(x_host, dev)
        y0, (idx, wt, counts) = moe.forward(x, W0, cfg, return_routing=True)
        torch.cuda.synchronize()
        alg = algorithmic(spec, T, counts.cpu().numpy())
        ncp = max(1, min(args.max_copies, int(np.ceil(args.min_rotation_bytes / max(alg["bytes"], 1.0)))))
        cps = get_copies(ncp)
        mask = _lib.STAGES["up"] | _lib.STAGES["down"]
        steps = args.steps if T == headline_T else max(args.steps, 100)
        secs, stages, per_step = run_eager(moe, cfg, cps, x, steps, args.warmup, mask, args.spinup_ms)
        t_step = secs / steps
        r = dict(T=T, copies=ncp, ms_per_step=t_step * 1e3, tokens_per_s=T / t_step,
                 hbm_gbps=alg["bytes"] / t_step / 1e9, mfma_tflops=alg["flops"] / t_step / 1e12,
                 distinct_experts=alg["D"], stage_ms=stages, alg=alg, path=cfg.kernel_path(T),
                 step_ms_p10=percentile(per_step, 10), step_ms_p50=percentile(per_step, 50),
                 step_ms_p90=percentile(per_step, 90))
        r["hbm_frac"] = r["hbm_gbps"] / HBM_PEAK_GBPS
        r["mfma_frac"] = r["mfma_tflops"] / BF16_PEAK_TFLOPS
        r["roofline_frac"] = max(alg["bytes"] / (HBM_PEAK_GBPS * 1e9),
                                 alg["flops"] / (BF16_PEAK_TFLOPS * 1e12)) / t_step
        up_ms = stages.get("up")
        if up_ms:
            if r["path"] == "prefill":
                r["up_tflops"] = alg["up_flops"] / (up_ms * 1e-3) / 1e12
                r["up_mfma_frac"] = r["up_tflops"] / BF16_PEAK_TFLOPS
            else:
                r["up_gbps"] = alg["up_bytes_decode"] / (up_ms * 1e-3) / 1e9
                r["up_hbm_frac"] = r["up_gbps"] / HBM_PEAK_GBPS
        if not args.no_graph:
            gsecs, ok = run_graph(moe, cfg, cps, x, steps, args.warmup, args.spinup_ms)
            gt = gsecs / steps
            r.update(graph_ms_per_step=gt * 1e3, graph_tokens_per_s=T / gt,
                     graph_hbm_gbps=alg["bytes"] / gt / 1e9,
                     graph_hbm_frac=alg["bytes"] / gt / 1e9 / HBM_PEAK_GBPS,
                     graph_roofline_frac=max(alg["bytes"] / (HBM_PEAK_GBPS * 1e9),
                                             alg["flops"] / (BF16_PEAK_TFLOPS * 1e12)) / gt,
                     graph_matches_eager=ok)
        y_h = y0.float().cpu().numpy().astype(np.float64)
        idx_h = idx.cpu().numpy()
        if cpu and T == headline_T and not args.no_cpu_baseline:
            cpu_rec, tok, first = cpu_baseline(spec, L_host, x_host, args.cpu_sample_tokens)
            if not args.no_parity:
                r["parity"] = parity_fields(spec, L_host, x_host, y_h, idx_h, tok, first)
        elif not args.no_parity:
            r["parity"] = parity_fields(spec, L_host, x_host, y_h, idx_h, parity_sample(T, args.parity_tokens))
        results[T] = r
    del all_copies, W0
    torch.cuda.empty_cache()
    return results, cpu_rec, gen_s


def brief(r):
    return {k: (round(v, 5) if isinstance(v, float) else v) for k, v in r.items() if k != "alg"}


def workload_name(spec):
    return (f"{spec.name} MoE layer: hidden {spec.hidden}, {spec.num_experts} experts top-{spec.top_k}, "
            f"moe_intermediate {spec.moe_intermediate}, shared {spec.shared_intermediate}, {spec.score_function}, "
            f"n_group {spec.n_group}, experts {spec.expert_dtype}")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this layer build has no multi-GPU path "
              "(expert-parallel sharding is a design note only); use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, ROOT)
    if args.dense:
        bench_dense(args)
        return
    import torch
    import synth

    spec = synth.SPECS[args.config]
    dev = torch.device("cuda:0")
    lb = synth.layer_bytes(spec)
    layer_bytes = spec.num_experts * lb["expert"] + lb["shared"] + lb["router"]
    digest = source_digest()
    Ts = [args.tokens] + [int(t) for t in args.decode_tokens.split(",") if t.strip()]
    results, cpu, gen_s = measure_workload(args, spec, Ts, dev, headline_T=args.tokens, cpu=True)

    per_config = []
    for item in [q for q in args.per_config.split(";") if q.strip()]:
        cid, ts = item.split(":")
        pspec = synth.SPECS[int(cid)]
        pT = [int(t) for t in ts.split(",") if t.strip()]
        pres, _, _ = measure_workload(args, pspec, pT, dev, headline_T=max(pT))
        per_config.append({"config": int(cid), "workload": workload_name(pspec),
                           "per_T": [brief(pres[t]) for t in pT]})

    copy_gbps = copy_bandwidth(dev)

    head = results[args.tokens]
    alg = head["alg"]
    up_ms = head["stage_ms"].get("up")
    prefill = head["path"] == "prefill"
    roof = None
    if up_ms:
        if prefill:
            ach = alg["up_flops"] / (up_ms * 1e-3) / 1e12
            key = f"up_tiled_cfg{args.config}_T{args.tokens}"
            roof = dict(bound="mfma", achieved=ach, peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                        frac=ach / BF16_PEAK_TFLOPS, traffic=recorded_traffic(key, digest),
                        kernel="routed gate/up grouped GEMM + SwiGLU (copy-pipeline tiles: k_tile_dma_split "
                               "when the last 256-column tile is at most half full, else k_tile_dma; gather, dual)",
                        avg_ms=up_ms, algorithmic_flops=alg["up_flops"])
        else:
            ach = alg["up_bytes_decode"] / (up_ms * 1e-3) / 1e9
            key = f"up_stream_cfg{args.config}_T{args.tokens}"
            roof = dict(bound="hbm", achieved=ach, peak=HBM_PEAK_GBPS, unit="GB/s",
                        frac=ach / HBM_PEAK_GBPS, traffic=recorded_traffic(key, digest),
                        kernel="routed+shared gate/up weight streaming + SwiGLU (" + {
                            "bf16": "k_stream_up", "u8": "k_stream_up_q<8>", "u4": "k_stream_up_q<4>",
                            "f32": "k_skinny_up"}[spec.expert_dtype] + ")",
                        avg_ms=up_ms, algorithmic_bytes=alg["up_bytes_decode"])

    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "spinup_ms": args.spinup_ms,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if spec.act_dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": workload_name(spec) + f"; T={args.tokens}",
                   "tokens": args.tokens, "layer_gb": round(layer_bytes / 1e9, 4)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "hbm_gbps": head["hbm_gbps"],
        "mfma_frac": head["mfma_frac"],
        "roofline_frac": head["roofline_frac"],
        "step_ms_p10": head["step_ms_p10"],
        "step_ms_p90": head["step_ms_p90"],
        "parity": head.get("parity"),
        "copy_gbps": copy_gbps,
        "per_T": [brief(results[T]) for T in Ts],
        "per_config": per_config,
        "source_digest": digest,
        "gen_seconds": round(gen_s, 2),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
