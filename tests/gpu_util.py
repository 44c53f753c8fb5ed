"""Helpers shared by the GPU parity tests: configs, device upload, comparisons.

Tolerances (the derivation is in the repository's design notes):
  * routing sets must match the oracle exactly on every token whose decision
    margin exceeds 1e-5; tokens at or under it are counted and checked against
    the oracle re-run with the GPU's own choice (forced routing);
  * routing weights: |w - w_oracle| <= 1e-5 * max(1, |w_oracle|);
  * outputs, per token: ||y - y_oracle||_inf / ||y_oracle||_inf <= 2e-2 for
    bf16 layers and 1e-4 for fp32 layers.
"""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle.moe_oracle as om
import synth
from dataclasses import fields

from mixture_experts_layer_03_amd import (MoEConfig, MoEWeights, host_tensor_to_device,
                                           weights_from_host)

MARGIN = 1e-5
W_TOL = 1e-5
Y_TOL = {"bf16": 2e-2, "f32": 1e-4}

# Reduced layers with the routing structure of the workloads: sizes the
# oracle finishes in seconds that still span several tiles and ragged tails.
SMALL = {
    1: synth.SPECS[1],
    2: synth.SPECS[2].variant("ling-lite-small", 102, hidden=512, moe_intermediate=192,
                               shared_intermediate=384, num_experts=16),
    3: synth.SPECS[3].variant("ling-2.6-small", 103, hidden=256, moe_intermediate=128,
                               shared_intermediate=128),
    4: synth.SPECS[4].variant("ling-3.0-small", 104, hidden=256, moe_intermediate=128,
                               shared_intermediate=128),
}
SMALL[5] = SMALL[4].variant("ling-3.0-small-u8", 104, expert_dtype="u8")
# packed int4 experts: more 128-element steps per row, fewer experts so that chunks of
# 4, 8 and 16 tokens and several chunks per expert all occur
SMALL[6] = SMALL[4].variant("ling-3.0-small-u4", 106, expert_dtype="u4", hidden=1024, moe_intermediate=384,
                            shared_intermediate=256, num_experts=64)
SMALL[7] = synth.SPECS[7].variant("ling-3.0-tiny-small", 107, hidden=256, moe_intermediate=128,
                                  shared_intermediate=128)


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def moe_cfg(spec: synth.LayerSpec, path: str = "auto") -> MoEConfig:
    return MoEConfig.from_object(spec, path=path)


def oracle_cfg(spec: synth.LayerSpec) -> om.OracleConfig:
    return om.OracleConfig(**{f.name: getattr(spec, f.name) for f in fields(om.OracleConfig)})


def to_dev(a, device="cuda"):
    return host_tensor_to_device(a, device)


def device_weights(L: dict, device="cuda") -> MoEWeights:
    return weights_from_host(L, device)


def y_to_f64(y: torch.Tensor) -> np.ndarray:
    return y.float().cpu().numpy().astype(np.float64)


def check_route(spec, idx_g, w_g, L, x, tokens=None):
    """Compare GPU routing with the oracle on `tokens` (all when None). Returns stats."""
    ocfg = oracle_cfg(spec)
    idx_o, w_o, margin, masked = om.route(x, L["router"], ocfg, L.get("router_bias"),
                                          L.get("expert_bias"), tokens=tokens)
    ig = idx_g if tokens is None else idx_g[tokens]
    wg = w_g if tokens is None else w_g[tokens]
    near = 0
    for t in range(idx_o.shape[0]):
        sg, so = ig[t].tolist(), idx_o[t].tolist()
        assert len(set(sg)) == len(sg), f"token {t}: duplicate experts {sg}"
        assert all(0 <= e < spec.num_experts for e in sg), f"token {t}: index out of range {sg}"
        if margin[t] > MARGIN:
            assert set(sg) == set(so), f"token {t} (margin {margin[t]:.3g}): gpu {sorted(sg)} oracle {sorted(so)}"
            ref = dict(zip(so, w_o[t]))
            for e, wv in zip(sg, wg[t]):
                assert abs(wv - ref[e]) <= W_TOL * max(1.0, abs(ref[e])), \
                    f"token {t} expert {e}: weight {wv} vs {ref[e]}"
        else:
            near += 1
    return dict(tokens=idx_o.shape[0], near_ties=near, masked_picks=int(masked.sum()),
                idx_o=idx_o, w_o=w_o, margin=margin)


def check_forward(spec, y_g, idx_g, L, x, tokens=None):
    """Compare GPU outputs with the oracle (forced to the GPU's sets on near-tie tokens)."""
    ocfg = oracle_cfg(spec)
    tok = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    y_o, d = om.forward(x, L, ocfg, tokens=tok)
    ig = idx_g[tok]
    near = np.nonzero(d["margin"] <= MARGIN)[0]
    if near.size:
        y_f, _ = om.forward(x, L, ocfg, tokens=tok[near], forced_idx=ig[near])
        y_o[near] = y_f
    yg = y_g[tok]
    num = np.abs(yg - y_o).max(axis=1)
    den = np.abs(y_o).max(axis=1)
    rel = num / np.maximum(den, 1e-30)
    tol = Y_TOL[spec.act_dtype]
    worst = int(rel.argmax())
    assert rel.max() <= tol, f"max rel err {rel.max():.3e} at token {tok[worst]} (tol {tol})"
    return dict(max_rel=float(rel.max()), near_ties=int(near.size), tokens=len(tok))
