"""GPU parity of the dense MLP (the layers in front of the MoE layers,
`first_k_dense_replace`) against the oracle's gated MLP, through the C ABI:
reduced sizes on every token, both paths and fp32; Ling-2.6-flash layer 0
(hidden 4096, intermediate 9216) at full size on sampled tokens."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as om
import synth
from gpu_util import log, to_dev, y_to_f64

pytestmark = pytest.mark.gpu

SMALL = {
    "bf16": synth.DenseSpec("dense-small", 131, hidden=256, intermediate=576),
    "f32": synth.DenseSpec("dense-small-f32", 132, hidden=256, intermediate=192, act_dtype="f32"),
}
TOL = {"bf16": 2e-2, "f32": 1e-4}
_CACHE = {}


def dense(spec):
    if spec.name not in _CACHE:
        _CACHE.clear()
        torch.cuda.empty_cache()
        W = synth.make_dense(spec)
        _CACHE[spec.name] = (W, {k: to_dev(v) for k, v in W.items()})
    return _CACHE[spec.name]


def cfg_of(spec, path):
    import mixture_experts_layer_03_amd as moe
    return moe.MoEConfig(hidden=spec.hidden, num_experts=8, top_k=2, moe_intermediate=64, shared_intermediate=0,
                         act_dtype=spec.act_dtype, expert_dtype=spec.act_dtype, path=path)


def check(spec, T, path, tokens=None):
    import mixture_experts_layer_03_amd as moe
    W, Wd = dense(spec)
    x = synth.make_x(spec, T)
    log(f"dense {spec.name} H={spec.hidden} I={spec.intermediate} T={T} path={path}")
    y = moe.dense_mlp(to_dev(x), Wd["gate"], Wd["up"], Wd["down"], cfg_of(spec, path))
    torch.cuda.synchronize()
    yg = y_to_f64(y)
    rows = np.arange(T) if tokens is None else tokens
    X = om.to_f64(x)[rows]
    y_o = om.swiglu_mlp(X, om.to_f64(W["gate"]), om.to_f64(W["up"]), om.to_f64(W["down"]))
    rel = np.abs(yg[rows] - y_o).max(axis=1) / np.abs(y_o).max(axis=1)
    log(f"  max rel err {rel.max():.3e}")
    assert rel.max() <= TOL[spec.act_dtype], rel.max()


@pytest.mark.parametrize("T,path", [(1, "auto"), (7, "auto"), (64, "auto"), (65, "auto"), (192, "auto"),
                                    (193, "auto"), (300, "auto"), (40, "prefill"), (65, "prefill"),
                                    (200, "decode")])
def test_dense_small(T, path):
    check(SMALL["bf16"], T, path)


@pytest.mark.parametrize("T", [1, 16, 100])
def test_dense_small_f32(T):
    check(SMALL["f32"], T, "auto")


def test_dense_zero_tokens_is_noop():
    import mixture_experts_layer_03_amd as moe
    spec = SMALL["bf16"]
    _, Wd = dense(spec)
    x = torch.empty((0, spec.hidden), dtype=torch.bfloat16, device="cuda")
    y = moe.dense_mlp(x, Wd["gate"], Wd["up"], Wd["down"], cfg_of(spec, "auto"))
    assert y.shape == (0, spec.hidden)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("T", synth.DENSE["ling-2.6-flash-dense0"].tokens)
def test_dense_full_size(T):
    spec = synth.DENSE["ling-2.6-flash-dense0"]
    tok = np.arange(T) if T <= 24 else np.sort(np.concatenate(
        [[0, T - 1], np.random.default_rng(T).choice(np.arange(1, T - 1), size=22, replace=False)]))
    check(spec, T, "auto", tokens=tok)
