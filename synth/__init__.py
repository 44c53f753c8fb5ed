"""Seeded synthetic inputs for the MoE layer: the workload shapes and their tensors.

This module is shared by the tests, the benchmark and the smoke check.  It
holds none of the layer's arithmetic: only shapes, seeded random streams,
bf16 encoding of the drawn values, the u8 affine encoder for quantised
experts and the Zipf expert-popularity skew.  It imports neither the oracle
nor the HIP package.

Recipe (every tensor is drawn in fp32 from numpy's PCG64, one independent
stream per (layer seed, layer copy, tensor, expert), then encoded):
  * weights   N(0, 0.02) (0.02 is the standard deviation), rounded
              to-nearest-even to bf16 (kept fp32 for the fp32 toy layer);
  * x         N(0, 1), bf16 (fp32 for the toy layer), stream keyed by T;
  * expert correction bias   N(0, 0.01), fp32;
  * Zipf skew (router bias)  a seeded permutation gives expert e a rank
              r_e in 1..E and b_e = -a ln r_e + a mean_e(ln r_e), a = 1.1;
  * u8 experts  per 64 consecutive elements along a row's reduction axis:
              lo = min(min w, 0), hi = max(max w, 0),
              s = fp16 rounded up of (hi - lo) / 254, z = rint(-lo / s),
              q = rint(w / s) + z  (always inside [0, 255]), z stored as fp16;
  * u4 experts  the same with (hi - lo) / 14 (q inside [0, 15]), codes packed
              two per byte along the row: element 2i in the low nibble of
              byte i, element 2i+1 in the high nibble.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

# tensor ids of the seed streams
_T_ROUTER, _T_ZIPF, _T_EBIAS, _T_GATE, _T_UP, _T_DOWN, _T_SGATE, _T_SUP, _T_SDOWN, _T_X = range(10)


@dataclass(frozen=True)
class LayerSpec:
    """Shape, routing parameters and storage types of one MoE layer workload."""

    name: str
    seed_id: int
    hidden: int
    num_experts: int
    top_k: int
    moe_intermediate: int
    shared_intermediate: int
    score_function: str = "softmax"
    n_group: int = 1
    topk_group: int = 1
    routed_scaling_factor: float = 1.0
    norm_topk_prob: bool = True
    use_expert_bias: bool = False
    zipf_skew: float = 0.0            # 0 = no router bias
    act_dtype: str = "bf16"           # "f32" | "bf16"
    expert_dtype: str = "bf16"        # "f32" | "bf16" | "u8" | "u4"
    quant_group: int = 64
    tokens: tuple = field(default=(1,))
    weight_std: float = 0.02
    bias_std: float = 0.01

    def variant(self, name: str, seed_id: int, **kw) -> "LayerSpec":
        return replace(self, name=name, seed_id=seed_id, **kw)


# The workloads (hidden, experts, routing and storage per the model pages' families).
SPECS = {
    1: LayerSpec("toy-f32", 1, hidden=256, num_experts=8, top_k=2, moe_intermediate=128,
                 shared_intermediate=128, act_dtype="f32", expert_dtype="f32", tokens=(16,)),
    2: LayerSpec("ling-lite", 2, hidden=2048, num_experts=64, top_k=6, moe_intermediate=1408,
                 shared_intermediate=2816, tokens=(1, 8, 64, 4096)),
    3: LayerSpec("ling-2.6-flash", 3, hidden=4096, num_experts=256, top_k=8,
                 moe_intermediate=1024, shared_intermediate=1024, score_function="sigmoid",
                 n_group=8, topk_group=4, routed_scaling_factor=2.5, use_expert_bias=True,
                 tokens=(1, 64, 4096)),
    4: LayerSpec("ling-3.0-flash", 4, hidden=4096, num_experts=512, top_k=8,
                 moe_intermediate=1024, shared_intermediate=1024, score_function="sigmoid",
                 n_group=8, topk_group=4, use_expert_bias=True, zipf_skew=1.1,
                 tokens=(1, 8192)),
}
# config 5 = config 4's layer with the routed experts stored u8-affine (same seeds)
SPECS[5] = SPECS[4].variant("ling-3.0-flash-u8", 4, expert_dtype="u8", tokens=(1, 64, 8192))
# config 4's layer with the routed experts stored as packed int4 affine (decode sizes)
SPECS[6] = SPECS[4].variant("ling-3.0-flash-u4", 4, expert_dtype="u4", tokens=(1, 64))
# Ling-3.0-tiny: 128 routed + 1 shared experts, 8 active, 24 layers, 7.9B total / 1.3B
# active.  The hidden size is not given; hidden 2048 with expert width 384 reproduces
# both totals (routed experts 24 x 128 x 3 x 2048 x 384 = 7.25B, active experts
# 24 x 9 x 3 x 2048 x 384 = 0.51B, the rest attention and embeddings).  Routing as the
# Ling-3.0 family's flash model (sigmoid, 8 groups keep 4, correction bias).
SPECS[7] = LayerSpec("ling-3.0-tiny", 7, hidden=2048, num_experts=128, top_k=8, moe_intermediate=384,
                     shared_intermediate=384, score_function="sigmoid", n_group=8, topk_group=4,
                     use_expert_bias=True, tokens=(1, 64, 4096))


@dataclass(frozen=True)
class DenseSpec:
    """A dense gated MLP: the layers in front of the MoE layers (first_k_dense_replace)."""

    name: str
    seed_id: int
    hidden: int
    intermediate: int
    act_dtype: str = "bf16"
    tokens: tuple = field(default=(1,))
    weight_std: float = 0.02


# Ling-2.6-flash layer 0: dense MLP of intermediate 9216 (hidden 4096 as the MoE layers)
DENSE = {
    "ling-2.6-flash-dense0": DenseSpec("ling-2.6-flash-dense0", 31, hidden=4096, intermediate=9216,
                                       tokens=(1, 64, 4096)),
}


def make_dense(spec: DenseSpec, copy: int = 0) -> dict:
    """gate/up [I,H] and down [H,I] of a dense MLP (bf16 bit patterns, or fp32)."""
    H, I = spec.hidden, spec.intermediate
    out = {}
    for name, tid, shp in (("gate", _T_SGATE, (I, H)), ("up", _T_SUP, (I, H)), ("down", _T_SDOWN, (H, I))):
        v = _rng(spec.seed_id, copy, tid, 0).standard_normal(shp, dtype=np.float32)
        v *= np.float32(spec.weight_std)
        out[name] = v if spec.act_dtype == "f32" else bf16_bits(v)
    return out


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def bf16_bits(a) -> np.ndarray:
    """fp32 values -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_values(bits) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def quantize_u8(w, group: int = 64):
    """u8 affine encoding of fp32 values along the last axis (see module docstring).

    Returns (q uint8 [...,n], s float16 [...,n/group], z float16 [...,n/group]).
    """
    w = np.asarray(w, dtype=np.float32)
    n = w.shape[-1]
    if n % group:
        raise ValueError("row length must be a multiple of the quant group")
    wg = w.reshape(w.shape[:-1] + (n // group, group)).astype(np.float64)
    lo = np.minimum(wg.min(axis=-1), 0.0)
    hi = np.maximum(wg.max(axis=-1), 0.0)
    s64 = (hi - lo) / 254.0
    s16 = s64.astype(np.float16)
    up = s16.astype(np.float64) < s64
    s16[up] = np.nextafter(s16[up], np.float16(np.inf))
    s16 = np.maximum(s16, np.float16(2.0 ** -14))
    s = s16.astype(np.float64)
    z = np.rint(-lo / s)
    q = np.rint(wg / s[..., None]) + z[..., None]
    if q.min() < 0 or q.max() > 255:
        raise AssertionError("u8 encoder left [0, 255]")
    return (q.astype(np.uint8).reshape(w.shape), s16, z.astype(np.float16))


def quantize_u4(w, group: int = 64):
    """u4 affine encoding of fp32 values along the last axis (see module docstring).

    Returns (packed uint8 [...,n/2], s float16 [...,n/group], z float16 [...,n/group]).
    """
    w = np.asarray(w, dtype=np.float32)
    n = w.shape[-1]
    if n % group or n % 2:
        raise ValueError("row length must be a multiple of the quant group")
    wg = w.reshape(w.shape[:-1] + (n // group, group)).astype(np.float64)
    lo = np.minimum(wg.min(axis=-1), 0.0)
    hi = np.maximum(wg.max(axis=-1), 0.0)
    s64 = (hi - lo) / 14.0
    s16 = s64.astype(np.float16)
    up = s16.astype(np.float64) < s64
    s16[up] = np.nextafter(s16[up], np.float16(np.inf))
    s16 = np.maximum(s16, np.float16(2.0 ** -14))
    s = s16.astype(np.float64)
    z = np.rint(-lo / s)
    q = (np.rint(wg / s[..., None]) + z[..., None]).reshape(w.shape)
    if q.min() < 0 or q.max() > 15:
        raise AssertionError("u4 encoder left [0, 15]")
    q = q.astype(np.uint8)
    packed = (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)
    return packed, s16, z.astype(np.float16)


def _threads(threads):
    if threads:
        return threads
    return max(1, min(16, os.cpu_count() or 1))


def _fill_expert_tensor(spec, copy, tid, shape_e, out_bits, E, threads):
    """Draw [E, *shape_e] weights, one stream per expert, into out_bits (bf16 or f32)."""
    def one(e):
        v = _rng(spec.seed_id, copy, tid, e).standard_normal(shape_e, dtype=np.float32)
        v *= np.float32(spec.weight_std)
        out_bits[e] = v if out_bits.dtype == np.float32 else bf16_bits(v)
    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(one, range(E)))


def make_layer(spec: LayerSpec, copy: int = 0, threads=None) -> dict:
    """All weights of one layer copy as numpy arrays (bf16 as uint16 bit patterns).

    Keys: router [E,H], router_bias [E] f32 or None, expert_bias [E] f32 or
    None, gate/up [E,I,H] and down [E,H,I] (or gate_q/gate_scale/gate_zero,
    ... for u8 experts; gate_q4/... with packed [E,I,H/2] codes for u4 experts),
    shared_gate/shared_up [I_s,H], shared_down [H,I_s]
    (None when there is no shared expert).
    """
    H, E, I, Is = spec.hidden, spec.num_experts, spec.moe_intermediate, spec.shared_intermediate
    f32 = spec.act_dtype == "f32"
    wdt = np.float32 if f32 else np.uint16

    def dense(tid, shape):
        v = _rng(spec.seed_id, copy, tid, 0).standard_normal(shape, dtype=np.float32)
        v *= np.float32(spec.weight_std)
        return v if f32 else bf16_bits(v)

    L = {"router": dense(_T_ROUTER, (E, H))}
    if spec.zipf_skew > 0:
        ranks = _rng(spec.seed_id, copy, _T_ZIPF, 0).permutation(E) + 1
        lr = np.log(ranks.astype(np.float64))
        L["router_bias"] = (-spec.zipf_skew * lr + spec.zipf_skew * lr.mean()).astype(np.float32)
    else:
        L["router_bias"] = None
    if spec.use_expert_bias:
        L["expert_bias"] = (_rng(spec.seed_id, copy, _T_EBIAS, 0).standard_normal(E)
                            * spec.bias_std).astype(np.float32)
    else:
        L["expert_bias"] = None

    edt = np.float32 if spec.expert_dtype == "f32" else np.uint16
    for name, tid, shp in (("gate", _T_GATE, (I, H)), ("up", _T_UP, (I, H)),
                           ("down", _T_DOWN, (H, I))):
        arr = np.empty((E,) + shp, dtype=edt)
        _fill_expert_tensor(spec, copy, tid, shp, arr, E, threads)
        if spec.expert_dtype in ("u8", "u4"):
            u4 = spec.expert_dtype == "u4"
            q = np.empty((E, shp[0], shp[1] // 2 if u4 else shp[1]), dtype=np.uint8)
            s = np.empty((E, shp[0], shp[1] // spec.quant_group), dtype=np.float16)
            z = np.empty_like(s)
            encode = quantize_u4 if u4 else quantize_u8

            def enc(e, arr=arr, q=q, s=s, z=z, encode=encode):
                q[e], s[e], z[e] = encode(bf16_values(arr[e]), spec.quant_group)
            with ThreadPoolExecutor(_threads(threads)) as ex:
                list(ex.map(enc, range(E)))
            L[name + ("_q4" if u4 else "_q")], L[name + "_scale"], L[name + "_zero"] = q, s, z
            del arr
        else:
            L[name] = arr
    if Is > 0:
        L["shared_gate"] = dense(_T_SGATE, (Is, H))
        L["shared_up"] = dense(_T_SUP, (Is, H))
        L["shared_down"] = dense(_T_SDOWN, (H, Is))
    else:
        L["shared_gate"] = L["shared_up"] = L["shared_down"] = None
    assert all(v is None or v.dtype in (wdt, np.float32, np.uint8, np.float16, np.uint16)
               for v in L.values())
    return L


def make_x(spec, T: int, stream: int = 0) -> np.ndarray:
    """Hidden states [T,H] ~ N(0,1): bf16 bit patterns (fp32 values for the toy layer).
    `spec` is a LayerSpec or a DenseSpec."""
    v = _rng(spec.seed_id, stream, _T_X, T).standard_normal((T, spec.hidden), dtype=np.float32)
    return v if spec.act_dtype == "f32" else bf16_bits(v)


def layer_bytes(spec: LayerSpec) -> dict:
    """Stored bytes per routed expert, shared expert and router."""
    H, I, Is, E = spec.hidden, spec.moe_intermediate, spec.shared_intermediate, spec.num_experts
    bw = {"f32": 4.0, "bf16": 2.0, "u8": 1.0 + 4.0 / spec.quant_group,
          "u4": 0.5 + 4.0 / spec.quant_group}[spec.expert_dtype]
    ba = 4.0 if spec.act_dtype == "f32" else 2.0
    return dict(expert=3 * I * H * bw, shared=3 * Is * H * ba, router=E * H * ba,
                act=ba)
