"""Plain fp64 CPU oracle of the Bailing/Ling MoE FFN layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this module: it is read by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark, and by nothing else.  It shares no code
with the HIP library (no kernels, headers, helpers or constants).

What it computes, per token t (sources are the web pages about the model
family; each step names the page and the section it follows):

  O1  logits  l_e = sum_h x_h W_r[e,h] (+ b_r[e] when a router bias is given)
      -- mlxcel #838 "Validation checkpoint" (router mlp.gate.weight [E,H]) and
         "Weight remap" (the router may carry a bias).
  O2  scores  softmax over all E (default) or elementwise sigmoid, on the
      logits -- mlxcel #838 "Config fields the checkpoint does not contain"
      (score_function, default softmax) and "Router: selection uses biased
      scores, weights come from unbiased scores".
  O3  orig = s; sel = s + beta when the expert (correction) bias is enabled
      -- mlxcel #838 "Router: ..."; Ling-2.6-flash-JANGTQ card "Architecture
      (bailing_hybrid)", MoE routing paragraph (selection on biased scores,
      weighting on the original sigmoid scores).
  O4  grouped mask (n_group > 1): experts are cut into n_group contiguous
      equal groups, each group is scored, the topk_group best groups are kept
      and every other expert's selection score is set to 0.0 before top-k
      -- mlxcel #838 "Architecture notes" (groups kept, the rest zeroed) and
      "Defensive requirements" (the lowest n_group - topk_group groups are the
      ones dropped).  The group score is the sum of the two largest biased
      scores in the group: the Ling-2.6-flash-JANGTQ card says the routing
      math is identical to DeepSeek-V3, whose grouped routing scores a group
      by its top-2 sum.  (The pages do not spell this out; see the readings
      list that ships with the repository.)
  O5  S = the top_k experts by masked selection score; ties go to the lower
      expert index (the pages use argpartition, whose order is unspecified).
  O6  w_j = orig[S_j]  -- weights from the unbiased scores (mlxcel #838
      "Router: ...").
  O7  if top_k > 1 and norm_topk_prob: w <- w / (sum(w) + 1e-20)
      -- mlxcel #838 "Router: ..." (conditional, with the epsilon).
  O8  w <- w * routed_scaling_factor, always -- mlxcel #838
      "moe_router_enable_routed_scaling is dead code upstream".
  O9  expert e: h = silu(W_g[e] x) * (W_u[e] x),  r = W_d[e] h
      -- mlxcel #838 "Validation checkpoint" (gate_proj/up_proj/down_proj per
      expert, [out,in] layout) and "Weight remap" (gate_proj is the SwiGLU
      gate).  silu(a) = a * sigmoid(a).
  O10 shared expert: one MLP of width shared_dim * num_shared_experts, run on
      every token -- mlxcel #838 "Shared experts are one wide MLP".
  O11 y = sum_j w_j r_j + y_shared (shared weight exactly 1.0) -- same
      section.

Quantised routed experts (u8 code q, fp16 scale s and fp16 zero point z per
64 consecutive elements along each row's reduction axis) are dequantised as
s * (q - z), exactly, in fp64.  The 8-bit affine group-64 format is the MLX
one named by the Ling-3.0-tiny-8bit-XL-mlx card ("XL Quantization Recipe")
and by mlxcel #838 "Weight remap" (quant_predicate, group 64, 8 bits),
written here in scale/zero-point form.

4-bit routed experts (u4) use the same affine form per 64 elements with
codes q in [0, 15] packed two per byte along each row's reduction axis,
element 2i in the low nibble of byte i and element 2i+1 in the high nibble.
The pages run routed experts at 4 bits (Ling-3.0-flash-GGUF card, conversion
recipe: IQ4_XS; clm-0015 record, structural facts: Q4_K_M) without giving a
layout; this plain affine int4 layout is a reading, listed with the others.

Stored inputs are converted exactly to fp64 first: arrays of dtype uint16 are
bf16 bit patterns (bits << 16 gives the fp32 value), float16/32/64 arrays are
taken as they are.  Nothing is rounded afterwards.

Batching: the expert MLP of O9 is evaluated per expert for all tokens routed
to it (one matrix product per projection).  Each output row depends only on
its own token, so this is the per-token definition with the rows stacked.

Every function here is pinned by the CPU tests (brute force, closed forms,
invariants, a hand-computed example); see tests/test_oracle_pins.py.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# Value written into the selection scores of dropped groups (O4).  The pages
# say the dropped groups are "zeroed"; this is that zero, literally.
MASK_FILL = 0.0

# Renormalisation epsilon (O7).
RENORM_EPS = 1e-20


# --------------------------------------------------------------------------
# configuration
# --------------------------------------------------------------------------

@dataclass
class OracleConfig:
    """Routing and shape parameters the oracle needs (HF config field names)."""

    hidden: int
    num_experts: int
    top_k: int
    moe_intermediate: int
    shared_intermediate: int = 0          # shared_dim * num_shared_experts; 0 = none
    n_group: int = 1
    topk_group: int = 1
    score_function: str = "softmax"
    norm_topk_prob: bool = True
    routed_scaling_factor: float = 1.0
    use_expert_bias: bool = False
    quant_group: int = 64


# --------------------------------------------------------------------------
# exact conversion of stored tensors
# --------------------------------------------------------------------------

def to_f64(a) -> np.ndarray:
    """Stored tensor -> exact fp64 values (uint16 arrays are bf16 bit patterns)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype in (np.float16, np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"oracle: unsupported stored dtype {a.dtype}")


def dequant_u8(q, scale, zero, group: int = 64) -> np.ndarray:
    """u8 affine dequantisation w = s * (q - z), per `group` elements of the last axis."""
    q = np.asarray(q)
    if q.dtype != np.uint8:
        raise TypeError("dequant_u8: codes must be uint8")
    s = to_f64(scale)
    z = to_f64(zero)
    n = q.shape[-1]
    if n % group != 0 or s.shape[-1] != n // group or z.shape != s.shape:
        raise ValueError("dequant_u8: scale/zero shape does not match the code shape")
    qg = q.astype(np.float64).reshape(q.shape[:-1] + (n // group, group))
    w = s[..., None] * (qg - z[..., None])
    return w.reshape(q.shape)


def unpack_u4(packed) -> np.ndarray:
    """Two 4-bit codes per byte along the last axis -> one code per uint8 element:
    element 2i is the low nibble of byte i, element 2i+1 its high nibble."""
    p = np.asarray(packed)
    if p.dtype != np.uint8:
        raise TypeError("unpack_u4: packed codes must be uint8")
    q = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    q[..., 0::2] = p & 0x0F
    q[..., 1::2] = p >> 4
    return q


def dequant_u4(packed, scale, zero, group: int = 64) -> np.ndarray:
    """u4 affine dequantisation: unpack the nibbles, then w = s * (q - z) per group."""
    return dequant_u8(unpack_u4(packed), scale, zero, group)


# --------------------------------------------------------------------------
# routing steps O1-O8 (module-level functions so each can be inspected alone)
# --------------------------------------------------------------------------

def router_logits(x: np.ndarray, W_r: np.ndarray, router_bias=None) -> np.ndarray:
    """O1: l[t,e] = sum_h x[t,h] W_r[e,h] (+ b_r[e])."""
    l = to_f64(x) @ to_f64(W_r).T
    if router_bias is not None:
        l = l + to_f64(router_bias)[None, :]
    return l


def score(logits: np.ndarray, score_function: str) -> np.ndarray:
    """O2: softmax over the expert axis, or elementwise sigmoid."""
    l = np.asarray(logits, dtype=np.float64)
    if score_function == "softmax":
        m = l.max(axis=-1, keepdims=True)
        p = np.exp(l - m)
        return p / p.sum(axis=-1, keepdims=True)
    if score_function == "sigmoid":
        return 1.0 / (1.0 + np.exp(-l))
    raise ValueError(f"unknown score_function {score_function!r}")


def selection_scores(s: np.ndarray, expert_bias, use_expert_bias: bool) -> np.ndarray:
    """O3: the biased copy used only for selection."""
    if use_expert_bias:
        return s + to_f64(expert_bias)
    return s.copy()


def group_score(block: np.ndarray) -> float:
    """Score of one expert group: sum of its two largest selection scores (O4)."""
    top2 = np.sort(block)[::-1][:2]
    return float(top2.sum())


def kept_groups(sel: np.ndarray, n_group: int, topk_group: int):
    """O4: indices of the kept groups (best group score first, ties -> lower group)."""
    E = sel.shape[0]
    gs = E // n_group
    sigma = np.array([group_score(sel[g * gs:(g + 1) * gs]) for g in range(n_group)])
    # stable sort on -sigma: equal scores keep ascending group order
    order = np.argsort(-sigma, kind="stable")
    return order[:topk_group], sigma


def mask_groups(sel: np.ndarray, keep, n_group: int) -> np.ndarray:
    """O4: selection scores of experts outside the kept groups become MASK_FILL."""
    E = sel.shape[0]
    gs = E // n_group
    out = np.full_like(sel, MASK_FILL)
    for g in keep:
        out[g * gs:(g + 1) * gs] = sel[g * gs:(g + 1) * gs]
    return out


def select_topk(sel_masked: np.ndarray, k: int) -> np.ndarray:
    """O5: the k largest scores, descending; equal scores -> lower index first."""
    order = np.argsort(-sel_masked, kind="stable")
    return order[:k]


def gather_weights(orig: np.ndarray, sel: np.ndarray, S: np.ndarray) -> np.ndarray:
    """O6: routing weights come from the unbiased scores."""
    return orig[S].copy()


def normalize(w: np.ndarray, top_k: int, norm_topk_prob: bool) -> np.ndarray:
    """O7: renormalise only when top_k > 1, with the 1e-20 epsilon."""
    if top_k > 1 and norm_topk_prob:
        return w / (w.sum() + RENORM_EPS)
    return w


def scale(w: np.ndarray, routed_scaling_factor: float) -> np.ndarray:
    """O8: unconditional routed scaling."""
    return w * float(routed_scaling_factor)


@dataclass
class TokenRoute:
    idx: np.ndarray            # [k] selected experts, descending masked selection score
    w: np.ndarray              # [k] final routing weights
    margin: float              # distance of the decision from a tie (see route_token)
    masked_pick: bool          # some selected expert lies in a dropped group
    sel_masked: np.ndarray = field(repr=False, default=None)


def route_token(l: np.ndarray, cfg: OracleConfig, expert_bias=None) -> TokenRoute:
    """O2-O8 for one token's logits l[E].

    margin = min(sel_(k) - sel_(k+1), sigma_(g) - sigma_(g+1)) on the masked
    fp64 selection scores (the group term only when groups are dropped); a
    token with a small margin can legitimately flip under rounding.
    """
    E = l.shape[0]
    k = cfg.top_k
    s = score(l[None, :], cfg.score_function)[0]
    orig = s
    sel = selection_scores(s, expert_bias, cfg.use_expert_bias)
    margin = math.inf
    dropped = np.zeros(E, dtype=bool)
    if cfg.n_group > 1 and cfg.topk_group < cfg.n_group:
        keep, sigma = kept_groups(sel, cfg.n_group, cfg.topk_group)
        sel_m = mask_groups(sel, keep, cfg.n_group)
        srt = np.sort(sigma)[::-1]
        margin = min(margin, srt[cfg.topk_group - 1] - srt[cfg.topk_group])
        gs = E // cfg.n_group
        dropped[:] = True
        for g in keep:
            dropped[g * gs:(g + 1) * gs] = False
    else:
        sel_m = sel
    S = select_topk(sel_m, k)
    if k < E:
        srt = np.sort(sel_m)[::-1]
        margin = min(margin, srt[k - 1] - srt[k])
    w = gather_weights(orig, sel, S)
    w = normalize(w, k, cfg.norm_topk_prob)
    w = scale(w, cfg.routed_scaling_factor)
    return TokenRoute(idx=S, w=w, margin=float(margin),
                      masked_pick=bool(dropped[S].any()), sel_masked=sel_m)


def route(x, W_r, cfg: OracleConfig, router_bias=None, expert_bias=None, tokens=None):
    """O1-O8 for the tokens listed in `tokens` (all when None).

    Returns idx [n,k] int64, w [n,k] fp64, margin [n], masked_pick [n].
    """
    x = np.asarray(x)
    if tokens is not None:
        x = x[np.asarray(tokens)]
    if cfg.use_expert_bias and expert_bias is None:
        raise ValueError("use_expert_bias set but no expert bias given")
    logits = router_logits(x, W_r, router_bias)
    n = logits.shape[0]
    k = cfg.top_k
    idx = np.zeros((n, k), dtype=np.int64)
    w = np.zeros((n, k), dtype=np.float64)
    margin = np.zeros(n)
    masked = np.zeros(n, dtype=bool)
    for t in range(n):
        r = route_token(logits[t], cfg, expert_bias)
        idx[t], w[t], margin[t], masked[t] = r.idx, r.w, r.margin, r.masked_pick
    return idx, w, margin, masked


# --------------------------------------------------------------------------
# expert MLPs and combine, O9-O11
# --------------------------------------------------------------------------

def silu(a: np.ndarray) -> np.ndarray:
    """silu(a) = a * sigmoid(a)."""
    return a / (1.0 + np.exp(-a))


def swiglu_mlp(X: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """O9/O10 for a stack of token rows X [n,H]: W_d (silu(W_g x) * (W_u x))."""
    h = silu(X @ Wg.T) * (X @ Wu.T)
    return h @ Wd.T


def expert_matrix(weights: dict, name: str, e: int, group: int) -> np.ndarray:
    """Routed expert e's projection `name` (gate/up/down) as exact fp64."""
    if name + "_q" in weights:
        return dequant_u8(weights[name + "_q"][e], weights[name + "_scale"][e],
                          weights[name + "_zero"][e], group)
    if name + "_q4" in weights:
        return dequant_u4(weights[name + "_q4"][e], weights[name + "_scale"][e],
                          weights[name + "_zero"][e], group)
    return to_f64(weights[name][e])


def combine(routed_terms: list, w_row: np.ndarray, y_shared):
    """O11: y = sum_j w_j r_j + y_shared (shared weight exactly 1.0)."""
    y = np.zeros_like(routed_terms[0]) if routed_terms else 0.0
    for j, r in enumerate(routed_terms):
        y = y + w_row[j] * r
    if y_shared is not None:
        y = y + y_shared
    return y


def forward(x, weights: dict, cfg: OracleConfig, tokens=None, forced_idx=None):
    """O1-O11.  Returns (y [n,H] fp64, diagnostics dict).

    weights keys: router [E,H], router_bias [E] or None, expert_bias [E] or
    None, gate/up [E,I,H] and down [E,H,I] (or gate_q/gate_scale/gate_zero...
    for u8 experts, gate_q4/... with [E,I,H/2] packed codes for u4 experts), shared_gate/shared_up [I_s,H], shared_down [H,I_s] (absent
    or None when there is no shared expert).

    tokens: optional list of token rows to evaluate (all when None).
    forced_idx: optional [n,k] expert sets to use instead of O4/O5's choice
    (forced-routing mode); weights are then recomputed from those sets by O6-O8.
    """
    x = np.asarray(x)
    T = x.shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    X = to_f64(x[tok])
    n, H = X.shape
    k = cfg.top_k
    logits = router_logits(x[tok], weights["router"], weights.get("router_bias"))
    idx = np.zeros((n, k), dtype=np.int64)
    w = np.zeros((n, k))
    margin = np.zeros(n)
    masked = np.zeros(n, dtype=bool)
    ebias = weights.get("expert_bias")
    for t in range(n):
        r = route_token(logits[t], cfg, ebias)
        margin[t], masked[t] = r.margin, r.masked_pick
        if forced_idx is None:
            idx[t], w[t] = r.idx, r.w
        else:
            S = np.asarray(forced_idx[t], dtype=np.int64)
            s = score(logits[t][None, :], cfg.score_function)[0]
            sel = selection_scores(s, ebias, cfg.use_expert_bias)
            ww = gather_weights(s, sel, S)
            ww = normalize(ww, k, cfg.norm_topk_prob)
            idx[t], w[t] = S, scale(ww, cfg.routed_scaling_factor)

    # O9: per-expert stacked evaluation of every (token, j) routed to it
    r_terms = np.zeros((n, k, H))
    E = cfg.num_experts
    for e in range(E):
        rows, js = np.nonzero(idx == e)
        if rows.size == 0:
            continue
        Wg = expert_matrix(weights, "gate", e, cfg.quant_group)
        Wu = expert_matrix(weights, "up", e, cfg.quant_group)
        Wd = expert_matrix(weights, "down", e, cfg.quant_group)
        r_terms[rows, js] = swiglu_mlp(X[rows], Wg, Wu, Wd)

    # O10
    y_s = None
    if cfg.shared_intermediate > 0:
        y_s = swiglu_mlp(X, to_f64(weights["shared_gate"]), to_f64(weights["shared_up"]),
                         to_f64(weights["shared_down"]))
    # O11
    y = np.zeros((n, H))
    for t in range(n):
        y[t] = combine([r_terms[t, j] for j in range(k)], w[t],
                       None if y_s is None else y_s[t])
    counts = np.bincount(idx.reshape(-1), minlength=E)
    diag = dict(idx=idx, w=w, margin=margin, masked_pick=masked, counts=counts,
                distinct=int((counts > 0).sum()), logits=logits)
    return y, diag


def expert_counts(idx: np.ndarray, num_experts: int):
    """Per-expert token counts and exclusive offsets of a routing table (permutation step)."""
    counts = np.bincount(np.asarray(idx).reshape(-1), minlength=num_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    return counts, offsets


def expert_slots(idx: np.ndarray, num_experts: int):
    """Permutation step: for each expert, the sorted slot ids t*k + j routed to it.

    The order of slots inside one expert's run is not fixed by the method
    (any order is a valid permutation); the set is.
    """
    flat = np.asarray(idx).reshape(-1)
    return [np.nonzero(flat == e)[0] for e in range(num_experts)]
