"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each check takes the oracle module and raises AssertionError when it fails.
They are collected by test_oracle_pins.py, and re-run by
test_oracle_mutants.py against oracles with one planted mistake each (every
planted mistake must make at least one check fail).

Kinds of pin used: closed forms, a hand-computed example (golden file),
brute-force enumeration of routing decisions on tiny inputs, special cases
that reduce to library routines (torch), and invariants of the definition.
"""

from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _cfg(om, **kw):
    base = dict(hidden=2, num_experts=4, top_k=2, moe_intermediate=1)
    base.update(kw)
    return om.OracleConfig(**base)


def _logit(p):
    return math.log(p / (1.0 - p))


# ---------------------------------------------------------------- P1 logits
def check_logits(om):
    rng = np.random.default_rng(11)
    W = rng.standard_normal((5, 7))
    for h in range(7):
        x = np.zeros((1, 7))
        x[0, h] = 1.0
        l = om.router_logits(x, W)
        assert np.array_equal(l[0], W[:, h]), "one-hot x must return a router column"
    x = rng.standard_normal((3, 7))
    b = rng.standard_normal(5)
    l = om.router_logits(x, W, b)
    for t in range(3):
        for e in range(5):
            acc = math.fsum(x[t, h] * W[e, h] for h in range(7)) + b[e]
            assert abs(l[t, e] - acc) < 1e-12


# ---------------------------------------------------------------- P2 scores
def check_scores(om):
    s = om.score(np.array([[math.log(3), 0.0, -math.log(3)]]), "sigmoid")[0]
    assert np.allclose(s, [0.75, 0.5, 0.25], atol=1e-15, rtol=0)
    s = om.score(np.array([[0.0, math.log(2), math.log(3)]]), "softmax")[0]
    assert np.allclose(s, [1 / 6, 2 / 6, 3 / 6], atol=1e-15, rtol=0)
    rng = np.random.default_rng(5)
    l = rng.standard_normal((4, 9)) * 3
    a = om.score(l, "softmax")
    assert np.allclose(a.sum(axis=1), 1.0, atol=1e-14)
    assert np.allclose(om.score(l + 17.25, "softmax"), a, atol=1e-14)
    try:
        om.score(l, "relu")
    except ValueError:
        pass
    else:
        raise AssertionError("unknown score function must be rejected")


# ------------------------------------------------- P3 plain top-k (n_group=1)
def check_plain_topk(om):
    import torch
    rng = np.random.default_rng(7)
    for trial in range(200):
        E = int(rng.integers(2, 40))
        k = int(rng.integers(1, E + 1))
        l = rng.standard_normal(E) * 2
        cfg = _cfg(om, num_experts=E, top_k=k, score_function="softmax" if trial % 2 else "sigmoid")
        r = om.route_token(l, cfg)
        ref = torch.topk(torch.tensor(l, dtype=torch.float64), k).indices.numpy()
        assert set(r.idx.tolist()) == set(ref.tolist()), "n_group=1 must be plain top-k"
        py = sorted(range(E), key=lambda e: (-l[e], e))[:k]
        assert r.idx.tolist() == py, "order: descending score, ties to the lower index"
    # exact ties (a reading, R4: the pages' argpartition leaves their order open):
    # equal scores go to the lower expert index
    l = np.array([0.5, 2.0, 2.0, -1.0, 2.0, 2.0])
    for k, want in ((1, [1]), (2, [1, 2]), (3, [1, 2, 4]), (5, [1, 2, 4, 5, 0])):
        for fn in ("sigmoid", "softmax"):
            r = om.route_token(l, _cfg(om, num_experts=6, top_k=k, score_function=fn))
            assert r.idx.tolist() == want, f"ties to the lower index ({fn}, k={k})"


# ------------------------------------------------ P4 brute-force enumeration
def _brute_route(sel, E, G, g, k):
    """Maximise sums over subsets: kept groups, then the best k-subset."""
    if G > 1 and g < G:
        gs = E // G
        sig = []
        for q in range(G):
            blk = sel[q * gs:(q + 1) * gs]
            sig.append(max(blk[a] + blk[b] for a, b in itertools.combinations(range(gs), 2)))
        best = None
        for keep in itertools.combinations(range(G), g):
            v = sum(sig[q] for q in keep)
            if best is None or v > best[0] + 1e-12:
                best = (v, keep, False)
            elif abs(v - best[0]) <= 1e-12:
                best = (best[0], best[1], True)
        keep = best[1]
        masked = np.zeros(E)
        for q in keep:
            masked[q * gs:(q + 1) * gs] = sel[q * gs:(q + 1) * gs]
        group_tie = best[2]
    else:
        masked, group_tie = sel.copy(), False
    combos = _combos(E, k)
    sums = masked[combos].sum(axis=1)
    top = sums.max()
    winners = [set(c.tolist()) for c in combos[np.abs(sums - top) <= 1e-12]]
    return winners, group_tie


_COMBOS = {}


def _combos(E, k):
    if (E, k) not in _COMBOS:
        _COMBOS[(E, k)] = np.array(list(itertools.combinations(range(E), k)), dtype=np.int64)
    return _COMBOS[(E, k)]


def check_bruteforce(om, cases=10000, seed=3):
    rng = np.random.default_rng(seed)
    shapes = [(E, G) for E in range(2, 13) for G in (1, 2, 3, 4, 6) if E % G == 0 and E // G >= 2]
    shapes += [(E, 1) for E in range(2, 13)]
    checked = 0
    for _ in range(cases):
        E, G = shapes[int(rng.integers(len(shapes)))]
        g = int(rng.integers(1, G + 1))
        kmax = g * (E // G) if G > 1 else E
        k = int(rng.integers(1, kmax + 1))
        sf = "sigmoid" if rng.random() < 0.5 else "softmax"
        bias = rng.random() < 0.5
        l = rng.standard_normal(E) * 1.5
        beta = rng.standard_normal(E) * 0.2
        cfg = _cfg(om, num_experts=E, top_k=k, n_group=G, topk_group=g, score_function=sf,
                   use_expert_bias=bias, norm_topk_prob=False)
        r = om.route_token(l, cfg, beta if bias else None)
        s = 1 / (1 + np.exp(-l)) if sf == "sigmoid" else np.exp(l) / np.exp(l).sum()
        sel = s + beta if bias else s
        winners, gtie = _brute_route(sel, E, G, g, k)
        if gtie:
            continue
        assert set(r.idx.tolist()) in winners, f"E={E} G={G} g={g} k={k}: {r.idx} not optimal"
        assert np.allclose(r.w, s[r.idx], atol=1e-15, rtol=0)
        checked += 1
    assert checked > cases * 0.9


# --------------------------------------------------- P5 bias semantics
def check_bias_semantics(om):
    rng = np.random.default_rng(9)
    for _ in range(200):
        E = int(rng.integers(4, 30))
        k = int(rng.integers(1, E))
        l = rng.standard_normal(E)
        beta = rng.standard_normal(E) * 0.3
        cfg = _cfg(om, num_experts=E, top_k=k, score_function="sigmoid", use_expert_bias=True,
                   norm_topk_prob=False)
        r = om.route_token(l, cfg, beta)
        s = 1 / (1 + np.exp(-l))
        py = sorted(range(E), key=lambda e: (-(s[e] + beta[e]), e))[:k]
        assert r.idx.tolist() == py, "selection must use the biased scores"
        assert np.array_equal(r.w, s[py]), "weights must be the unbiased scores"


# --------------------------------------------- P6 group score = top-2 sum
def check_group_score_reading(om):
    p = [0.9, 0.1, 0.1, 0.55, 0.5, 0.02]
    l = np.array([_logit(v) for v in p])
    cfg = _cfg(om, num_experts=6, top_k=1, n_group=2, topk_group=1, score_function="sigmoid")
    r = om.route_token(l, cfg)
    # top-2 sums: 1.0 vs 1.05 -> group 1; max (0.9 vs 0.55) or full sum (1.1 vs 1.07)
    # would keep group 0 and pick expert 0
    assert r.idx.tolist() == [3]


# ------------------------------------------------------ P7 literal zero mask
def check_zero_mask(om):
    cfg = _cfg(om, num_experts=4, top_k=2, n_group=2, topk_group=1, score_function="softmax",
               use_expert_bias=True)
    r = om.route_token(np.zeros(4), cfg, np.array([-0.5, -0.5, -0.9, -0.9]))
    # sel = [-0.25,-0.25,-0.65,-0.65]; group 0 kept; dropped group zeroed to 0 > -0.25
    assert sorted(r.idx.tolist()) == [2, 3]
    assert r.masked_pick


# ------------------------------------------------ P8 renormalise and scale
def check_renorm_scale(om):
    rng = np.random.default_rng(13)
    for _ in range(100):
        E = int(rng.integers(3, 20))
        k = int(rng.integers(2, E))
        rsf = float(rng.uniform(0.5, 3.0))
        l = rng.standard_normal(E)
        base = dict(num_experts=E, top_k=k, score_function="sigmoid")
        r1 = om.route_token(l, _cfg(om, routed_scaling_factor=1.0, **base))
        r2 = om.route_token(l, _cfg(om, routed_scaling_factor=rsf, **base))
        raw = 1 / (1 + np.exp(-l[r1.idx]))
        assert abs(r1.w.sum() - raw.sum() / (raw.sum() + 1e-20)) < 1e-14
        assert np.allclose(r2.w, rsf * r1.w, rtol=1e-14, atol=0), "routed scaling is linear"
        rn = om.route_token(l, _cfg(om, routed_scaling_factor=rsf, norm_topk_prob=False, **base))
        assert np.allclose(rn.w, rsf * raw, rtol=1e-14, atol=0)
    # top_k == 1: no renormalisation, the weight is the raw score times the factor
    l = np.array([0.3, -1.0, 2.0])
    r = om.route_token(l, _cfg(om, num_experts=3, top_k=1, score_function="sigmoid",
                               routed_scaling_factor=2.5))
    assert r.idx.tolist() == [2]
    assert abs(r.w[0] - 2.5 / (1 + math.exp(-2.0))) < 1e-15
    # the 1e-20 epsilon: softmax scores are never all zero, so check the formula on tiny scores
    w = om.normalize(np.array([1e-21, 1e-21]), 2, True)
    assert abs(w[0] - 1e-21 / (2e-21 + 1e-20)) < 1e-30


# --------------------------------------------------------- P9 SwiGLU
def check_swiglu(om):
    import torch
    rng = np.random.default_rng(17)
    a = rng.standard_normal(50) * 4
    ref = torch.nn.functional.silu(torch.tensor(a, dtype=torch.float64)).numpy()
    assert np.allclose(om.silu(a), ref, rtol=1e-14, atol=1e-15)
    X = rng.standard_normal((3, 5))
    Wg, Wu, Wd = rng.standard_normal((4, 5)), rng.standard_normal((4, 5)), rng.standard_normal((5, 4))
    y = om.swiglu_mlp(X, Wg, Wu, Wd)
    for t in range(3):
        h = []
        for i in range(4):
            g = math.fsum(Wg[i, c] * X[t, c] for c in range(5))
            u = math.fsum(Wu[i, c] * X[t, c] for c in range(5))
            h.append(g / (1 + math.exp(-g)) * u)
        for o in range(5):
            assert abs(y[t, o] - math.fsum(Wd[o, i] * h[i] for i in range(4))) < 1e-12


# ------------------------------------------------- P10 hand-computed example
def hand_example_inputs():
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        gold = json.load(f)
    ln3 = math.log(3.0)
    W = dict(
        router=np.array(gold["inputs"]["router_ln3_coeffs"], dtype=np.float64) * ln3,
        router_bias=None,
        expert_bias=np.array(gold["inputs"]["expert_bias"]),
        gate=np.ones((4, 1, 2)),
        up=np.array([[[e + 1.0, -(e + 1.0)]] for e in range(4)]),
        down=np.array([[[1.0], [-1.0]]] * 4),
        shared_gate=np.array(gold["inputs"]["shared_gate"], dtype=np.float64),
        shared_up=np.array(gold["inputs"]["shared_up"], dtype=np.float64),
        shared_down=np.array(gold["inputs"]["shared_down"], dtype=np.float64),
    )
    return gold, np.array(gold["inputs"]["x"]), W


def check_hand_example(om):
    gold, x, W = hand_example_inputs()
    cfg = om.OracleConfig(**gold["config"])
    y, d = om.forward(x, W, cfg)
    exp = gold["expected"]
    tol = exp["tolerance"]
    assert np.allclose(y, exp["y"], atol=tol, rtol=0), (y, exp["y"])
    s1 = exp["silu_1"]
    assert np.allclose(y, [[s1 * 28 / 3, -s1 * 22 / 3], [-3 * s1, 5 * s1]], atol=tol, rtol=0)
    assert d["idx"].tolist() == exp["idx"]
    assert np.allclose(d["w"], exp["w"], atol=tol, rtol=0)
    assert np.allclose(d["margin"], exp["margin"], atol=tol, rtol=0)


# ------------------------------------------------ P11 dense mixture closed form
def check_dense_mixture(om):
    rng = np.random.default_rng(19)
    E, H, I, Is = 5, 6, 3, 4
    cfg = om.OracleConfig(hidden=H, num_experts=E, top_k=E, moe_intermediate=I,
                          shared_intermediate=Is, routed_scaling_factor=1.7)
    W = dict(router=rng.standard_normal((E, H)), router_bias=None, expert_bias=None,
             gate=rng.standard_normal((E, I, H)), up=rng.standard_normal((E, I, H)),
             down=rng.standard_normal((E, H, I)), shared_gate=rng.standard_normal((Is, H)),
             shared_up=rng.standard_normal((Is, H)), shared_down=rng.standard_normal((H, Is)))
    x = rng.standard_normal((3, H))
    y, _ = om.forward(x, W, cfg)

    def mlp(xv, g, u, dn):
        gg, uu = g @ xv, u @ xv
        return dn @ (gg / (1 + np.exp(-gg)) * uu)
    for t in range(3):
        l = W["router"] @ x[t]
        s = np.exp(l - l.max())
        s /= s.sum()
        ref = sum(s[e] * 1.7 * mlp(x[t], W["gate"][e], W["up"][e], W["down"][e]) for e in range(E))
        ref = ref + mlp(x[t], W["shared_gate"], W["shared_up"], W["shared_down"])
        assert np.allclose(y[t], ref, rtol=1e-12, atol=1e-12)
    # identical experts: the mixture collapses to RSF * expert(x) + shared(x)
    for key in ("gate", "up", "down"):
        W[key] = np.repeat(W[key][:1], E, axis=0)
    cfg2 = om.OracleConfig(hidden=H, num_experts=E, top_k=2, moe_intermediate=I,
                           shared_intermediate=Is, routed_scaling_factor=1.7)
    y2, _ = om.forward(x, W, cfg2)
    for t in range(3):
        ref = 1.7 * mlp(x[t], W["gate"][0], W["up"][0], W["down"][0]) + \
            mlp(x[t], W["shared_gate"], W["shared_up"], W["shared_down"])
        assert np.allclose(y2[t], ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------ P12 combine invariants
def _rand_layer(rng, E=6, H=8, I=4, Is=5):
    return dict(router=rng.standard_normal((E, H)), router_bias=None, expert_bias=None,
                gate=rng.standard_normal((E, I, H)), up=rng.standard_normal((E, I, H)),
                down=rng.standard_normal((E, H, I)), shared_gate=rng.standard_normal((Is, H)),
                shared_up=rng.standard_normal((Is, H)), shared_down=rng.standard_normal((H, Is)))


def check_combine_invariants(om):
    rng = np.random.default_rng(23)
    E, H, I, Is = 6, 8, 4, 5
    W = _rand_layer(rng, E, H, I, Is)
    cfg = om.OracleConfig(hidden=H, num_experts=E, top_k=3, moe_intermediate=I,
                          shared_intermediate=Is, routed_scaling_factor=1.3)
    x = rng.standard_normal((7, H))
    y, d = om.forward(x, W, cfg)
    # zero routed down projections -> only the shared expert remains, at weight 1.0
    Wz = dict(W, down=np.zeros_like(W["down"]))
    yz, _ = om.forward(x, Wz, cfg)
    ys = np.stack([W["shared_down"] @ (om.silu(W["shared_gate"] @ x[t]) * (W["shared_up"] @ x[t]))
                   for t in range(7)])
    assert np.allclose(yz, ys, rtol=1e-13, atol=1e-13)
    # no shared expert -> routed mixture only
    cfg0 = om.OracleConfig(hidden=H, num_experts=E, top_k=3, moe_intermediate=I,
                           shared_intermediate=0, routed_scaling_factor=1.3)
    y0, _ = om.forward(x, dict(W, shared_gate=None, shared_up=None, shared_down=None), cfg0)
    assert np.allclose(y0 + ys, y, rtol=1e-12, atol=1e-12)
    # permuting tokens permutes outputs; each row equals its single-token result
    perm = rng.permutation(7)
    yp, _ = om.forward(x[perm], W, cfg)
    assert np.allclose(yp, y[perm], rtol=1e-13, atol=1e-13)
    for t in (0, 4):
        y1, _ = om.forward(x[t:t + 1], W, cfg)
        assert np.allclose(y1[0], y[t], rtol=1e-13, atol=1e-13)
    # the tokens= subset selects rows
    ysub, _ = om.forward(x, W, cfg, tokens=[5, 2])
    assert np.allclose(ysub, y[[5, 2]], rtol=1e-13, atol=1e-13)
    # forced routing with the oracle's own sets reproduces the same outputs
    yf, _ = om.forward(x, W, cfg, forced_idx=d["idx"])
    assert np.allclose(yf, y, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------- P13 u8 dequant
def check_dequant(om):
    rng = np.random.default_rng(29)
    q = rng.integers(0, 256, size=(3, 128)).astype(np.uint8)
    s = (rng.random((3, 2)) * 0.01 + 1e-4).astype(np.float16)
    z = rng.integers(0, 256, size=(3, 2)).astype(np.float16)
    w = om.dequant_u8(q, s, z, 64)
    for r in range(3):
        for c in range(128):
            ref = float(s[r, c // 64]) * (int(q[r, c]) - float(z[r, c // 64]))
            assert w[r, c] == ref, "s*(q-z) is exact in fp64"
    # bf16 bit patterns decode exactly
    bits = np.array([0x3F80, 0xC000, 0x3E80, 0x0000], dtype=np.uint16)
    assert om.to_f64(bits).tolist() == [1.0, -2.0, 0.25, 0.0]


# ------------------------------------------------------------- P14 u4 dequant
def check_dequant_u4(om):
    import synth
    # hand-decoded bytes: 0x21 -> codes 1 (low nibble, element 0), 2 (element 1);
    # 0xF0 -> 0, 15.  Group of 4, s = 0.5, z = 1: w = 0.5 * (q - 1)
    p = np.array([[0x21, 0xF0]], dtype=np.uint8)
    w = om.dequant_u4(p, np.array([[0.5]], dtype=np.float16), np.array([[1.0]], dtype=np.float16), 4)
    assert w.tolist() == [[0.0, 0.5, -0.5, 7.0]]
    # packing written out here independently: equals the u8 definition on the codes
    rng = np.random.default_rng(31)
    q = rng.integers(0, 16, size=(3, 128)).astype(np.uint8)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    s = (rng.random((3, 2)) * 0.01 + 1e-4).astype(np.float16)
    z = rng.integers(0, 16, size=(3, 2)).astype(np.float16)
    assert np.array_equal(om.dequant_u4(packed, s, z, 64), om.dequant_u8(q, s, z, 64))
    # the synthetic encoder's codes decode to within half a step of the input
    wv = rng.standard_normal((4, 256)).astype(np.float32) * 0.02
    pk, sc, zp = synth.quantize_u4(wv, 64)
    err = np.abs(om.dequant_u4(pk, sc, zp, 64) - wv.astype(np.float64)).reshape(4, 4, 64)
    assert (err <= sc.astype(np.float64)[..., None] * 0.5 * (1 + 1e-6)).all()
    # a routed expert stored packed is read through the u4 decoder
    W = {"gate_q4": pk[None], "gate_scale": sc[None], "gate_zero": zp[None]}
    assert np.array_equal(om.expert_matrix(W, "gate", 0, 64), om.dequant_u4(pk, sc, zp, 64))


# ------------------------------------------- P15 the batch router route()
def _route_by_definition(x, W, b_r, beta, cfg):
    """One token's routing written out from the definition: fsum logits (plus the
    router bias), the score function, the biased copy for selection, the kept groups
    and the selected set by enumeration of subsets, weights from the unbiased scores
    renormalised and scaled, and the decision margin."""
    E, H = W.shape
    l = np.array([math.fsum(x[h] * W[e, h] for h in range(H)) + (b_r[e] if b_r is not None else 0.0)
                  for e in range(E)])
    if cfg.score_function == "sigmoid":
        s = np.array([1.0 / (1.0 + math.exp(-v)) for v in l])
    else:
        m = max(l)
        ex = [math.exp(v - m) for v in l]
        tot = math.fsum(ex)
        s = np.array([v / tot for v in ex])
    sel = s + beta if cfg.use_expert_bias else s.copy()
    G, g, k = cfg.n_group, cfg.topk_group, cfg.top_k
    winners, gtie = _brute_route(sel, E, G, g, k)
    margin = math.inf
    masked = sel.copy()
    if G > 1 and g < G:
        gs = E // G
        sig = sorted((max(sel[q * gs + a] + sel[q * gs + b]
                          for a, b in itertools.combinations(range(gs), 2)) for q in range(G)), reverse=True)
        margin = sig[g - 1] - sig[g]
        # the kept groups are the ones holding the winning set's best pair sums; rebuild
        # the masked scores from the g largest group scores (no ties on random inputs)
        best = sorted(range(G), key=lambda q: -max(sel[q * gs + a] + sel[q * gs + b]
                                                   for a, b in itertools.combinations(range(gs), 2)))[:g]
        masked = np.zeros(E)
        for q in best:
            masked[q * gs:(q + 1) * gs] = sel[q * gs:(q + 1) * gs]
    if k < E:
        srt = sorted(masked, reverse=True)
        margin = min(margin, srt[k - 1] - srt[k])
    return s, winners, gtie, margin


def check_route(om):
    """route() -- the batch entry every GPU routing comparison is checked against --
    equals routing written out from the definition on random layers (router bias,
    correction bias, groups, both score functions), its tokens= subset selects the
    same rows, and it agrees with forward()'s routing."""
    rng = np.random.default_rng(37)
    cases = [
        dict(E=12, H=6, G=3, g=2, k=3, sf="sigmoid", bias=True, rsf=2.5, rb=True),
        dict(E=10, H=5, G=1, g=1, k=4, sf="softmax", bias=False, rsf=1.0, rb=True),
        dict(E=8, H=7, G=4, g=2, k=2, sf="softmax", bias=True, rsf=1.7, rb=False),
    ]
    for c in cases:
        E, H, T = c["E"], c["H"], 9
        W = rng.standard_normal((E, H))
        b_r = rng.standard_normal(E) * 0.5 if c["rb"] else None
        beta = rng.standard_normal(E) * 0.3
        x = rng.standard_normal((T, H))
        cfg = om.OracleConfig(hidden=H, num_experts=E, top_k=c["k"], moe_intermediate=1, n_group=c["G"],
                              topk_group=c["g"], score_function=c["sf"], use_expert_bias=c["bias"],
                              routed_scaling_factor=c["rsf"])
        eb = beta if c["bias"] else None
        idx, w, margin, masked = om.route(x, W, cfg, router_bias=b_r, expert_bias=eb)
        assert idx.shape == (T, c["k"]) and w.shape == (T, c["k"])
        for t in range(T):
            s, winners, gtie, mg = _route_by_definition(x[t], W, b_r, beta, cfg)
            assert not gtie
            assert set(idx[t].tolist()) in winners, f"route(): token {t} set {idx[t]} not optimal"
            raw = s[idx[t]]
            want = c["rsf"] * raw / (raw.sum() + 1e-20)
            assert np.allclose(w[t], want, rtol=1e-13, atol=0), "route(): weights"
            assert abs(margin[t] - mg) <= 1e-13, f"route(): margin {margin[t]} vs {mg}"
        sub = [7, 0, 4, 4]
        i2, w2, m2, k2 = om.route(x, W, cfg, router_bias=b_r, expert_bias=eb, tokens=sub)
        assert np.array_equal(i2, idx[sub]) and np.array_equal(w2, w[sub]) and np.array_equal(m2, margin[sub])
        Wl = dict(router=W, router_bias=b_r, expert_bias=eb, gate=np.zeros((E, 1, H)), up=np.zeros((E, 1, H)),
                  down=np.zeros((E, H, 1)))
        _, d = om.forward(x, Wl, cfg, tokens=sub)
        assert np.array_equal(d["idx"], i2) and np.allclose(d["w"], w2, rtol=1e-15, atol=0)
    # the expert bias is refused when enabled but missing
    try:
        om.route(x, W, om.OracleConfig(hidden=H, num_experts=E, top_k=2, moe_intermediate=1,
                                       use_expert_bias=True))
    except ValueError:
        pass
    else:
        raise AssertionError("route(): a missing correction bias must be rejected")


# ------------------------------------------- P16 u8 routed experts in forward()
def check_u8_layer(om):
    """forward() on a layer whose routed experts are stored u8 (code, fp16 scale and
    fp16 zero point per 64 elements of each row's reduction axis) equals forward() on
    the same layer stored as the values s * (q - z), expanded here group by group.
    Every matrix has its own scale and zero-point arrays, so reading one matrix's
    parameters for another changes the result."""
    rng = np.random.default_rng(41)
    E, H, I, Is, T = 4, 128, 64, 64, 6
    shapes = dict(gate=(E, I, H), up=(E, I, H), down=(E, H, I))
    Wq, Wf = {}, {}
    for n, shp in shapes.items():
        q = rng.integers(0, 256, size=shp).astype(np.uint8)
        sc = (rng.random(shp[:-1] + (shp[-1] // 64,)) * 0.002 + 1e-4).astype(np.float16)
        zp = rng.integers(0, 256, size=sc.shape).astype(np.float16)
        Wq[n + "_q"], Wq[n + "_scale"], Wq[n + "_zero"] = q, sc, zp
        full = np.empty(shp)
        for gi in range(shp[-1] // 64):
            cols = slice(64 * gi, 64 * gi + 64)
            full[..., cols] = sc[..., gi:gi + 1].astype(np.float64) * (
                q[..., cols].astype(np.float64) - zp[..., gi:gi + 1].astype(np.float64))
        Wf[n] = full
    common = dict(router=rng.standard_normal((E, H)), router_bias=None, expert_bias=None,
                  shared_gate=rng.standard_normal((Is, H)) * 0.1, shared_up=rng.standard_normal((Is, H)) * 0.1,
                  shared_down=rng.standard_normal((H, Is)) * 0.1)
    Wq.update(common)
    Wf.update(common)
    cfg = om.OracleConfig(hidden=H, num_experts=E, top_k=2, moe_intermediate=I, shared_intermediate=Is,
                          quant_group=64)
    x = rng.standard_normal((T, H))
    yq, dq = om.forward(x, Wq, cfg)
    yf, df = om.forward(x, Wf, cfg)
    assert np.array_equal(dq["idx"], df["idx"])
    assert np.allclose(yq, yf, rtol=1e-12, atol=1e-12), "u8 experts must read as s * (q - z)"
    assert np.abs(yq).max() > 1e-3
    for n in shapes:
        assert np.array_equal(om.expert_matrix(Wq, n, 1, 64), Wf[n][1])


ALL_CHECKS = [check_logits, check_scores, check_plain_topk, check_bruteforce,
              check_bias_semantics, check_group_score_reading, check_zero_mask,
              check_renorm_scale, check_swiglu, check_hand_example, check_dense_mixture,
              check_combine_invariants, check_dequant, check_dequant_u4, check_route,
              check_u8_layer]
