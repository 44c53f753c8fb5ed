"""Mutation check of the oracle pins: each planted mistake must turn a pin red.

Every mutant is planted in the oracle (on the CPU) through monkeypatch and
undone afterwards; the unmodified oracle passes all pins (test_oracle_pins).
"""
import numpy as np
import pytest

import oracle.moe_oracle as om
from oracle_checks import ALL_CHECKS


def _m1_bias_in_weights(mp):      # weights gathered from the biased scores
    mp.setattr(om, "gather_weights", lambda orig, sel, S: sel[S].copy())


def _m2_renorm_unguarded(mp):      # renormalise also when top_k == 1
    mp.setattr(om, "normalize", lambda w, k, norm: w / (w.sum() + om.RENORM_EPS) if norm else w)


def _m3_no_scaling(mp):            # routed scaling skipped
    mp.setattr(om, "scale", lambda w, rsf: w)


def _m4_neg_inf_mask(mp):          # dropped groups masked with -inf instead of zero
    mp.setattr(om, "MASK_FILL", -np.inf)


def _m5_group_max(mp):             # group score = max instead of top-2 sum
    mp.setattr(om, "group_score", lambda block: float(np.max(block)))


def _m6_weighted_shared(mp):       # shared expert weighted by a routing weight
    orig = om.combine

    def bad(terms, w_row, y_s):
        return orig(terms, w_row, None if y_s is None else w_row[0] * y_s)
    mp.setattr(om, "combine", bad)


def _m7_nibble_order(mp):          # u4: high nibble taken as the even element
    def bad(packed):
        p = np.asarray(packed)
        q = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
        q[..., 0::2] = p >> 4
        q[..., 1::2] = p & 0x0F
        return q
    mp.setattr(om, "unpack_u4", bad)


def _m8_router_bias_dropped(mp):   # the router's own bias left out of the logits
    mp.setattr(om, "router_logits", lambda x, W, b=None: om.to_f64(x) @ om.to_f64(W).T)


def _m9_sigmoid_sign(mp):          # sigmoid of -l
    orig = om.score

    def bad(l, fn):
        return 1.0 / (1.0 + np.exp(np.asarray(l, dtype=np.float64))) if fn == "sigmoid" else orig(l, fn)
    mp.setattr(om, "score", bad)


def _m10_gate_without_silu(mp):    # sigmoid(a) in place of a * sigmoid(a)
    mp.setattr(om, "silu", lambda a: 1.0 / (1.0 + np.exp(-a)))


def _m11_down_from_up(mp):         # wrong operand: the up matrix as the down projection
    def bad(X, Wg, Wu, Wd):
        h = om.silu(X @ Wg.T) * (X @ Wu.T)
        return h @ Wu if Wu.shape[::-1] == Wd.shape else h @ Wd
    mp.setattr(om, "swiglu_mlp", bad)


def _m12_zero_point_sign(mp):      # s * (q + z)
    orig = om.dequant_u8

    def bad(q, s, z, group=64):
        return orig(q, s, -om.to_f64(z), group)
    mp.setattr(om, "dequant_u8", bad)


def _m13_ties_to_higher_index(mp):  # equal selection scores: the higher expert index first
    def bad(sel, k):
        n = sel.shape[0]
        order = np.argsort(-sel[::-1], kind="stable")
        return (n - 1 - order)[:k]
    mp.setattr(om, "select_topk", bad)


def _m14_shared_dropped(mp):       # the shared expert left out of the sum
    orig = om.combine
    mp.setattr(om, "combine", lambda terms, w_row, y_s: orig(terms, w_row, None))


def _m15_worst_groups_kept(mp):    # the lowest-scoring groups kept
    orig = om.kept_groups

    def bad(sel, G, g):
        keep, sigma = orig(sel, G, G)
        return keep[G - g:], sigma
    mp.setattr(om, "kept_groups", bad)


def _m16_renorm_without_epsilon(mp):  # w / sum(w), no 1e-20
    mp.setattr(om, "normalize", lambda w, k, norm: w / w.sum() if (k > 1 and norm) else w)


def _m17_softmax_over_tokens(mp):  # softmax taken over the wrong axis
    orig = om.score

    def bad(l, fn):
        if fn != "softmax":
            return orig(l, fn)
        a = np.asarray(l, dtype=np.float64)
        p = np.exp(a - a.max(axis=0, keepdims=True))
        return p / p.sum(axis=0, keepdims=True)
    mp.setattr(om, "score", bad)


def _m18_route_bias_arguments_swapped(mp):  # router bias taken as the correction bias and back
    orig = om.route

    def bad(x, W_r, cfg, router_bias=None, expert_bias=None, tokens=None):
        return orig(x, W_r, cfg, router_bias=expert_bias, expert_bias=router_bias, tokens=tokens)
    mp.setattr(om, "route", bad)


def _m19_route_tokens_off_by_one(mp):  # the tokens= subset shifted by one row
    orig = om.route

    def bad(x, W_r, cfg, router_bias=None, expert_bias=None, tokens=None):
        if tokens is not None:
            tokens = (np.asarray(tokens) + 1) % np.asarray(x).shape[0]
        return orig(x, W_r, cfg, router_bias=router_bias, expert_bias=expert_bias, tokens=tokens)
    mp.setattr(om, "route", bad)


def _m20_gate_reads_up_scale(mp):  # u8 gate codes dequantised with the up matrix's scales
    orig = om.expert_matrix

    def bad(weights, name, e, group):
        if name == "gate" and "gate_q" in weights:
            weights = dict(weights, gate_scale=weights["up_scale"])
        return orig(weights, name, e, group)
    mp.setattr(om, "expert_matrix", bad)


MUTANTS = [_m1_bias_in_weights, _m2_renorm_unguarded, _m3_no_scaling, _m4_neg_inf_mask,
           _m5_group_max, _m6_weighted_shared, _m7_nibble_order, _m8_router_bias_dropped,
           _m9_sigmoid_sign, _m10_gate_without_silu, _m11_down_from_up, _m12_zero_point_sign,
           _m13_ties_to_higher_index, _m14_shared_dropped, _m15_worst_groups_kept,
           _m16_renorm_without_epsilon, _m17_softmax_over_tokens, _m18_route_bias_arguments_swapped,
           _m19_route_tokens_off_by_one, _m20_gate_reads_up_scale]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__)
def test_mutant_is_caught(mutant, monkeypatch):
    mutant(monkeypatch)
    failed = []
    for check in ALL_CHECKS:
        try:
            if check.__name__ == "check_bruteforce":
                check(om, cases=600)
            else:
                check(om)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"{mutant.__name__} passed every pin"
