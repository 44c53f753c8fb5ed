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


MUTANTS = [_m1_bias_in_weights, _m2_renorm_unguarded, _m3_no_scaling, _m4_neg_inf_mask,
           _m5_group_max, _m6_weighted_shared, _m7_nibble_order]


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
