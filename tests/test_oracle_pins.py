"""The fp64 oracle against its pins (closed forms, brute force, hand example, invariants)."""
import pytest

import oracle.moe_oracle as om
from oracle_checks import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(om)


def test_margin_and_masked_pick_diagnostics():
    import numpy as np
    cfg = om.OracleConfig(hidden=1, num_experts=4, top_k=2, moe_intermediate=1)
    r = om.route_token(np.log(np.array([4.0, 3.0, 2.0, 1.0])), cfg)
    # softmax scores 0.4, 0.3, 0.2, 0.1: margin between 2nd and 3rd = 0.1
    assert abs(r.margin - 0.1) < 1e-14 and not r.masked_pick
    cfg_all = om.OracleConfig(hidden=1, num_experts=4, top_k=4, moe_intermediate=1)
    assert om.route_token(np.zeros(4), cfg_all).margin == float("inf")


def test_permutation_oracle():
    import numpy as np
    idx = np.array([[2, 0], [2, 1], [0, 2]])
    counts, offsets = om.expert_counts(idx, 4)
    assert counts.tolist() == [2, 1, 3, 0] and offsets.tolist() == [0, 2, 3, 6, 6]
    slots = om.expert_slots(idx, 4)
    assert [s.tolist() for s in slots] == [[1, 4], [3], [0, 2, 5], []]
