"""Pins for the replication gate oracle (oracle/gate.py).

The rule is a definition (keep the plan when 1000 * (fixed objective - plan
objective) > rho_milli * replicas, else fixed placement), so the pins check
it on hand-computed cases on both sides of the threshold, on the boundary
(equality falls to fixed placement), plans without replicas, rho = 0, and
that the fixed placement it returns is exactly the owner placement produced
by the planners with s = 0.
"""
import numpy as np
import pytest

from oracle.gate import GATED_SEARCH_ID, gate
from oracle.plan import FWD, plan
from oracle.quota import quota_plan


def test_hand_cases():
    # b=[6,2] on worker 0 of 2: fixed objective 8; greedy: one replica, objective 5
    b, h = [6, 2, 1, 1], [0, 0, 1, 1]
    p = plan(b, h, 2, 1, FWD)
    assert p["plan_info"].tolist()[0] == 5 and p["plan_info"][2] == 1
    # saving 8 - 5 = 3 blocks: kept while rho < 3 blocks per replica
    kept = gate(p, b, h, 2, 2999)
    np.testing.assert_array_equal(kept["q"], p["q"])
    fixed = gate(p, b, h, 2, 3000)                     # equality: not a saving
    np.testing.assert_array_equal(fixed["q"], [[6, 0], [2, 0], [0, 1], [0, 1]])
    np.testing.assert_array_equal(fixed["load"], [8, 2])
    np.testing.assert_array_equal(fixed["block_worker"], [0] * 8 + [1, 1])
    assert fixed["plan_info"].tolist() == [8, GATED_SEARCH_ID, 0, p["plan_info"][3]]


def test_plan_without_replicas_is_kept():
    b, h = [4, 4, 4, 4], [0, 1, 2, 3]
    p = plan(b, h, 4, 2, FWD)
    assert p["plan_info"][2] == 0
    g = gate(p, b, h, 4, 10 ** 6)
    for k in p:
        np.testing.assert_array_equal(g[k], p[k])


@pytest.mark.parametrize("seed", range(20))
def test_fixed_branch_equals_zero_budget_plan(seed):
    rng = np.random.default_rng(seed)
    P = int(rng.choice([2, 4, 8]))
    E = int(rng.integers(2, 30))
    h = rng.integers(0, P, size=E).tolist()
    b = (rng.integers(0, 10, size=E) + (rng.random(E) < 0.2) * 30).tolist()
    p = quota_plan(b, h, P, 2, 1)
    g = gate(p, b, h, P, 10 ** 9)                     # a price no saving beats
    z = plan(b, h, P, 0, FWD)                          # the planner with no budget
    np.testing.assert_array_equal(g["q"], z["q"])
    np.testing.assert_array_equal(g["load"], z["load"])
    np.testing.assert_array_equal(g["block_worker"], z["block_worker"])
    if p["plan_info"][2] > 0:
        assert g["plan_info"][1] == GATED_SEARCH_ID and g["plan_info"][2] == 0
    g0 = gate(p, b, h, P, 0)                           # free replicas: kept iff it saves
    saves = int(np.asarray(z["load"]).max()) > int(p["load"].max())
    assert np.array_equal(g0["q"], p["q"]) == (saves or p["plan_info"][2] == 0)


def test_negative_price_rejected():
    with pytest.raises(ValueError):
        gate(plan([1], [0], 1, 0), [1], [0], 1, -1)
