"""Pins for the quota-driven planner oracle (oracle/quota.py).

What the pages fix (UltraEP reading notes, section 4, Algorithm 1): a binary
search for the smallest load threshold tau that a greedy feasibility pass
meets, with excess/slack per worker, recipients that do not host the expert
yet, and a quota floor u_min below which no replica is made; the program's
constraints are those of the MegaFlux "Problem Formulation" (sum_r q_er = b_e,
at most s replicas per worker).  Checked here: hand-worked fixtures
(tests/golden/quota_cases.json), the constraints, the floor, tau bounds, the
binary search's boundary (tau - 1 fails unless tau is the lower bound), the
exact optimum as a lower bound, and special cases.
"""
import json
import os

import numpy as np
import pytest

from oracle.plan import FWD, bruteforce_optimum, objective_of
from oracle.quota import QUOTA_SEARCH_ID, feasibility_pass, quota_plan

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quota_cases.json")


def _check(b, h, P, s, u_min, out):
    q = out["q"]
    E = len(b)
    assert q.shape == (E, P) and (q >= 0).all()
    np.testing.assert_array_equal(q.sum(axis=1), b)
    np.testing.assert_array_equal(out["load"], q.sum(axis=0))
    reps = 0
    for r in range(P):
        mine = [e for e in range(E) if h[e] != r and q[e, r] > 0]
        assert len(mine) <= s
        for e in mine:
            assert q[e, r] >= u_min          # a replica carries at least the floor
        reps += len(mine)
    obj, sid, nrep, tau = (int(v) for v in out["plan_info"])
    assert sid == QUOTA_SEARCH_ID and nrep == reps
    assert obj == int(q.sum(axis=0).max()) == objective_of(q, h, FWD)
    B = sum(b)
    fixed_max = max(sum(b[e] for e in range(E) if h[e] == r) for r in range(P))
    assert obj <= tau <= fixed_max
    assert tau >= (B + P - 1) // P
    bw = out["block_worker"]
    pos = 0
    for e in range(E):
        seq = [h[e]] * q[e, h[e]] + [t for t in range(P) if t != h[e] for _ in range(q[e, t])]
        np.testing.assert_array_equal(bw[pos: pos + b[e]], seq)
        pos += b[e]
    assert pos == len(bw)


def _random_instance(rng, E, P):
    h = rng.integers(0, P, size=E)
    b = rng.integers(0, 12, size=E) * (rng.random(E) < 0.8)
    hot = rng.integers(0, E)
    b[hot] += rng.integers(0, 40)
    return b.astype(int).tolist(), h.astype(int).tolist()


def test_golden_cases():
    doc = json.load(open(GOLDEN))
    assert len(doc["cases"]) >= 6
    for c in doc["cases"]:
        out = quota_plan(c["b"], c["owner"], c["P"], c["s"], c["u_min"])
        np.testing.assert_array_equal(out["q"], c["q"], err_msg=c["name"])
        np.testing.assert_array_equal(out["load"], c["load"], err_msg=c["name"])
        np.testing.assert_array_equal(out["plan_info"], c["plan_info"], err_msg=c["name"])
        np.testing.assert_array_equal(out["block_worker"], c["block_worker"], err_msg=c["name"])
        _check(c["b"], c["owner"], c["P"], c["s"], c["u_min"], out)


@pytest.mark.parametrize("seed", range(40))
def test_invariants_random(seed):
    rng = np.random.default_rng(seed)
    P = int(rng.choice([1, 2, 4, 8]))
    E = int(rng.integers(1, 40))
    s = int(rng.integers(0, 4))
    u_min = int(rng.integers(1, 6))
    b, h = _random_instance(rng, E, P)
    out = quota_plan(b, h, P, s, u_min)
    _check(b, h, P, s, u_min, out)
    # the binary search's boundary: tau passes; tau - 1 fails unless tau is the
    # lower end of the range
    tau = int(out["plan_info"][3])
    assert feasibility_pass(b, h, P, s, u_min, tau)[0]
    if tau > (sum(b) + P - 1) // P:
        assert not feasibility_pass(b, h, P, s, u_min, tau - 1)[0]


@pytest.mark.parametrize("seed", range(12))
def test_never_beats_the_optimum(seed):
    rng = np.random.default_rng(100 + seed)
    P = int(rng.choice([2, 3]))
    E = int(rng.integers(1, 5))
    s = int(rng.integers(0, 3))
    h = rng.integers(0, P, size=E).tolist()
    b = rng.integers(0, 9, size=E).tolist()
    out = quota_plan(b, h, P, s, 1)
    assert int(out["plan_info"][0]) >= bruteforce_optimum(b, h, P, s, FWD)


def test_special_cases():
    b, h = [5, 3, 9, 1], [0, 1, 1, 0]
    one = quota_plan(b, [0] * 4, 1, 3)                     # one worker keeps everything
    assert one["plan_info"].tolist() == [18, QUOTA_SEARCH_ID, 0, 18]
    fixed = quota_plan(b, h, 2, 0)                         # no budget: fixed placement
    np.testing.assert_array_equal(fixed["q"], [[5, 0], [0, 3], [0, 9], [1, 0]])
    assert fixed["plan_info"][2] == 0
    bal = quota_plan([4, 4, 4, 4], [0, 1, 2, 3], 4, 2)     # balanced: nothing moves
    assert bal["plan_info"].tolist() == [4, QUOTA_SEARCH_ID, 0, 4]
    floor = quota_plan(b, h, 2, 3, u_min=100)              # floor above any move
    np.testing.assert_array_equal(floor["q"], fixed["q"])
    empty = quota_plan([0, 0, 0], [0, 1, 0], 2, 1)
    assert empty["plan_info"].tolist() == [0, QUOTA_SEARCH_ID, 0, 0]
    assert len(empty["block_worker"]) == 0


def test_deterministic():
    rng = np.random.default_rng(7)
    b, h = _random_instance(rng, 30, 8)
    a1, a2 = quota_plan(b, h, 8, 2, 2), quota_plan(b, h, 8, 2, 2)
    for k in a1:
        np.testing.assert_array_equal(a1[k], a2[k])


def test_bad_arguments_rejected():
    with pytest.raises(ValueError):
        quota_plan([1, 2], [0, 2], 2, 1)
    with pytest.raises(ValueError):
        quota_plan([1, 2], [0, 1], 2, -1)
    with pytest.raises(ValueError):
        quota_plan([1, 2], [0, 1], 2, 1, u_min=0)
