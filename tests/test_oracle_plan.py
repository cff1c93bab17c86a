"""Pins for the planner oracle (oracle/plan.py).

What the pages fix (MegaFlux summary, "Problem Formulation" and "Bounded
Greedy Search"): the constraints sum_r q_er = b_e and at most s non-home
experts per worker, tau = ceil(sum b / P), the objective max_r l_r (and
max_r (l_r + lambda n_r) for backward).  Checked here: the constraints,
max load >= tau, never worse than fixed placement, special cases (P = 1,
s = 0, already balanced), an exact optimum that bounds the greedy (itself
checked against exhaustive enumeration), and hand-worked fixtures
(tests/golden/plan_cases.json) that pin the documented search order.
"""
import json
import os

import numpy as np
import pytest

from oracle.plan import (BWD, FWD, bruteforce_optimum, enumerate_optimum, objective_of,
                         plan)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "plan_cases.json")


def _check_invariants(b, h, P, s, mode, lam, out):
    q = out["q"]
    E = len(b)
    assert q.shape == (E, P) and (q >= 0).all()
    np.testing.assert_array_equal(q.sum(axis=1), b)
    for r in range(P):
        assert sum(1 for e in range(E) if h[e] != r and q[e, r] > 0) <= s
    np.testing.assert_array_equal(out["load"], q.sum(axis=0))
    tau = (sum(b) + P - 1) // P
    assert out["plan_info"][3] == tau
    assert q.sum(axis=0).max() >= tau
    fixed = np.zeros_like(q)
    fixed[np.arange(E), h] = b
    obj = objective_of(q, h, mode, lam)
    assert obj == out["plan_info"][0]
    assert obj <= objective_of(fixed, h, mode, lam)
    reps = sum(1 for e in range(E) for r in range(P) if h[e] != r and q[e, r] > 0)
    assert reps == out["plan_info"][2]
    # owner-first contiguous expansion of q into per-block workers
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


@pytest.mark.parametrize("mode", [FWD, BWD])
def test_invariants_random(mode):
    rng = np.random.default_rng(11 + mode)
    for _ in range(150):
        E = int(rng.integers(1, 24))
        P = int(rng.choice([1, 2, 3, 4, 8]))
        s = int(rng.integers(0, 4))
        lam = int(rng.integers(0, 15))
        b, h = _random_instance(rng, E, P)
        _check_invariants(b, h, P, s, mode, lam, plan(b, h, P, s, mode, lam))


def test_single_worker_keeps_everything():
    b = [5, 0, 7, 1]
    out = plan(b, [0, 0, 0, 0], 1, 3)
    np.testing.assert_array_equal(out["q"][:, 0], b)
    assert out["plan_info"][2] == 0


@pytest.mark.parametrize("mode", [FWD, BWD])
def test_zero_budget_is_fixed_placement(mode):
    rng = np.random.default_rng(5)
    for _ in range(30):
        b, h = _random_instance(rng, 12, 4)
        out = plan(b, h, 4, 0, mode)
        fixed = np.zeros((12, 4), dtype=int)
        fixed[np.arange(12), h] = b
        np.testing.assert_array_equal(out["q"], fixed)


def test_balanced_needs_no_replicas():
    # every worker already at or below tau
    b = [3, 2, 5, 4, 1, 4]
    h = [0, 0, 1, 2, 2, 3]
    out = plan(b, h, 4, 2)
    assert out["plan_info"][2] == 0


def test_bruteforce_matches_enumeration():
    rng = np.random.default_rng(9)
    for mode in (FWD, BWD):
        for _ in range(40):
            E = int(rng.integers(1, 4))
            P = int(rng.integers(1, 4))
            s = int(rng.integers(0, 3))
            b = rng.integers(0, 6, size=E).tolist()
            h = rng.integers(0, P, size=E).tolist()
            lam = int(rng.integers(0, 4))
            assert bruteforce_optimum(b, h, P, s, mode, lam) == enumerate_optimum(b, h, P, s, mode, lam)


@pytest.mark.parametrize("mode", [FWD, BWD])
def test_greedy_never_beats_the_optimum(mode):
    rng = np.random.default_rng(21 + mode)
    gaps = []
    for _ in range(40):
        E = int(rng.integers(2, 7))
        P = int(rng.integers(2, 4))
        s = int(rng.integers(1, 3))
        b, h = _random_instance(rng, E, P)
        lam = 3 if mode == BWD else 12
        out = plan(b, h, P, s, mode, lam)
        opt = bruteforce_optimum(b, h, P, s, mode, lam)
        assert out["plan_info"][0] >= opt
        gaps.append(out["plan_info"][0] - opt)
    assert min(gaps) == 0          # the greedy does reach the optimum on many instances


def test_tiny_workload_shape_optimum():
    # the tiny workload's planner shape: E=8, P=4, s=1
    b = [12, 6, 3, 2, 2, 1, 1, 1]
    h = [e * 4 // 8 for e in range(8)]
    out = plan(b, h, 4, 1)
    opt = bruteforce_optimum(b, h, 4, 1)
    assert opt == 7 and out["plan_info"][0] >= opt


def test_golden_cases():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        mode = FWD if c["mode"] == "fwd" else BWD
        out = plan(c["b"], c["owner"], c["P"], c["s"], mode, c["lambda"])
        np.testing.assert_array_equal(out["q"], c["q"], err_msg=c["name"])
        np.testing.assert_array_equal(out["load"], c["load"], err_msg=c["name"])
        np.testing.assert_array_equal(out["block_worker"], c["block_worker"], err_msg=c["name"])
        np.testing.assert_array_equal(out["plan_info"], c["plan_info"], err_msg=c["name"])
        opt = bruteforce_optimum(c["b"], c["owner"], c["P"], c["s"], mode, c["lambda"])
        assert opt == c["optimum"], c["name"]


def test_deterministic():
    rng = np.random.default_rng(1)
    b, h = _random_instance(rng, 128, 8)
    a1 = plan(b, h, 8, 4)
    a2 = plan(list(b), list(h), 8, 4)
    for key in a1:
        np.testing.assert_array_equal(a1[key], a2[key])


def test_bad_arguments_rejected():
    with pytest.raises(ValueError):
        plan([1, 2], [0, 2], 2, 1)
    with pytest.raises(ValueError):
        plan([1, 2], [0, 1], 2, -1)
