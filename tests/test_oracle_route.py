"""Pins for the routing-statistics oracle (oracle/route.py).

Counts, offsets and slots are checked against numpy library routines
(bincount, cumsum, stable argsort); kappa against closed forms of the skew
definition in the MegaFlux summary ("Routing Skew Problem": uniform routing
gives 1) and against exact rational arithmetic.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle.route import route_stats


def _random_ids(rng, T, k, E, neg_frac=0.0):
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    if neg_frac:
        ids[rng.random(ids.shape) < neg_frac] = -1
    return ids


@pytest.mark.parametrize("T,k,E,beta,neg", [(64, 2, 8, 16, 0.0), (300, 4, 16, 7, 0.2),
                                            (1, 1, 3, 1, 0.0), (513, 8, 64, 128, 0.1)])
def test_counts_offsets_slots_match_library(T, k, E, beta, neg):
    rng = np.random.default_rng(T * 7 + E)
    ids = _random_ids(rng, T, k, E, neg)
    st = route_stats(ids, E, beta)
    flat = ids.reshape(-1)
    valid = flat >= 0
    c = np.bincount(flat[valid], minlength=E)
    np.testing.assert_array_equal(st["counts"], c)
    np.testing.assert_array_equal(st["offsets"], np.concatenate([[0], np.cumsum(c)]))
    b = -(-c // beta)
    np.testing.assert_array_equal(st["block_counts"], b)
    boff = np.concatenate([[0], np.cumsum(b)])
    np.testing.assert_array_equal(st["block_offsets"], boff)
    # stable counting sort: argsort by expert id, stable in flat index
    order = np.argsort(np.where(valid, flat, E), kind="stable")[: valid.sum()]
    expected_slot = np.full(flat.shape, -1)
    pos = 0
    for e in range(E):
        rows = order[pos: pos + c[e]]
        expected_slot[rows] = beta * boff[e] + np.arange(c[e])
        pos += c[e]
    np.testing.assert_array_equal(st["row_to_slot"], expected_slot)
    inv = np.full(st["max_slots"], -1)
    inv[expected_slot[valid]] = np.nonzero(valid)[0]
    np.testing.assert_array_equal(st["slot_to_row"], inv)
    assert st["max_slots"] == T * k + E * (beta - 1)


def test_kappa_uniform_is_one():
    E, k = 16, 4
    ids = (np.arange(64 * k) % E).reshape(64, k)
    assert route_stats(ids, E, 8)["kappa"] == 1.0


@pytest.mark.parametrize("E,k", [(8, 2), (64, 8), (128, 8), (5, 5)])
def test_kappa_k_hot_experts_is_E_over_k(E, k):
    ids = np.tile(np.arange(k), (37, 1))
    assert route_stats(ids, E, 16)["kappa"] == float(Fraction(E, k))


def test_kappa_single_expert_is_E():
    assert route_stats(np.full((9, 1), 3), 7, 4)["kappa"] == 7.0


def test_kappa_empty_is_one_and_negative_ids_skipped():
    st = route_stats(np.full((5, 2), -1), 4, 2)
    assert st["kappa"] == 1.0 and st["counts"].sum() == 0
    assert (st["row_to_slot"] == -1).all() and (st["slot_to_row"] == -1).all()
    assert route_stats(np.zeros((0, 2), dtype=np.int32), 4, 2)["kappa"] == 1.0


def test_kappa_two_level_exact_rational():
    # a experts with count hi, the rest with count lo: kappa = E*sum c^2 / (sum c)^2
    rng = np.random.default_rng(3)
    for _ in range(20):
        E = int(rng.integers(2, 40))
        a = int(rng.integers(1, E))
        hi, lo = int(rng.integers(1, 50)), int(rng.integers(0, 50))
        ids = np.array([e for e in range(E) for _ in range(hi if e < a else lo)]).reshape(-1, 1)
        exact = Fraction(E * (a * hi * hi + (E - a) * lo * lo), (a * hi + (E - a) * lo) ** 2)
        assert route_stats(ids, E, 3)["kappa"] == float(exact)


def test_id_out_of_range_rejected():
    with pytest.raises(ValueError):
        route_stats(np.array([[0, 8]]), 8, 4)
