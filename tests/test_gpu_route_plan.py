"""GPU parity of the routing statistics and the planner: bit-exact against the
oracle (counts, offsets, blocks, slots, kappa, q, loads, block workers, plan
info), deterministic across runs, on every workload and on edge cases."""
import numpy as np
import pytest
import torch

from moe_expert_ffn_amd import binding as B
from moe_expert_ffn_amd.inputs import WORKLOADS, Workload, contiguous_owners, make_routing
from oracle.plan import plan as oracle_plan
from oracle.route import route_stats as oracle_route
from tests.gpu_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _ws(E, T, k, beta, P=8, s=4):
    L = B.Layer(E, 128, 64, B.MOE_F32, B.MOE_F32, 1, 1, None, None)
    return B.workspace(L, T, k, beta, P, s, False, DEV)


def _gpu_route(ids_np, E, beta):
    T, k = ids_np.shape
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).to(DEV)
    out = B.alloc_route(T, k, E, beta, DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    B.route_stats(ids, E, beta, out, _ws(E, T, k, beta), st)
    torch.cuda.synchronize()
    return {k_: v.cpu().numpy() for k_, v in out.items()}, int(st.item())


def _check_route(ids_np, E, beta):
    g, st = _gpu_route(ids_np, E, beta)
    o = oracle_route(ids_np, E, beta)
    assert st == 0
    for key in ("counts", "offsets", "block_counts", "block_offsets"):
        np.testing.assert_array_equal(g[key], o[key], err_msg=key)
    N = ids_np.size
    np.testing.assert_array_equal(g["row_to_slot"][:N], o["row_to_slot"])
    np.testing.assert_array_equal(g["slot_to_row"][:o["max_slots"]], o["slot_to_row"])
    assert g["kappa"][0] == o["kappa"], (g["kappa"][0], o["kappa"])
    return o


ROUTE_CASES = [(n, k) for n in ("tiny_f32", "olmoe_bf16", "qwen3_bf16", "dsv3_fp8")
               for k in WORKLOADS[n].kappas]


@pytest.mark.parametrize("name,kappa", ROUTE_CASES)
def test_route_stats_workloads(name, kappa):
    say(f"[route] {name} kappa={kappa}")
    w = WORKLOADS[name]
    ids, _ = make_routing(w, kappa)
    _check_route(ids, w.E, w.beta)


@pytest.mark.parametrize("T,k,E,beta,neg", [(1, 1, 1, 1, 0.0), (5, 2, 4, 2, 1.0), (257, 3, 37, 7, 0.3),
                                            (1000, 8, 512, 128, 0.0), (300, 6, 1024, 1, 0.1),
                                            (4097, 2, 2, 3, 0.0), (0, 4, 8, 16, 0.0),
                                            # more than 32 chunks of 256 rows per scan thread
                                            # (1024 threads = E x groups): the scan's general path
                                            (3000, 4, 1024, 16, 0.1), (9000, 8, 128, 128, 0.05)])
def test_route_stats_edges(T, k, E, beta, neg):
    say(f"[route-edge] T={T} k={k} E={E} beta={beta} neg={neg}")
    rng = np.random.default_rng(T + E)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    ids[rng.random((T, k)) < neg] = -1
    if T == 0:
        g, st = _gpu_route(np.zeros((1, k), np.int32)[:0], E, beta)
        assert g["kappa"][0] == 1.0 and g["counts"].sum() == 0
        return
    _check_route(ids, E, beta)


def test_route_bad_expert_flagged():
    ids = np.array([[0, 9], [3, 1]], dtype=np.int32)
    _, st = _gpu_route(ids, 8, 4)
    assert st & B.DEV_BAD_EXPERT


def _gpu_plan(b, boff, owner, P, s, mode, lam, reps=1):
    dev = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).to(DEV)
    bt, bo, ow = dev(b), dev(boff), dev(owner)
    E = len(b)
    outs = []
    for _ in range(reps):
        out = B.alloc_plan(E, P, max(int(boff[-1]), 1), DEV)
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        B.plan(bt, bo, ow, P, s, mode, lam, out, _ws(E, 1, 1, 1), st)
        torch.cuda.synchronize()
        outs.append(({k_: v.cpu().numpy() for k_, v in out.items()}, int(st.item())))
    return outs


def _check_plan(b, owner, P, s, mode, lam, reps=1):
    boff = np.concatenate([[0], np.cumsum(b)]).astype(np.int32)
    o = oracle_plan(b, owner, P, s, mode, lam)
    outs = _gpu_plan(b, boff, owner, P, s, mode, lam, reps)
    nb = int(boff[-1])
    for g, st in outs:
        assert st == 0
        np.testing.assert_array_equal(g["q"], o["q"])
        np.testing.assert_array_equal(g["load"], o["load"])
        np.testing.assert_array_equal(g["block_worker"][:nb], o["block_worker"])
        np.testing.assert_array_equal(g["plan_info"], o["plan_info"])
    return o


PLAN_CASES = [(n, k) for n in ("tiny_f32", "olmoe_bf16", "qwen3_bf16", "dsv3_fp8")
              for k in WORKLOADS[n].kappas]


@pytest.mark.parametrize("name,kappa", PLAN_CASES)
def test_plan_workloads(name, kappa):
    w = WORKLOADS[name]
    ids, _ = make_routing(w, kappa)
    b = oracle_route(ids, w.E, w.beta)["block_counts"]
    owner = contiguous_owners(w.E, w.P)
    for mode in (B.PLAN_FWD, B.PLAN_BWD):
        for s in (w.s, 0):
            say(f"[plan] {name} kappa={kappa} mode={mode} s={s}")
            _check_plan(b, owner, w.P, s, mode, 12, reps=3 if s else 1)


def test_plan_random_instances():
    rng = np.random.default_rng(7)
    for it in range(60):
        E = int(rng.choice([1, 3, 8, 37, 64, 128, 512]))
        P = int(rng.choice([1, 2, 4, 8]))
        s = int(rng.choice([0, 1, 2, 4, 8]))
        lam = int(rng.choice([0, 3, 12]))
        mode = int(rng.integers(0, 2))
        b = (rng.integers(0, 30, size=E) * (rng.random(E) < 0.7)).astype(np.int32)
        b[rng.integers(0, E)] += int(rng.integers(0, 200))
        owner = rng.integers(0, P, size=E).astype(np.int32)
        say(f"[plan-rand] it={it} E={E} P={P} s={s} lam={lam} mode={mode}")
        _check_plan(b, owner, P, s, mode, lam)


def test_plan_deterministic_many_runs():
    w = WORKLOADS["qwen3_bf16"]
    ids, _ = make_routing(w, 8)
    b = oracle_route(ids, w.E, w.beta)["block_counts"]
    _check_plan(b, contiguous_owners(w.E, w.P), 8, 4, B.PLAN_FWD, 12, reps=10)


def test_plan_bad_owner_flagged():
    b = np.array([3, 4], dtype=np.int32)
    outs = _gpu_plan(b, np.array([0, 3, 7], np.int32), np.array([0, 5], np.int32), 2, 1,
                     B.PLAN_FWD, 12)
    assert outs[0][1] & B.DEV_BAD_OWNER
