"""GPU parity of the runtime replication gate (moe_plan_gate) applied to the
planners' outputs: bit-exact against the oracle gate (q, loads, block
workers, plan info) on every workload and kappa, for prices on both sides of
each plan's saving, and on random instances; bad owners are flagged."""
import numpy as np
import pytest
import torch

from moe_expert_ffn_amd import binding as B
from moe_expert_ffn_amd.inputs import WORKLOADS, contiguous_owners, make_routing
from oracle.gate import gate as oracle_gate
from oracle.plan import BWD, FWD
from oracle.plan import plan as oracle_plan
from oracle.quota import quota_plan
from oracle.route import route_stats as oracle_route
from tests.gpu_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _ws(E):
    L = B.Layer(E, 128, 64, B.MOE_F32, B.MOE_F32, 1, 1, None, None)
    return B.workspace(L, 1, 1, 1, 8, 4, False, DEV)


def _gpu_plan_gate(b, owner, P, s, mode, lam, rho):
    b = np.asarray(b, dtype=np.int32)
    boff = np.concatenate([[0], np.cumsum(b)]).astype(np.int32)
    dev = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).to(DEV)
    bt, bo, ow = dev(b), dev(boff), dev(owner)
    out = B.alloc_plan(len(b), P, max(int(boff[-1]), 1), DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    B.plan(bt, bo, ow, P, s, mode, lam, out, _ws(len(b)), st)
    B.plan_gate(bt, bo, ow, P, rho, out, st)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}, int(st.item()), int(boff[-1])


def _oracle(b, owner, P, s, mode, lam):
    if mode == B.PLAN_QUOTA:
        return quota_plan(b, owner, P, s, lam)
    return oracle_plan(b, owner, P, s, FWD if mode == B.PLAN_FWD else BWD, lam)


def _check(b, owner, P, s, mode, lam, rho):
    o = oracle_gate(_oracle(b, owner, P, s, mode, lam), b, owner, P, rho)
    g, st, nb = _gpu_plan_gate(b, owner, P, s, mode, lam, rho)
    assert st == 0
    np.testing.assert_array_equal(g["q"], o["q"])
    np.testing.assert_array_equal(g["load"], o["load"])
    np.testing.assert_array_equal(g["block_worker"][:nb], o["block_worker"])
    np.testing.assert_array_equal(g["plan_info"], o["plan_info"])
    return o


CASES = [(n, k) for n in ("tiny_f32", "olmoe_bf16", "qwen3_bf16", "dsv3_fp8")
         for k in WORKLOADS[n].kappas]


@pytest.mark.parametrize("name,kappa", CASES)
def test_gate_workloads(name, kappa):
    w = WORKLOADS[name]
    ids, _ = make_routing(w, kappa)
    b = oracle_route(ids, w.E, w.beta)["block_counts"]
    owner = contiguous_owners(w.E, w.P)
    for mode, lam in ((B.PLAN_FWD, 12), (B.PLAN_BWD, 12), (B.PLAN_QUOTA, 1)):
        o = _oracle(b, owner, w.P, w.s, mode, lam)
        reps = int(o["plan_info"][2])
        fixed = int(np.bincount(owner, weights=b, minlength=w.P).max())
        saving = fixed - int(o["load"].max())
        # prices just below and at the break-even point, and free replicas
        prices = {0, 1000}
        if reps:
            prices |= {max(1000 * saving // reps - 1, 0), 1000 * saving // reps + 1}
        for rho in sorted(prices):
            say(f"[gate] {name} kappa={kappa} mode={mode} rho={rho} reps={reps} saving={saving}")
            _check(b, owner, w.P, w.s, mode, lam, rho)


def test_gate_random_instances():
    rng = np.random.default_rng(5)
    for it in range(40):
        E = int(rng.choice([1, 8, 37, 128, 512]))
        P = int(rng.choice([1, 2, 4, 8]))
        s = int(rng.choice([0, 1, 2, 4]))
        b = (rng.integers(0, 30, size=E) * (rng.random(E) < 0.7)).astype(np.int32)
        b[rng.integers(0, E)] += int(rng.integers(0, 200))
        owner = rng.integers(0, P, size=E).astype(np.int32)
        mode = int(rng.choice([B.PLAN_FWD, B.PLAN_QUOTA]))
        rho = int(rng.choice([0, 500, 1000, 4000, 10 ** 6]))
        say(f"[gate-rand] it={it} E={E} P={P} s={s} mode={mode} rho={rho}")
        _check(b, owner, P, s, mode, 1 if mode == B.PLAN_QUOTA else 12, rho)


def test_gate_bad_owner_flagged():
    dev = lambda a: torch.tensor(a, dtype=torch.int32, device=DEV)
    out = B.alloc_plan(2, 2, 7, DEV)
    out["plan_info"].copy_(dev([7, 0, 1, 4]))
    out["load"].copy_(dev([4, 3]))
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    B.plan_gate(dev([3, 4]), dev([0, 3, 7]), dev([0, 5]), 2, 1000, out, st)
    torch.cuda.synchronize()
    assert int(st.item()) & B.DEV_BAD_OWNER
