"""GPU parity of the wave-quantized cost model (moe_predict_cost): bit-exact
against the oracle on the planners' outputs for every P in {1, 2, 4, 8} on
the bf16 and fp8 workloads at every kappa."""
import numpy as np
import pytest
import torch

from moe_expert_ffn_amd import binding as B
from moe_expert_ffn_amd.inputs import WORKLOADS, contiguous_owners, make_routing
from oracle.route import route_stats as oracle_route
from oracle.sizing import predicted_cost
from tests.gpu_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _ws(E):
    L = B.Layer(E, 128, 64, B.MOE_F32, B.MOE_F32, 1, 1, None, None)
    return B.workspace(L, 1, 1, 1, 8, 4, False, DEV)


CASES = [(n, k) for n in ("olmoe_bf16", "qwen3_bf16", "dsv3_fp8") for k in WORKLOADS[n].kappas]


@pytest.mark.parametrize("name,kappa", CASES)
def test_predict_cost_matches_oracle(name, kappa):
    w = WORKLOADS[name]
    ids, _ = make_routing(w, kappa)
    rs = oracle_route(ids, w.E, w.beta)
    dev = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).to(DEV)
    counts, boff, bc = dev(rs["counts"]), dev(rs["block_offsets"]), dev(rs["block_counts"])
    nb = int(rs["block_offsets"][-1])
    for P in (1, 2, 4, 8):
        owner_np = contiguous_owners(w.E, P)
        owner = dev(owner_np)
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        pf = B.alloc_plan(w.E, P, max(nb, 1), DEV)
        pb = B.alloc_plan(w.E, P, max(nb, 1), DEV)
        B.plan(bc, boff, owner, P, w.s, B.PLAN_FWD, 12, pf, _ws(w.E), st)
        B.plan(bc, boff, owner, P, w.s, B.PLAN_BWD, 12, pb, _ws(w.E), st)
        cost = torch.zeros(2, dtype=torch.int64, device=DEV)
        B.predict_cost(counts, boff, pf["block_worker"], pb["block_worker"], owner, w.beta, P, w.d,
                       w.d_ff, cost[0:1], st, num_workgroups=256)
        B.predict_cost(counts, boff, pf["block_worker"], pb["block_worker"], owner, w.beta, P, w.d,
                       w.d_ff, cost[1:2], st, num_workgroups=0)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        want = predicted_cost(rs["counts"], pf["block_worker"].cpu().numpy()[:nb],
                              pb["block_worker"].cpu().numpy()[:nb], owner_np, w.beta, P, w.d, w.d_ff,
                              G=256)
        say(f"[cost] {name} kappa={kappa} P={P} cost={want}")
        assert int(cost[0].item()) == want
        assert int(cost[1].item()) == want          # 256 CUs on this device


@pytest.mark.parametrize("name,kappa", CASES)
def test_predict_split_matches_oracle(name, kappa):
    """moe_predict_split (every two-phase mode's predicted time and the choice)
    is bit-exact with the oracle for both directions' plans at every P."""
    from oracle.sizing import select_split, split_costs
    w = WORKLOADS[name]
    ids, _ = make_routing(w, kappa)
    rs = oracle_route(ids, w.E, w.beta)
    dev = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).to(DEV)
    counts, boff, bc = dev(rs["counts"]), dev(rs["block_offsets"]), dev(rs["block_counts"])
    nb = int(rs["block_offsets"][-1])
    for P in (1, 2, 4, 8):
        owner = dev(contiguous_owners(w.E, P))
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        for mode, backward in ((B.PLAN_FWD, False), (B.PLAN_BWD, True)):
            pl = B.alloc_plan(w.E, P, max(nb, 1), DEV)
            B.plan(bc, boff, owner, P, w.s, mode, 12, pl, _ws(w.E), st)
            n = 256 // P
            costs = torch.full((n + 1,), -7, dtype=torch.int64, device=DEV)
            choice = torch.full((1,), -9, dtype=torch.int32, device=DEV)
            B.predict_split(counts, boff, pl["block_worker"], w.beta, P, w.d, w.d_ff, backward,
                            costs, choice, st, num_workgroups=256)
            torch.cuda.synchronize()
            assert int(st.item()) == 0
            want = split_costs(rs["counts"], pl["block_worker"].cpu().numpy()[:nb], w.beta, P, w.d,
                               w.d_ff, backward, G=256)
            got = costs.cpu().tolist()
            say(f"[split] {name} kappa={kappa} P={P} bwd={backward} choice={select_split(want)} "
                f"two={want[0]} temporal={want[1]}")
            assert got == want
            assert int(choice.item()) == select_split(want)
