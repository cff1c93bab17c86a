"""Oracle: runtime replication gate -- TEST INFRASTRUCTURE ONLY.

The MegaFlux summary (picx.dev/p/e4jAzZ) observes that near-balanced routes
gain nothing from replication and can lose to its exposed cost
("Empirical Validation / Results": balanced routes near parity, small skewed
backward workloads down to 0.91x; "Practical Implications": balanced
workloads), and lists as future work a runtime gate that enables replication
only when the predicted saving exceeds the cost ("Limitations").

Reading implemented here (and by the HIP gate): a plan's predicted cost, in
blocks on the busiest worker, is its objective plus rho per replica, where
rho (given in thousandths of a block) prices one replica; the fixed
placement (every expert on its owner) has no replica.  The plan is kept when

    1000 * (objective_fixed - objective_plan) > rho_milli * replicas,

otherwise it is replaced by the fixed placement: q[e][h(e)] = b_e, loads of
the fixed placement, every block on its owner, plan_info = {fixed objective,
-1 (the gate chose fixed placement), 0, tau}.  A plan without replicas is
kept as it is.  The objective is max_r l_r (the forward objective; a
backward plan's lambda term is not part of the comparison).
"""
from __future__ import annotations

import numpy as np

GATED_SEARCH_ID = -1


def fixed_loads(block_counts, owner, P):
    ell = np.zeros(P, dtype=np.int64)
    for e, b in enumerate(block_counts):
        ell[int(owner[e])] += int(b)
    return ell


def gate(plan, block_counts, owner, P: int, rho_milli: int) -> dict:
    """plan: dict with q, load, block_worker, plan_info (a moe_plan result)."""
    if rho_milli < 0:
        raise ValueError("rho_milli must be >= 0")
    b = [int(v) for v in block_counts]
    h = [int(v) for v in owner]
    info = np.asarray(plan["plan_info"]).astype(np.int64)
    reps = int(info[2])
    ell_fix = fixed_loads(b, h, P)
    obj_fix = int(ell_fix.max()) if P else 0
    obj_plan = int(np.asarray(plan["load"]).max()) if P else 0
    if reps == 0 or 1000 * (obj_fix - obj_plan) > rho_milli * reps:
        return {k: np.array(v, copy=True) for k, v in plan.items()}
    E = len(b)
    q = np.zeros((E, P), dtype=np.int32)
    q[np.arange(E), h] = b
    bw = np.concatenate([np.full(b[e], h[e], dtype=np.int32) for e in range(E)]) if sum(b) else \
        np.zeros(0, dtype=np.int32)
    return {"q": q, "load": ell_fix.astype(np.int32), "block_worker": bw,
            "plan_info": np.array([obj_fix, GATED_SEARCH_ID, 0, int(info[3])], dtype=np.int32)}
