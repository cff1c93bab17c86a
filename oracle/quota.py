"""Oracle: quota-driven planner -- TEST INFRASTRUCTURE ONLY.

Written from the UltraEP reading notes (jianyuh.github.io, "UltraEP: Exact
Load Balancing for Rack-Scale MoE"), section 4 "The Quota-Driven Planning
Solver" and its Algorithm 1 (joint solving), in the units of this layer:

* loads are token blocks: expert e carries b_e blocks, all routed from one
  source, so the load matrix collapses to the vector b and its home worker
  h(e); l_r = sum of the blocks a worker holds;
* the slot budget N_slot is the per-worker replica budget s;
* the quota table U is q[e][r] (blocks of e on worker r);
* the quota floor u_min is in blocks.

The solver binary-searches the smallest load threshold tau for which a greedy
feasibility pass succeeds.  For a threshold tau the pass starts from the
no-replica placement q[e][h(e)] = b_e and takes
    exc_r = max(l_r - tau, 0),  slk_r = max(tau - l_r, 0);
it visits the overloaded workers by decreasing excess and each one's own
experts by decreasing load; an expert's blocks go to the worker with the most
slack that does not yet host that expert, in amounts
    delta = min(exc_r, slk_t, blocks of e still on r),
and a transfer (which creates a replica) is made only when delta >= u_min.
tau is feasible when no excess is left.

Readings where the notes leave a step open (the HIP quota planner implements
the same ones):
* the search range is [ceil(B / P), max_r l_r of the fixed placement]; the
  upper end is always feasible (no move needed); the midpoint is rounded down;
  a feasible midpoint lowers the upper end, an infeasible one raises the lower
  end past it; the plan returned is the pass at the final threshold;
* donor order is the excess at the start of the pass, ties -> smaller r;
  expert order is b_e, ties -> smaller e;
* an expert keeps giving blocks while its worker is in excess (one transfer
  per recipient, several recipients possible: the notes' relay tree for
  experts with more than four replicas implies multi-way replication);
* a recipient needs t != r, no copy of e yet, fewer than s replicas, and slack
  > 0; the largest slack wins, ties -> smaller t; when the best recipient's
  delta is below u_min, the expert gives nothing more in this pass;
* plan_info = {objective max_r l_r, 4 (the quota solver), replica count, tau};
* block_worker hands out expert e's blocks owner first, then ascending
  worker, as in the bounded greedy planner.
"""
from __future__ import annotations

import numpy as np

QUOTA_SEARCH_ID = 4


def _fixed(b, h, P):
    E = len(b)
    q = [[0] * P for _ in range(E)]
    ell = [0] * P
    for e in range(E):
        q[e][h[e]] = b[e]
        ell[h[e]] += b[e]
    return q, ell


def feasibility_pass(b, h, P, s, u_min, tau):
    """One greedy pass at threshold tau: (feasible, q, ell, replicas)."""
    E = len(b)
    q, ell = _fixed(b, h, P)
    exc = [max(ell[r] - tau, 0) for r in range(P)]
    slk = [max(tau - ell[r], 0) for r in range(P)]
    rep = [0] * P
    donors = sorted((r for r in range(P) if exc[r] > 0), key=lambda r: (-exc[r], r))
    for r in donors:
        for e in sorted((e for e in range(E) if h[e] == r), key=lambda e: (-b[e], e)):
            if exc[r] == 0:
                break
            while exc[r] > 0 and q[e][r] > 0:
                best = None
                for t in range(P):
                    if t == r or q[e][t] > 0 or rep[t] >= s or slk[t] <= 0:
                        continue
                    if best is None or slk[t] > slk[best]:
                        best = t
                if best is None:
                    break
                delta = min(exc[r], slk[best], q[e][r])
                if delta < u_min:
                    break
                q[e][r] -= delta
                q[e][best] += delta
                ell[r] -= delta
                ell[best] += delta
                exc[r] -= delta
                slk[best] -= delta
                rep[best] += 1
    return all(x == 0 for x in exc), q, ell, sum(rep)


def quota_plan(block_counts, owner, P: int, s: int, u_min: int = 1) -> dict:
    b = [int(v) for v in block_counts]
    h = [int(v) for v in owner]
    E = len(b)
    if P < 1 or s < 0 or u_min < 1 or any(not 0 <= x < P for x in h):
        raise ValueError("bad planner arguments")
    B = sum(b)
    _, ell0 = _fixed(b, h, P)
    lo, hi = (B + P - 1) // P, max(ell0)
    while lo < hi:
        mid = (lo + hi) // 2
        if feasibility_pass(b, h, P, s, u_min, mid)[0]:
            hi = mid
        else:
            lo = mid + 1
    tau = lo
    ok, q, ell, reps = feasibility_pass(b, h, P, s, u_min, tau)
    assert ok, "the upper end of the search range is always feasible"
    boff = [0] * (E + 1)
    for e in range(E):
        boff[e + 1] = boff[e] + b[e]
    block_worker = [-1] * boff[E]
    for e in range(E):
        pos = boff[e]
        for t in [h[e]] + [t for t in range(P) if t != h[e]]:
            for _ in range(q[e][t]):
                block_worker[pos] = t
                pos += 1
    return {
        "q": np.array(q, dtype=np.int32).reshape(E, P),
        "load": np.array(ell, dtype=np.int32),
        "block_worker": np.array(block_worker, dtype=np.int32),
        "plan_info": np.array([max(ell) if P else 0, QUOTA_SEARCH_ID, reps, tau], dtype=np.int32),
    }
