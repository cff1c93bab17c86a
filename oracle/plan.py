"""Oracle: replica placement and token-block assignment -- TEST INFRASTRUCTURE ONLY.

The program (MegaFlux summary, picx.dev/p/e4jAzZ, "Problem Formulation"):

    minimise over integer q >= 0 (E x P):  max_r l_r,   l_r = sum_e q[e][r]
    subject to  sum_r q[e][r] = b_e  for every e,
                #{e : h(e) != r, q[e][r] > 0} <= s  for every worker r.

The heuristic ("Bounded Greedy Search"): four greedy searches, each starting
from the no-replica assignment q[e][h(e)] = b_e and shifting blocks from
overloaded owners toward tau = ceil(sum_e b_e / P) blocks per worker.  The
searches differ in donor priority (decreasing total overload, or largest
remaining home-expert load) and in fan-out (at most one new copy of an expert
per round, or several).  The backward variant scores a plan by
C_lambda = max_r (l_r + lambda * n_r), n_r = number of remote replicas of the
experts that r owns, lambda = 12.

The pages leave the search's inner order open.  Reading used here (the same
reading the HIP planner implements):
* a "round" visits every worker whose effective load L_r (l_r, or
  l_r + lambda*n_r in backward mode) exceeds tau, in decreasing order of the
  donor key taken at the start of the round (overload L_r - tau, or the
  largest q[e][r] over r's own experts); ties -> smaller r;
* a donor walks its own experts with q[e][r] > 0 by decreasing q[e][r], ties
  -> smaller e, and moves blocks while L_r > tau;
* a recipient t != r must have L_t < tau and either already hold a copy of e
  (q[e][t] > 0) or have a free replica slot (fewer than s non-home experts);
  with fan-out "one", an expert gets at most one new copy per round;
* the recipient with the most slack tau - L_t wins, ties -> smaller t;
* the move is delta = min(L_r - tau, tau - L_t, q[e][r]) blocks; in backward
  mode a new copy raises the owner's L_r by lambda, so it is made only when
  delta = min(L_r - tau + lambda, tau - L_t, q[e][r]) > lambda (it must lower
  the owner's cost strictly);
* at most P rounds; a search stops early after a round without a move or
  once every L_r <= tau;
* the plan kept is the search with the smallest objective (max_r L_r), then
  fewest replicas, then the lower search index;
* blocks of expert e are handed out owner first, then ascending worker, so
  every (expert, worker) pair holds one contiguous run of blocks.
"""
from __future__ import annotations

import itertools

import numpy as np

FWD, BWD = 0, 1
EXCESS, HOMELOAD = 0, 1
ONE, MULTI = 0, 1
SEARCHES = ((EXCESS, ONE), (EXCESS, MULTI), (HOMELOAD, ONE), (HOMELOAD, MULTI))


def _greedy(b, h, P, s, mode, lam, donor_key, fanout):
    E = len(b)
    B = sum(b)
    tau = (B + P - 1) // P
    q = [[0] * P for _ in range(E)]
    ell = [0] * P
    for e in range(E):
        q[e][h[e]] = b[e]
        ell[h[e]] += b[e]
    rep = [0] * P      # non-home experts with a copy on r
    nrem = [0] * P     # remote copies of experts owned by r

    def L(r):
        return ell[r] + (lam * nrem[r] if mode == BWD else 0)

    for _round in range(P):
        moved = False
        newcopy = [False] * E
        if donor_key == EXCESS:
            key = [L(r) - tau for r in range(P)]
        else:
            key = [max([q[e][r] for e in range(E) if h[e] == r], default=0) for r in range(P)]
        donors = sorted((r for r in range(P) if L(r) > tau), key=lambda r: (-key[r], r))
        for r in donors:
            own = sorted((e for e in range(E) if h[e] == r and q[e][r] > 0),
                         key=lambda e: (-q[e][r], e))
            for e in own:
                while L(r) > tau and q[e][r] > 0:
                    best = None
                    for t in range(P):
                        if t == r or L(t) >= tau:
                            continue
                        if q[e][t] > 0:
                            delta, new = min(L(r) - tau, tau - L(t), q[e][r]), False
                        else:
                            if rep[t] >= s or (fanout == ONE and newcopy[e]):
                                continue
                            if mode == BWD:
                                delta = min(L(r) - tau + lam, tau - L(t), q[e][r])
                                if delta <= lam:
                                    continue
                            else:
                                delta = min(L(r) - tau, tau - L(t), q[e][r])
                            new = True
                        slack = tau - L(t)
                        if best is None or slack > best[0]:
                            best = (slack, t, delta, new)
                    if best is None:
                        break
                    _, t, delta, new = best
                    q[e][r] -= delta
                    q[e][t] += delta
                    ell[r] -= delta
                    ell[t] += delta
                    if new:
                        rep[t] += 1
                        nrem[r] += 1
                        newcopy[e] = True
                    moved = True
                if L(r) <= tau:
                    break
        if not moved or max(L(r) for r in range(P)) <= tau:
            break
    objective = max(L(r) for r in range(P))
    return q, ell, sum(rep), objective, tau


def plan(block_counts, owner, P: int, s: int, mode: int = FWD, lam: int = 12) -> dict:
    b = [int(v) for v in block_counts]
    h = [int(v) for v in owner]
    E = len(b)
    if P < 1 or s < 0 or lam < 0 or any(not 0 <= x < P for x in h):
        raise ValueError("bad planner arguments")
    best = None
    for sigma, (dk, fo) in enumerate(SEARCHES):
        q, ell, reps, obj, tau = _greedy(b, h, P, s, mode, lam, dk, fo)
        cand = (obj, reps, sigma)
        if best is None or cand < best[0]:
            best = (cand, q, ell, tau)
    (obj, reps, sigma), q, ell, tau = best

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
        "plan_info": np.array([obj, sigma, reps, tau], dtype=np.int32),
    }


def objective_of(q, owner, mode=FWD, lam=12):
    """max_r (l_r + lambda*n_r) for an arbitrary plan (n_r only counted in BWD)."""
    q = np.asarray(q)
    E, P = q.shape
    ell = q.sum(axis=0)
    nrem = np.zeros(P, dtype=np.int64)
    for e in range(E):
        for t in range(P):
            if t != owner[e] and q[e, t] > 0:
                nrem[owner[e]] += 1
    return int((ell + (lam * nrem if mode == BWD else 0)).max())


def _hall_ok(b, nbrs, cap):
    """Transportation feasibility (max-flow / min-cut): every expert set S must fit
    into the total capacity of the workers adjacent to S."""
    E = len(b)
    for mask in range(1, 1 << E):
        need = 0
        nb = set()
        for e in range(E):
            if mask >> e & 1:
                need += b[e]
                nb |= nbrs[e]
        if need > sum(cap[r] for r in nb):
            return False
    return True


def bruteforce_optimum(block_counts, owner, P: int, s: int, mode: int = FWD, lam: int = 12):
    """Exact optimum of the min-max program for tiny E and P.  Enumerates every
    pattern of allowed (expert, worker) pairs -- the home pairs plus at most s
    non-home experts per worker -- and, for each, the smallest T such that the
    blocks fit into capacities T (forward) or T - lambda*n_r (backward)."""
    b = [int(v) for v in block_counts]
    h = [int(v) for v in owner]
    E = len(b)
    B = sum(b)
    if B == 0:
        return 0
    per_worker = []
    for r in range(P):
        foreign = [e for e in range(E) if h[e] != r and b[e] > 0]
        opts = []
        for m in range(0, min(s, len(foreign)) + 1):
            opts.extend(itertools.combinations(foreign, m))
        per_worker.append(opts)
    best = None
    for pattern in itertools.product(*per_worker):
        nbrs = [{h[e]} for e in range(E)]
        nrem = [0] * P
        for r, chosen in enumerate(pattern):
            for e in chosen:
                nbrs[e].add(r)
                nrem[h[e]] += 1
        pen = [lam * nrem[r] if mode == BWD else 0 for r in range(P)]
        lo = max(pen)
        hi = B + max(pen)
        if best is not None:
            hi = min(hi, best)
            if not _hall_ok(b, nbrs, [max(hi - pen[r], 0) for r in range(P)]):
                continue
        while lo < hi:
            mid = (lo + hi) // 2
            if _hall_ok(b, nbrs, [max(mid - pen[r], 0) for r in range(P)]):
                hi = mid
            else:
                lo = mid + 1
        if best is None or lo < best:
            best = lo
    return best


def enumerate_optimum(block_counts, owner, P: int, s: int, mode: int = FWD, lam: int = 12):
    """Exhaustive search over every integer q for very small instances."""
    b = [int(v) for v in block_counts]
    h = [int(v) for v in owner]
    E = len(b)

    def comps(n, parts):
        if parts == 1:
            yield (n,)
            return
        for i in range(n + 1):
            for rest in comps(n - i, parts - 1):
                yield (i,) + rest
    best = None
    for rows in itertools.product(*[list(comps(b[e], P)) for e in range(E)]):
        ok = True
        for r in range(P):
            if sum(1 for e in range(E) if h[e] != r and rows[e][r] > 0) > s:
                ok = False
                break
        if not ok:
            continue
        val = objective_of(np.array(rows), h, mode, lam)
        if best is None or val < best:
            best = val
    return best
