"""Oracle: wave-quantized cost model for choosing the CU partition count P
-- TEST INFRASTRUCTURE ONLY.

The page "Analytical Resource Management for Fine-grained MoE
Computation-Communication Overlap" (weekinpapers.com, abstract) selects a
launch's resource partition before the launch from routed-tile counts, kernel
occupancy and residency, with a wave-quantized analytical model and no
candidate execution.  Here the resource partition is P, the number of CU
partitions (workers) the expert layer runs on, and the model predicts the
time of one forward + backward pass of a plan made for that P.

Reading (the HIP cost kernel computes exactly the same integers):
* a worker owns G / P workgroups (G = one workgroup per CU); the persistent
  GEMM launches deal a worker's items round-robin: workgroup j takes items
  j, j + n, j + 2n, ... (n = G / P), so a phase lasts, on that worker, as long
  as its busiest workgroup, and the phase as long as its busiest worker;
* items: a (row tile, N tile) pair for FC1, FC2, dA and dX, and a (segment,
  256 x 256 output tile) pair for the weight gradients; a row tile is up to
  bm = 256 consecutive slots of one (expert, worker) run of blocks: a run of
  n_b blocks gives ceil(n_b * beta / bm) tiles when beta divides bm, and
  every block gives ceil(rows / bm) tiles otherwise; N tiles: 2 d_ff / 256
  (FC1), d / 256 (FC2, dX), d_ff / 256 (dA); a segment is the rows of one
  (expert, worker) pair of the backward plan, replica segments first, each
  in expert order, with (d / 256)(d_ff / 256) + (2 d_ff / 256)(d / 256) tiles;
* an item costs its K steps (K / 64; d / 64 for FC1 and dA, d_ff / 64 for
  FC2, 2 d_ff / 64 for dX, max(2, ceil(rows / 64)) for a weight-gradient
  tile) plus its epilogue, counted in thousandths of a step: the bytes it
  writes (and for dA the bytes of [G, U] it reads) divided by what one CU
  stores during one step (EPI_BYTES_PER_STEP, 214,000 bytes: 121 GB/s per CU
  times 1.77 us per step, both measured once on MI355X for this engine);
* the predicted cost of a plan is the sum over the five phases, in
  thousandths of a step; the selector takes the P of smallest cost, ties to
  the larger P.
"""
from __future__ import annotations

import numpy as np

EPI_BYTES_PER_STEP = 214_000
CANDIDATE_P = (1, 2, 4, 8)


def epilogue_milli(bytes_moved: int) -> int:
    return (bytes_moved * 1000) // EPI_BYTES_PER_STEP


def _row_tiles(counts, block_worker, beta, P, bm=256):
    """Row tiles per worker (how the executors cut each (expert, worker) run)."""
    E = len(counts)
    nb = [(int(c) + beta - 1) // beta for c in counts]
    tiles = [0] * P
    g = 0
    for e in range(E):
        per_w = {}
        for i in range(nb[e]):
            w = int(block_worker[g + i])
            rows = min(beta, int(counts[e]) - beta * i)
            per_w.setdefault(w, []).append(rows)
        for w, rows in per_w.items():
            if bm % beta == 0:
                f = bm // beta
                tiles[w] += (len(rows) + f - 1) // f
            else:
                tiles[w] += sum((r + bm - 1) // bm for r in rows)
        g += nb[e]
    return tiles


def _segments(counts, block_worker, owner, beta, P):
    """Weight-gradient segments per worker: list of row counts in execution order."""
    E = len(counts)
    rows = np.zeros((E, P), dtype=np.int64)
    g = 0
    for e in range(E):
        nbe = (int(counts[e]) + beta - 1) // beta
        for i in range(nbe):
            rows[e, int(block_worker[g + i])] += min(beta, int(counts[e]) - beta * i)
        g += nbe
    segs = []
    for r in range(P):
        order = [e for e in range(E) if owner[e] != r] + [e for e in range(E) if owner[e] == r]
        segs.append([int(rows[e, r]) for e in order if rows[e, r] > 0])
    return segs


def _phase(items_per_worker_costs, n):
    """Busiest workgroup over all workers; items are dealt round-robin."""
    worst = 0
    for costs in items_per_worker_costs:
        wg = [0] * n
        for i, c in enumerate(costs):
            wg[i % n] += c
        worst = max(worst, max(wg) if wg else 0)
    return worst


def predicted_cost(counts, bw_fwd, bw_bwd, owner, beta, P, d, d_ff, G=256, bm=256) -> int:
    """Predicted forward + backward time of the plans, thousandths of a step."""
    n = G // P
    tf = _row_tiles(counts, bw_fwd, beta, P, bm)
    tb = _row_tiles(counts, bw_bwd, beta, P, bm)
    fc1 = 1000 * (d // 64) + epilogue_milli(bm * (128 + 256) * 2)    # A and the saved [G, U]
    fc2 = 1000 * (d_ff // 64) + epilogue_milli(bm * 256 * 2)
    da = 1000 * (d // 64) + epilogue_milli(bm * 256 * 3 * 2 + bm * 512 * 2)
    dx = 1000 * (2 * d_ff // 64) + epilogue_milli(bm * 256 * 2)
    cost = 0
    cost += _phase([[fc1] * (t * (2 * d_ff // 256)) for t in tf], n)
    cost += _phase([[fc2] * (t * (d // 256)) for t in tf], n)
    cost += _phase([[da] * (t * (d_ff // 256)) for t in tb], n)
    cost += _phase([[dx] * (t * (d // 256)) for t in tb], n)
    per_seg = (d // 256) * (d_ff // 256) + (2 * d_ff // 256) * (d // 256)
    dw_epi = epilogue_milli(256 * 256 * 4)
    dw = []
    for segs in _segments(counts, bw_bwd, owner, beta, P):
        costs = []
        for rows in segs:
            c = 1000 * max(2, (rows + 63) // 64) + dw_epi
            costs += [c] * per_seg
        dw.append(costs)
    cost += _phase(dw, n)
    return int(cost)


def select_partition(costs: dict) -> int:
    """P of smallest predicted cost; ties go to the larger P."""
    return min(costs, key=lambda p: (costs[p], -p))


# ---------------------------------------------------------------------------
# Producer/consumer split of a two-phase launch.
#
# The same page selects, besides the partition, how many CTAs of a
# dependency-coupled pipeline produce and how many consume, from routed-tile
# counts and split-level readiness, with no candidate run.  Here the pipeline
# is one direction's pair of GEMM phases in one persistent launch: FC1 -> FC2
# (forward) or dA -> dX (backward); the second phase's item of row tile t
# needs every first-phase item of row tile t.  On each worker (n = G / P
# workgroups, per-worker row tiles T_r as above, items tile-major: item i of a
# phase belongs to row tile i // nnt) the modes are:
# * mode -1, two launches: the second phase starts once the first has ended
#   everywhere: max_r ceil(T_r nnt1 / n) c1 + max_r ceil(T_r nnt2 / n) c2;
# * mode 0, temporal: workgroup j runs first-phase items j, j + n, ... and then
#   second-phase items j, j + n, ...; a second-phase item starts when the
#   workgroup is free and its row tile is ready;
# * mode n1 (1 <= n1 < n), spatial: workgroups j < n1 deal the first-phase
#   items among themselves, the other n - n1 deal the second-phase items;
#   a consumer's item starts when it is free and its row tile is ready.
# A first-phase item i dealt over m workgroups ends at (i // m + 1) c1 (all
# items of a phase cost the same), so row tile t is ready at
# ((t nnt1 + nnt1 - 1) // m + 1) c1.  The mode's time is the latest
# workgroup over all workers; the selector takes the smallest, ties to the
# lower mode (two launches first).
# ---------------------------------------------------------------------------
def _ready(t: int, nnt1: int, m: int, c1: int) -> int:
    return ((t * nnt1 + nnt1 - 1) // m + 1) * c1


def _consume(items: range, nnt2: int, c2: int, start: int, ready) -> int:
    clock = start
    for i2 in items:
        clock = max(clock, ready(i2 // nnt2)) + c2
    return clock


def pair_cost(T, n, mode, nnt1, nnt2, c1, c2) -> int:
    """Predicted time of one direction's phase pair under `mode`."""
    if mode == -1:
        m1 = max((t * nnt1 + n - 1) // n for t in T)
        m2 = max((t * nnt2 + n - 1) // n for t in T)
        return m1 * c1 + m2 * c2
    worst = 0
    for t_r in T:
        N1, N2 = t_r * nnt1, t_r * nnt2
        if mode == 0:
            rd = lambda t: _ready(t, nnt1, n, c1)
            for j in range(n):
                own = len(range(j, N1, n)) * c1
                worst = max(worst, _consume(range(j, N2, n), nnt2, c2, own, rd))
        else:
            n1, n2 = mode, n - mode
            rd = lambda t: _ready(t, nnt1, n1, c1)
            worst = max(worst, ((N1 + n1 - 1) // n1) * c1)
            for j in range(n2):
                worst = max(worst, _consume(range(j, N2, n2), nnt2, c2, 0, rd))
    return worst


def split_costs(counts, block_worker, beta, P, d, d_ff, backward, G=256, bm=256) -> list:
    """Predicted times of every mode -1, 0, 1, ..., n - 1 (list index mode + 1)
    of the forward (backward=False: FC1 -> FC2) or backward (dA -> dX) pair."""
    n = G // P
    T = _row_tiles(counts, block_worker, beta, P, bm)
    if backward:
        nnt1, nnt2 = d_ff // 256, d // 256
        c1 = 1000 * (d // 64) + epilogue_milli(bm * 256 * 3 * 2 + bm * 512 * 2)
        c2 = 1000 * (2 * d_ff // 64) + epilogue_milli(bm * 256 * 2)
    else:
        nnt1, nnt2 = 2 * d_ff // 256, d // 256
        c1 = 1000 * (d // 64) + epilogue_milli(bm * (128 + 256) * 2)
        c2 = 1000 * (d_ff // 64) + epilogue_milli(bm * 256 * 2)
    return [pair_cost(T, n, m, nnt1, nnt2, c1, c2) for m in range(-1, n)]


def select_split(costs: list) -> int:
    """Mode of smallest predicted time; ties to the lower mode."""
    best = min(range(len(costs)), key=lambda i: (costs[i], i))
    return best - 1
