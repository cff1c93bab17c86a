"""Oracle: routing statistics -- TEST INFRASTRUCTURE ONLY.

Follows the MegaFlux summary (picx.dev/p/e4jAzZ):
* c_e = number of routed (token, k-slot) pairs whose expert is e, and the skew
  kappa = E * sum_e (c_e / sum_j c_j)^2 -- "Routing Skew Problem", kappa eq.
* b_e = ceil(c_e / beta) token blocks of at most beta rows -- "Problem
  Formulation".
Readings where the pages are silent:
* a slot id < 0 means "no expert here" and is skipped;
* kappa = 1 when no rows are routed (all counts equal);
* rows inside an expert keep the order of their flat index t*k + j, and each
  expert's rows start at slot beta * (blocks of all earlier experts), so
  every block of beta slots belongs to one expert (padded layout).
"""
from __future__ import annotations

import numpy as np


def route_stats(topk_ids, E: int, beta: int) -> dict:
    ids = [int(v) for v in np.asarray(topk_ids).reshape(-1)]
    n = len(ids)
    for v in ids:
        if v >= E:
            raise ValueError(f"expert id {v} >= E={E}")

    counts = [0] * E
    for v in ids:
        if v >= 0:
            counts[v] += 1

    offsets = [0] * (E + 1)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]

    blocks = [(c + beta - 1) // beta for c in counts]
    block_offsets = [0] * (E + 1)
    for e in range(E):
        block_offsets[e + 1] = block_offsets[e] + blocks[e]

    total = sum(counts)
    sq = sum(c * c for c in counts)
    # exact integers, then one correctly rounded division (Python int / int)
    kappa = 1.0 if total == 0 else (E * sq) / (total * total)

    cap = n + E * (beta - 1)
    row_to_slot = [-1] * n
    slot_to_row = [-1] * cap
    seen = [0] * E
    for i, v in enumerate(ids):
        if v < 0:
            continue
        slot = beta * block_offsets[v] + seen[v]
        seen[v] += 1
        row_to_slot[i] = slot
        slot_to_row[slot] = i

    i32 = np.int32
    return {
        "counts": np.array(counts, dtype=i32),
        "offsets": np.array(offsets, dtype=i32),
        "block_counts": np.array(blocks, dtype=i32),
        "block_offsets": np.array(block_offsets, dtype=i32),
        "kappa": float(kappa),
        "row_to_slot": np.array(row_to_slot, dtype=i32),
        "slot_to_row": np.array(slot_to_row, dtype=i32),
        "max_slots": cap,
    }
