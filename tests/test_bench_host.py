"""Host logic of bench.py (no GPU): the replica reduction's byte count from a
backward plan, and the per-kernel algorithmic byte model it feeds."""
import numpy as np
import torch

import bench
from moe_expert_ffn_amd.inputs import WORKLOADS


class _Runner:
    def __init__(self, q):
        self.plan_b = {"q": torch.tensor(q, dtype=torch.int32)}


class _W:
    d, d_ff, E = 128, 64, 4


def test_reduce_bytes_hand_plan():
    # owners 0, 0, 1, 1.  e0: owner partial only -> untouched; e1: no blocks anywhere ->
    # the owner slot is written (zeros); e2: owner partial + one replica -> read 2, write 1;
    # e3: all blocks on its owner -> untouched
    case = {"runner": _Runner([[2, 0], [0, 0], [1, 1], [0, 3]]), "owner_np": np.array([0, 0, 1, 1])}
    per = 3 * _W.d * _W.d_ff * 4
    assert bench.reduce_bytes(case, _W) == (1 + 3) * per


def test_reduce_bytes_replicas_without_owner_partial():
    # e0's owner gave away all its blocks to workers 1 and 2: two partials read, owner written
    case = {"runner": _Runner([[0, 2, 1], [1, 0, 0]]), "owner_np": np.array([0, 0])}

    class W:
        d, d_ff, E = 256, 128, 2
    assert bench.reduce_bytes(case, W) == 3 * (3 * 256 * 128 * 4)


def test_kernel_model_reduce_entry_only_with_bytes():
    w = WORKLOADS["qwen3_bf16_fwdbwd"]
    R, T = 65536, 8192
    m0 = bench.kernel_model(w, R, T, w.E, 0, 0)
    assert "bwd.reduce" not in m0
    m1 = bench.kernel_model(w, R, T, w.E, 3, 12345)
    assert m1["bwd.reduce"] == (0, 12345)
    # every replica adds one fp32 partial (3 d d_ff values) to the weight-gradient writes
    assert m1["bwd.dW"][1] - m0["bwd.dW"][1] == 3 * (3 * w.d * w.d_ff * 4)
    # the useful flops of the five contractions add up to 18 d d_ff per routed row
    fl = sum(v[0] for v in m1.values())
    assert fl == 18 * w.d * w.d_ff * R
