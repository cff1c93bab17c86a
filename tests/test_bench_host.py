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
    # (the two-phase launches' entries are sums of two of them)
    fl = sum(v[0] for k, v in m1.items() if "+" not in k)
    assert fl == 18 * w.d * w.d_ff * R
    for a, b in (("fwd.fc1", "fwd.fc2"), ("bwd.dA", "bwd.dX")):
        both = m1[a + "+" + b.split(".")[1]]
        assert both == (m1[a][0] + m1[b][0], m1[a][1] + m1[b][1])
    # routing statistics: the ids read once, row_to_slot and the slots in use written
    m2 = bench.kernel_model(w, R, T, w.E, 0, 0, slots_used=70000)
    assert m2["route"] == (0, 4 * (2 * T * w.k + 70000))


def test_worker_spread_from_a_hand_timeline():
    # 16 workgroups, P = 2: workers own workgroups with g % 8 < 4 (worker 0) and >= 4 (worker 1)
    tl = np.zeros((5, 1024, 2), dtype=np.int64)
    g = np.arange(16)
    tl[0, :16, 0] = 100
    tl[0, :16, 1] = np.where(g % 8 < 4, 200, 400)       # worker 0 ends at +100, worker 1 at +300
    sp = bench.worker_spread(tl, 2)
    assert sp == {"fc1": round(300 / 200, 3)}


def test_profiled_traffic_only_for_its_own_workload():
    """The counter-based traffic figure is reported only for the kernel,
    workload, kappa and placement it was measured on, and only while the
    kernel sources are the ones it was measured on."""
    w = WORKLOADS["qwen3_bf16_fwdbwd"]
    R, T = 65536, 8192
    stages = {"bwd.dW": 1.0, "fwd.fc1": 0.4}
    pt = bench.PROFILED_TRAFFIC
    own = (pt["workload"], pt["kappa"], pt["fixed"])
    roof, _ = bench.roofline(w, stages, R, T, w.E, 0, 0, run=own)
    assert roof["kernel"] == "bwd.dW"
    assert roof["traffic"] == (pt["bytes"] if pt["source"] == bench.source_hash() else None)
    for other in (("dsv3_fp8_fwdbwd", 1.0, False), (pt["workload"], 8.0, False),
                  (pt["workload"], 1.0, True)):
        assert bench.roofline(w, stages, R, T, w.E, 0, 0, run=other)[0]["traffic"] is None
    assert bench.roofline(w, stages, R, T, w.E, 0, 0)[0]["traffic"] is None
