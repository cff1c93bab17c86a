"""Pins for the wave-quantized cost model (oracle/sizing.py).

The model is defined arithmetic over tile counts, so the pins are a small
case computed by hand from its definition (every phase and the weight-
gradient round-robin spelled out), wave quantization at the n / n + 1 item
boundary, equal costs for every P on a uniform route (every plan is then the
fixed placement, with whole experts per worker), and a balanced plan costing
less than the fixed placement it improves.
"""
import numpy as np

from oracle.plan import BWD, FWD, plan
from oracle.route import route_stats
from oracle.sizing import epilogue_milli, predicted_cost, select_partition


def test_hand_case():
    # E=2, counts [512, 256], beta=128, one worker with 2 workgroups, d = d_ff = 256.
    # Row tiles: e0 4 blocks -> 2 tiles, e1 2 blocks -> 1 tile: 3 tiles.
    fc1 = 4 * 1000 + 196608 * 1000 // 214000        # K=d/64=4 steps; A + [G, U] = 196,608 B
    fc2 = 4 * 1000 + 131072 * 1000 // 214000        # K=d_ff/64; 131,072 B
    da = 4 * 1000 + 655360 * 1000 // 214000         # writes 393,216 B, reads 262,144 B
    dx = 8 * 1000 + 131072 * 1000 // 214000         # K=2 d_ff/64
    assert (fc1, fc2, da, dx) == (4918, 4612, 7062, 8612)
    phases = 3 * fc1 + 2 * fc2 + 2 * da + 2 * dx      # 6, 3, 3, 3 items over 2 workgroups
    # weight gradients: 3 tiles per segment; e0 has 8 steps, e1 4; item costs
    # [c0, c0, c0, c1, c1, c1] round-robin: wg0 = c0 + c0 + c1, wg1 = c0 + c1 + c1
    c0, c1 = 8000 + 1224, 4000 + 1224
    assert epilogue_milli(256 * 256 * 4) == 1224
    want = phases + max(2 * c0 + c1, c0 + 2 * c1)
    bw = np.zeros(6, dtype=np.int32)
    got = predicted_cost([512, 256], bw, bw, [0, 0], 128, 1, 256, 256, G=2)
    assert got == want == 78998


def test_wave_quantization():
    # One expert, beta = 256 (a block is a row tile), d = d_ff = 256, 4 workgroups.
    # 4 blocks: FC1 8 items (2 waves), FC2/dA/dX 4 items (1 wave each);
    # 5 blocks: FC1 10 items (3 waves), FC2/dA/dX 5 items (2 waves each).
    # The weight-gradient segment has 3 tiles (one wave) of 16 vs 20 K steps.
    def cost(nblocks):
        bw = np.zeros(nblocks, dtype=np.int32)
        return predicted_cost([256 * nblocks], bw, bw, [0], 256, 1, 256, 256, G=4)
    fc1, fc2, da, dx = 4918, 4612, 7062, 8612
    assert cost(5) - cost(4) == fc1 + fc2 + da + dx + (20 - 16) * 1000


def test_uniform_route_equal_for_every_P():
    E, beta = 16, 128
    counts = np.full(E, 512)
    ids = np.repeat(np.arange(E), 512).reshape(-1, 8)
    rs = route_stats(ids, E, beta)
    costs = {}
    for P in (1, 2, 4, 8):
        owner = [e * P // E for e in range(E)]
        pf = plan(rs["block_counts"], owner, P, 2, FWD)
        pb = plan(rs["block_counts"], owner, P, 2, BWD)
        assert pf["plan_info"][2] == 0 and pb["plan_info"][2] == 0
        costs[P] = predicted_cost(counts, pf["block_worker"], pb["block_worker"], owner, beta, P,
                                  512, 512, G=64)
    assert len(set(costs.values())) == 1
    assert select_partition(costs) == 8                 # ties go to the larger P


def test_balanced_plan_costs_less():
    E, beta, P = 8, 128, 4
    counts = np.array([4096, 256, 256, 256, 256, 256, 256, 256])
    ids = np.repeat(np.arange(E), counts).reshape(-1, 8)
    rs = route_stats(ids, E, beta)
    owner = [e * P // E for e in range(E)]
    fixed = plan(rs["block_counts"], owner, P, 0, FWD)["block_worker"]
    bal = plan(rs["block_counts"], owner, P, 3, FWD)["block_worker"]
    c_fixed = predicted_cost(counts, fixed, fixed, owner, beta, P, 256, 256, G=16)
    c_bal = predicted_cost(counts, bal, bal, owner, beta, P, 256, 256, G=16)
    assert c_bal < c_fixed
