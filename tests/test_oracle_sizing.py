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


# ---- producer/consumer split of the two-phase launches --------------------------
from oracle.sizing import pair_cost, select_split, split_costs  # noqa: E402


def test_split_hand_case():
    """One worker of n = 4 workgroups, one expert of 512 rows in blocks of 256
    (2 row tiles), d = d_ff = 256, forward: FC1 has nnt1 = 2 N tiles per row
    tile (4 items, c1 = 4918), FC2 nnt2 = 1 (2 items, c2 = 4612).
    - two launches: one FC1 wave + one FC2 wave = 9530;
    - temporal: every workgroup ends its FC1 item at 4918, both row tiles are
      ready then (items 0..3 over 4 workgroups end at 4918), FC2 items 0 and 1
      end at 9530;
    - n1 = 1: the producer ends its 4 items at 19672; row tile 0 is ready at
      9836 (item 1), row tile 1 at 19672; consumers end at 14448 and 24284;
    - n1 = 2: producers end at 9836; tile 0 ready at 4918 (item 1 on the
      second producer), tile 1 at 9836; consumers end at 9530 and 14448;
    - n1 = 3: producers end at 9836 (one has 2 items); tile 0 ready at 4918,
      tile 1 at 9836 (item 3 is the first producer's second); the one
      consumer runs item 0 to 9530 and item 1 from 9836 to 14448.
    Two launches and temporal tie; the tie goes to two launches."""
    bw = np.zeros(2, dtype=np.int32)
    costs = split_costs([512], bw, 256, 1, 256, 256, backward=False, G=4)
    assert costs == [9530, 9530, 24284, 14448, 14448]
    assert select_split(costs) == -1


def _simulate(T, n, mode, nnt1, nnt2, c1, c2):
    """Event-driven simulation of one worker (T row tiles): each workgroup
    keeps a queue of items in the order it takes them and runs the head of
    its queue once the head's inputs exist; first-phase completions are
    recorded as they happen, so a row tile's readiness is observed, not
    computed from a formula."""
    if mode == -1:
        ends1 = [0] * n
        for i in range(T * nnt1):
            ends1[i % n] += c1
        ends2 = [0] * n
        for i in range(T * nnt2):
            ends2[i % n] += c2
        return max(ends1) + max(ends2)
    if mode == 0:
        queues = [[(1, i) for i in range(j, T * nnt1, n)] + [(2, i) for i in range(j, T * nnt2, n)]
                  for j in range(n)]
    else:
        queues = [[(1, i) for i in range(j, T * nnt1, mode)] for j in range(mode)]
        queues += [[(2, i) for i in range(j, T * nnt2, n - mode)] for j in range(n - mode)]
    clock = [0] * len(queues)
    done1 = {}                               # row tile -> first-phase items finished, latest end
    pos = [0] * len(queues)
    while any(p < len(q) for p, q in zip(pos, queues)):
        progressed = False
        for w, q in enumerate(queues):
            while pos[w] < len(q):
                ph, i = q[pos[w]]
                if ph == 1:
                    clock[w] += c1
                    t = i // nnt1
                    cnt, last = done1.get(t, (0, 0))
                    done1[t] = (cnt + 1, max(last, clock[w]))
                else:
                    cnt, last = done1.get(i // nnt2, (0, 0))
                    if cnt < nnt1:
                        break                # inputs missing: try the other workgroups
                    clock[w] = max(clock[w], last) + c2
                pos[w] += 1
                progressed = True
        assert progressed, "deadlock"
    return max(clock)


def test_split_matches_event_simulation():
    rng = np.random.default_rng(7)
    for _ in range(40):
        n = int(rng.integers(2, 9))
        T = int(rng.integers(0, 12))
        nnt1, nnt2 = int(rng.integers(1, 7)), int(rng.integers(1, 9))
        c1, c2 = int(rng.integers(1, 9000)), int(rng.integers(1, 9000))
        for mode in range(-1, n):
            assert pair_cost([T], n, mode, nnt1, nnt2, c1, c2) == \
                _simulate(T, n, mode, nnt1, nnt2, c1, c2), (n, T, nnt1, nnt2, c1, c2, mode)


def test_split_bounds():
    """One launch never takes longer than two (a second-phase item never
    starts later than the end of the first phase plus the items ahead of it
    on its workgroup); with free producers a split costs exactly the
    consumers' waves; with free consumers, the producers' waves."""
    rng = np.random.default_rng(3)
    for _ in range(60):
        P = int(rng.choice([1, 2, 4]))
        n = int(rng.integers(2, 12))
        T = [int(t) for t in rng.integers(0, 20, size=P)]
        nnt1, nnt2 = int(rng.integers(1, 7)), int(rng.integers(1, 9))
        c1, c2 = int(rng.integers(1, 9000)), int(rng.integers(1, 9000))
        assert pair_cost(T, n, 0, nnt1, nnt2, c1, c2) <= pair_cost(T, n, -1, nnt1, nnt2, c1, c2)
        for n1 in range(1, n):
            free_p = pair_cost(T, n, n1, nnt1, nnt2, 0, c2)
            assert free_p == max(-(-t * nnt2 // (n - n1)) for t in T) * c2
            free_c = pair_cost(T, n, n1, nnt1, nnt2, c1, 0)
            assert free_c == max(-(-t * nnt1 // n1) for t in T) * c1


def test_split_costs_follow_the_plan_tiles():
    """The forward pair of a plan equals the pair cost over the plan's row
    tiles with FC1 / FC2 items; the backward pair uses dA / dX items."""
    E, beta, P = 8, 128, 2
    counts = [700, 300, 128, 0, 900, 256, 50, 513]
    ids = np.concatenate([np.full(c, e) for e, c in enumerate(counts)]).reshape(-1, 1)
    rs = route_stats(ids, E, beta)
    owner = [e * P // E for e in range(E)]
    for mode_b, backward in ((FWD, False), (BWD, True)):
        p = plan(rs["block_counts"], owner, P, 1, mode_b)
        got = split_costs(rs["counts"], p["block_worker"], beta, P, 512, 256, backward, G=16)
        assert len(got) == 16 // P + 1
        fc1, fc2 = 8000 + 196608 * 1000 // 214000, 4000 + 131072 * 1000 // 214000
        da, dx = 8000 + 655360 * 1000 // 214000, 8000 + 131072 * 1000 // 214000
        from oracle.sizing import _row_tiles
        T = _row_tiles(rs["counts"], p["block_worker"], beta, P)
        args = (1, 2, da, dx) if backward else (2, 2, fc1, fc2)
        assert got == [pair_cost(T, 8, m, *args) for m in range(-1, 8)]
