"""GPU parity of the backward expert layer against the oracle's gradients:
dx, dW1, dW2 (fp32 weight gradients with replica partials reduced into the
owner slot), for planned and fixed placement; dx bitwise independent of the
plan."""
import numpy as np
import pytest
import torch

from moe_expert_ffn_amd.inputs import WORKLOADS, Workload
from oracle import ffn as offn
from tests.conftest import rel_l2
from tests.gpu_util import Case, say

pytestmark = pytest.mark.gpu

SMALL = {
    "small_bf16": Workload("small_bf16", "bf16", "bf16", T=300, k=4, E=16, d=256, d_ff=192,
                           beta=128, P=4, s=2, kappas=(0,), cfg_id=21),
    "beta32_bf16": Workload("beta32_bf16", "bf16", "bf16", T=200, k=3, E=12, d=128, d_ff=128,
                            beta=32, P=8, s=3, kappas=(0,), cfg_id=22),
    "small_f32": Workload("small_f32", "f32", "f32", T=150, k=3, E=6, d=256, d_ff=128,
                          beta=16, P=2, s=1, kappas=(0,), cfg_id=23),
    # d and d_ff multiples of 256: the persistent 256 x 256 tile kernels (dA, dX,
    # dW through the per-wave LDS store staging), replicas reduced into owners
    "stream_bf16": Workload("stream_bf16", "bf16", "bf16", T=700, k=4, E=8, d=512, d_ff=256,
                            beta=128, P=8, s=4, kappas=(0,), cfg_id=24),
    # the most experts the planner takes and tiny blocks: 4,608 block slots, so
    # the scheduler keeps block_worker in global memory instead of LDS
    "many_experts_bf16": Workload("many_experts_bf16", "bf16", "bf16", T=2048, k=8, E=512, d=128,
                                  d_ff=128, beta=4, P=8, s=2, kappas=(0,), cfg_id=25),
}


def _run(c, s=None):
    r = c.runner
    r.status.zero_()
    r.step(c.x, c.gates, c.ids, dy=c.dy, s=s)
    torch.cuda.synchronize()
    return r.dx.clone(), r.dw1.clone(), r.dw2.clone()


def _oracle(c, tokens=None, experts=None):
    x, w1, w2, ids, gates = c.oracle_inputs()
    return offn.backward(x, w1, w2, ids, gates, c.dy.double().cpu().numpy(), tokens=tokens,
                         experts=experts)


@pytest.mark.parametrize("name", ["tiny_f32", *SMALL])
def test_backward_full_parity(name):
    w = WORKLOADS.get(name) or SMALL[name]
    say(f"[bwd] {name}")
    c = Case(w, 0, backward=True)
    dx, dw1, dw2 = _run(c)
    assert c.status() == 0
    info = c.runner.plan_b["plan_info"].cpu().numpy()
    say(f"  bwd plan_info={info.tolist()}")
    o = _oracle(c)
    tol = 1e-5 if w.act == "f32" else 2e-2
    e_dx = rel_l2(dx.double().cpu().numpy(), o["dx"])
    e_w1 = rel_l2(dw1.double().cpu().numpy(), np.stack([o["dw1"][e] for e in range(w.E)]))
    e_w2 = rel_l2(dw2.double().cpu().numpy(), np.stack([o["dw2"][e] for e in range(w.E)]))
    say(f"  dx={e_dx:.3e} dw1={e_w1:.3e} dw2={e_w2:.3e}")
    assert max(e_dx, e_w1, e_w2) <= tol


@pytest.mark.parametrize("name", ["tiny_f32", "small_bf16", "beta32_bf16", "stream_bf16",
                                  "many_experts_bf16"])
def test_backward_plan_invariance(name):
    w = WORKLOADS.get(name) or SMALL[name]
    say(f"[bwd-invariance] {name}")
    c = Case(w, 0, backward=True)
    dx_p, dw1_p, dw2_p = _run(c)
    dx_f, dw1_f, dw2_f = _run(c, s=0)
    assert torch.equal(dx_p, dx_f)
    # weight gradients: the split of the row sum across workers depends on the plan
    assert rel_l2(dw1_p.double().cpu().numpy(), dw1_f.double().cpu().numpy()) < 1e-6
    assert rel_l2(dw2_p.double().cpu().numpy(), dw2_f.double().cpu().numpy()) < 1e-6


@pytest.mark.parametrize("kappa", WORKLOADS["qwen3_bf16_fwdbwd"].kappas)
def test_backward_full_size_sampled(kappa):
    w = WORKLOADS["qwen3_bf16_fwdbwd"]
    say(f"[bwd-full] kappa={kappa}")
    c = Case(w, kappa, backward=True)
    dx, dw1, dw2 = _run(c)
    assert c.status() == 0
    q = c.runner.plan_b["q"].cpu().numpy()
    info = c.runner.plan_b["plan_info"].cpu().numpy()
    say(f"  bwd plan_info={info.tolist()}")
    counts = np.bincount(c.ids_np[c.ids_np >= 0], minlength=w.E)
    hot = int(np.argmax(counts))
    replicated = [e for e in range(w.E) if (q[e] > 0).sum() > 1]
    # also the expert with the fewest rows: the shortest weight-gradient
    # segment, whose last K step is mostly padding; each expert is checked on
    # its own so that a small one is not hidden in a large one's norm
    held = [e for e in range(w.E) if counts[e] > 0]
    cold = min(held, key=lambda e: (counts[e], e))
    experts = sorted({hot, *(replicated[:1]), 5, cold})
    rng = np.random.default_rng(kappa)
    tok = np.sort(rng.choice(c.T, size=32, replace=False))
    o = _oracle(c, tokens=tok, experts=experts)
    e_dx = rel_l2(dx[tok].double().cpu().numpy(), o["dx"])
    e_w1 = max(rel_l2(dw1[e].double().cpu().numpy(), o["dw1"][e]) for e in experts)
    e_w2 = max(rel_l2(dw2[e].double().cpu().numpy(), o["dw2"][e]) for e in experts)
    say(f"  experts={experts} rows={counts[experts].tolist()} replicated={len(replicated)} "
        f"dx={e_dx:.3e} dw1={e_w1:.3e} dw2={e_w2:.3e}")
    assert max(e_dx, e_w1, e_w2) <= 2e-2


def _masked_routes(w, T, frac_tokens_masked, seed):
    """Routes with whole tokens masked (every slot -1) and, in the rest, some
    single slots masked; gates renormalised over the kept slots."""
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(w.E, size=w.k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[rng.random((T, w.k)) < 0.2] = -1
    ids[rng.random(T) < frac_tokens_masked] = -1
    g = rng.random((T, w.k)).astype(np.float32) * (ids >= 0)
    s = g.sum(axis=1, keepdims=True)
    gates = np.where(s > 0, g / np.where(s > 0, s, 1), 0).astype(np.float32)
    return ids, gates


@pytest.mark.parametrize("name", ["stream_bf16", "small_f32"])
def test_nothing_routed_writes_zeros(name):
    """No routed row at all: y, dx and every expert's weight gradients are
    written as zeros (buffers filled with NaN beforehand), status stays 0."""
    w = SMALL[name]
    say(f"[nothing-routed] {name}")
    T = 64
    ids = np.full((T, w.k), -1, dtype=np.int32)
    gates = np.zeros((T, w.k), dtype=np.float32)
    c = Case(w, 0, backward=True, ids=ids, gates=gates)
    r = c.runner
    for t in (r.y, r.dx, r.dw1, r.dw2):
        t.fill_(float("nan"))
    dx, dw1, dw2 = _run(c)
    assert c.status() == 0
    for name_, t in (("y", r.y), ("dx", dx), ("dw1", dw1), ("dw2", dw2)):
        assert not torch.isnan(t).any(), f"{name_} left unwritten"
        assert torch.count_nonzero(t) == 0, f"{name_} not zero"


def test_masked_tokens_match_oracle():
    """Whole tokens without an expert (all slots -1) and single masked slots,
    on the persistent kernels with replicas: dx of a masked token is zero and
    everything matches the oracle."""
    w = SMALL["stream_bf16"]
    say("[masked-tokens] stream_bf16")
    ids, gates = _masked_routes(w, 500, 0.3, 7)
    c = Case(w, 0, backward=True, ids=ids, gates=gates)
    c.runner.dx.fill_(float("nan"))
    dx, dw1, dw2 = _run(c)
    assert c.status() == 0
    gone = np.where((ids < 0).all(axis=1))[0]
    assert gone.size > 0 and torch.count_nonzero(dx[torch.from_numpy(gone).to(dx.device)]) == 0
    o = _oracle(c)
    refs = (o["dx"], np.stack([o["dw1"][e] for e in range(w.E)]),
            np.stack([o["dw2"][e] for e in range(w.E)]))
    for got, ref in zip((dx, dw1, dw2), refs):
        assert rel_l2(got.double().cpu().numpy(), ref) <= 2e-2


@pytest.mark.parametrize("name", ["stream_bf16", "small_bf16"])
def test_single_worker_matches_oracle(name):
    """P = 1: one worker owns every CU and every expert (no replica is possible);
    the layer still matches the oracle and dx equals the P = 8 result bit for bit."""
    w = SMALL[name]
    say(f"[single-worker] {name}")
    c1 = Case(w, 0, backward=True, P=1)
    dx1, dw1, dw2 = _run(c1)
    assert c1.status() == 0
    o = _oracle(c1)
    refs = (o["dx"], np.stack([o["dw1"][e] for e in range(w.E)]),
            np.stack([o["dw2"][e] for e in range(w.E)]))
    for got, ref in zip((dx1, dw1, dw2), refs):
        assert rel_l2(got.double().cpu().numpy(), ref) <= 2e-2
    c8 = Case(w, 0, backward=True)
    dx8, _, _ = _run(c8)
    assert torch.equal(dx1, dx8)


@pytest.mark.parametrize("name", ["stream_bf16", "many_experts_bf16"])
def test_runs_are_bitwise_deterministic(name):
    """Two steps on the same inputs give identical y, dx, dW1 and dW2, bit for
    bit: fixed tile accumulation order, slot-order combines and the fixed-order
    replica reduction (lambda 1, so the backward plan places replicas)."""
    w = SMALL[name]
    say(f"[determinism] {name}")
    c = Case(w, 0, backward=True, lam=1)
    dx_a, dw1_a, dw2_a = _run(c)
    y_a = c.runner.y.clone()
    reps = int(c.runner.plan_b["plan_info"][2].item())
    say(f"  backward replicas {reps}")
    assert reps > 0
    for t in (c.runner.y, c.runner.dx, c.runner.dw1, c.runner.dw2):
        t.fill_(float("nan"))
    dx_b, dw1_b, dw2_b = _run(c)
    assert torch.equal(y_a, c.runner.y)
    assert torch.equal(dx_a, dx_b)
    assert torch.equal(dw1_a, dw1_b) and torch.equal(dw2_a, dw2_b)


def _guarded(n, dev, guard=4096, fill=12345.0):
    """A float32 view of n elements inside a buffer with `guard` sentinel
    elements on each side."""
    buf = torch.full((n + 2 * guard,), fill, dtype=torch.float32, device=dev)
    return buf, buf[guard:guard + n]


def test_bad_backward_plan_is_flagged_and_stays_in_bounds():
    """A backward plan that breaks its constraints -- non-home experts beyond
    the replica budget, an expert whose blocks on one worker are not one run,
    or more blocks than the slot space -- sets MOE_DEV_BAD_PLAN, drops those
    segments, and writes nothing outside dw1 and dw2 (regression: such
    segments used to reach the weight-gradient kernel with expert -1)."""
    from moe_expert_ffn_amd import binding as B
    w = SMALL["stream_bf16"]
    say("[bwd-bad-plan] stream_bf16")
    c = Case(w, 0, backward=True)
    r = c.runner
    dev = c.x.device
    r.status.zero_()
    r.route(c.ids)
    r.make_plan(B.PLAN_FWD, s=0)
    r.forward(c.x, c.gates, c.ids)
    r.backward(c.x, c.gates, c.dy, c.ids, block_worker=r.plan_f["block_worker"])   # fixed placement
    torch.cuda.synchronize()
    assert c.status() == 0
    dx_ref, dw1_ref, dw2_ref = r.dx.clone(), r.dw1.clone(), r.dw2.clone()

    bc = r.rs["block_counts"].cpu().numpy()
    boff = r.rs["block_offsets"].cpu().numpy()
    owner = c.owner_np
    bw = np.repeat(owner, bc).astype(np.int32)               # every block at home
    moved = [e for e in range(w.E) if bc[e] >= 1][:2]        # all blocks on another worker
    for e in moved:
        bw[boff[e]:boff[e + 1]] = (owner[e] + 1) % w.P
    split = [e for e in range(w.E) if bc[e] >= 3 and e not in moved][:1]
    for e in split:                                          # home, other, home: two runs at home
        bw[boff[e] + 1] = (owner[e] + 2) % w.P
    assert moved and split
    cap = B.max_blocks(c.T, w.k, w.E, w.beta)
    bw = np.concatenate([bw, np.zeros(cap - len(bw), np.int32)])   # entries past sum b unused
    bw_dev = torch.from_numpy(bw).to(dev)
    n1, n2 = w.E * 2 * w.d_ff * w.d, w.E * w.d * w.d_ff
    G = 4096
    for case in ("over_budget", "too_many_blocks"):
        buf1, dw1 = _guarded(n1, dev, G)
        buf2, dw2 = _guarded(n2, dev, G)
        dx = torch.empty_like(r.dx)
        rs = dict(r.rs)
        if case == "too_many_blocks":
            bo = rs["block_offsets"].clone()
            bo[w.E] = B.max_blocks(c.T, w.k, w.E, w.beta) + 1
            rs["block_offsets"] = bo
        r.status.zero_()
        B.backward(r.layer, c.x, c.gates, c.dy, r.z, c.ids, w.beta, w.P, 0, rs, r.owner, bw_dev,
                   dx, dw1, dw2, r.ws, r.status)
        torch.cuda.synchronize()
        st = c.status()
        say(f"  {case}: status={st}")
        assert st & B.DEV_BAD_PLAN
        assert torch.all(buf1[:G] == 12345.0) and torch.all(buf1[G + n1:] == 12345.0)
        assert torch.all(buf2[:G] == 12345.0) and torch.all(buf2[G + n2:] == 12345.0)
        dw1 = dw1.view(w.E, 2 * w.d_ff, w.d)
        dw2 = dw2.view(w.E, w.d, w.d_ff)
        if case == "too_many_blocks":                        # nothing scheduled: owner slots zeroed
            assert torch.all(dw1 == 0) and torch.all(dw2 == 0)
            continue
        # rows are still computed by the plan's tiles, so dx is the fixed placement's
        assert torch.equal(dx, dx_ref)
        bad = set(moved) | set(split)
        for e in range(w.E):
            if e in bad:                                      # no segment holds them: zeros
                assert torch.all(dw1[e] == 0) and torch.all(dw2[e] == 0), e
            else:                                             # untouched experts: bit for bit
                assert torch.equal(dw1[e], dw1_ref[e]) and torch.equal(dw2[e], dw2_ref[e]), e


def test_runner_rejects_a_budget_above_its_own():
    from moe_expert_ffn_amd import binding as B
    w = SMALL["small_bf16"]
    c = Case(w, 0, backward=True)
    with pytest.raises(B.MoeError, match="replica budget"):
        c.runner.step(c.x, c.gates, c.ids, dy=c.dy, s=w.s + 1)
