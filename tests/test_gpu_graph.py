"""The whole step (routing statistics, both plans on two streams, forward and
backward) captured in a HIP graph: no entry point allocates, synchronises or
clears memory with a memset, so the step can be captured as it is.  Every
replay must reproduce the eager step bit for bit, including after the inputs
are rewritten in place between replays (the graph reads them afresh), with the
program's own eager steps and synchronisations in between."""
import pytest
import torch

from moe_expert_ffn_amd.inputs import Workload, make_dy, make_routing, make_x
from tests.gpu_util import Case, say

pytestmark = pytest.mark.gpu

# skewed enough that the backward plan places replicas (and the reduction runs)
W = Workload("graph_bf16", "bf16", "bf16", T=900, k=4, E=16, d=512, d_ff=256, beta=128, P=8,
             s=4, kappas=(4,), cfg_id=31)


def _outs(r):
    return [t.clone() for t in (r.y, r.dx, r.dw1, r.dw2)]


def _eager(c):
    c.runner.status.zero_()
    c.runner.step(c.x, c.gates, c.ids, dy=c.dy)
    torch.cuda.synchronize()
    assert c.status() == 0
    return _outs(c.runner)


@pytest.mark.parametrize("quota", [None, 1])
def test_captured_step_replays_bit_identical(quota):
    say(f"[graph] graph_bf16 kappa 4 quota={quota}")
    c = Case(W, 4, backward=True, lam=1)
    r = c.runner
    r.quota_umin = quota
    ref = _eager(c)
    assert int(r.plan_b["plan_info"][2].item()) > 0, "the case should place backward replicas"
    # warm the capture stream once, then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        r.step(c.x, c.gates, c.ids, dy=c.dy)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        r.step(c.x, c.gates, c.ids, dy=c.dy)
    torch.cuda.synchronize()
    for rep in range(3):
        r.status.zero_()
        for t in (r.y, r.dx, r.dw1, r.dw2):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert c.status() == 0
        for a, b in zip(_outs(r), ref):
            assert torch.equal(a, b), f"replay {rep}"
        _eager(c)                                  # the program's own work between replays
    # new inputs of the same shape, written into the captured buffers
    ids, gates = make_routing(W, 4, salt=7)
    c.ids.copy_(torch.from_numpy(ids))
    c.gates.copy_(torch.from_numpy(gates))
    c.x.copy_(make_x(W, c.T, c.x.device, salt=7))
    c.dy.copy_(make_dy(W, c.T, c.x.device, salt=7))
    ref2 = _eager(c)
    assert not torch.equal(ref2[0], ref[0])
    r.status.zero_()
    g.replay()
    torch.cuda.synchronize()
    assert c.status() == 0
    for a, b in zip(_outs(r), ref2):
        assert torch.equal(a, b), "replay on rewritten inputs"
    del g
