"""The optional per-workgroup timeline of the persistent GEMM phases: writing
it changes no output bit, and every workgroup of each phase's launch leaves a
start and an end stamp (end >= start) while the entries past the launch stay
untouched."""
import numpy as np
import pytest
import torch

from moe_expert_ffn_amd import binding as B
from moe_expert_ffn_amd.inputs import Workload
from tests.gpu_util import Case, say

pytestmark = pytest.mark.gpu

W = Workload("timeline_bf16", "bf16", "bf16", T=700, k=4, E=8, d=512, d_ff=256, beta=128, P=8,
             s=4, kappas=(0,), cfg_id=27)


def _step(c, timeline=None):
    r = c.runner
    r.status.zero_()
    r.step(c.x, c.gates, c.ids, dy=c.dy, timeline=timeline)
    torch.cuda.synchronize()
    assert c.status() == 0
    return [t.clone() for t in (r.y, r.dx, r.dw1, r.dw2)]


def test_timeline_changes_nothing_and_stamps_every_workgroup():
    say("[timeline] timeline_bf16")
    c = Case(W, 0, backward=True)
    ref = _step(c)
    tl = B.alloc_timeline(c.x.device)
    got = _step(c, tl)
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    t = tl.cpu().numpy()
    for ph in range(B.TL_PHASES):
        written = np.nonzero(t[ph, :, 0])[0]
        n = len(written)
        say(f"  phase {ph}: {n} workgroups")
        assert n >= 8 and n % 8 == 0 and np.array_equal(written, np.arange(n))
        assert np.all(t[ph, :n, 1] >= t[ph, :n, 0])
        assert np.all(t[ph, n:] == 0)
    # the phases of one step run in order on one stream
    assert t[B.TL_FC2, :, 0][t[B.TL_FC2, :, 0] > 0].min() >= t[B.TL_FC1, :, 0][t[B.TL_FC1, :, 0] > 0].min()
    assert t[B.TL_DW, :, 0][t[B.TL_DW, :, 0] > 0].min() >= t[B.TL_DX, :, 1].max()
