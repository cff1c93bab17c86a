"""GPU parity of the forward expert layer against the dense per-token oracle:
fp32 within rel-L2 1e-5, bf16 within 2e-2, fp8 weights within 6e-2; output
bitwise independent of the plan; saved [G, U] rows; device status bits."""
import numpy as np
import pytest
import torch

from moe_expert_ffn_amd import binding as B
from moe_expert_ffn_amd.inputs import WORKLOADS, Workload
from oracle import ffn as offn
from oracle.route import route_stats as oracle_route
from tests.conftest import rel_l2
from tests.gpu_util import Case, say

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}

SMALL = {
    # several M and N tiles, ragged last blocks, d_ff not a multiple of 128
    "small_bf16": Workload("small_bf16", "bf16", "bf16", T=300, k=4, E=16, d=256, d_ff=192,
                           beta=128, P=4, s=2, kappas=(0,), cfg_id=11),
    # blocks smaller than a tile
    "beta32_bf16": Workload("beta32_bf16", "bf16", "bf16", T=200, k=3, E=12, d=128, d_ff=128,
                            beta=32, P=8, s=2, kappas=(0,), cfg_id=12),
    # blocks larger than a tile
    "beta256_bf16": Workload("beta256_bf16", "bf16", "bf16", T=500, k=2, E=4, d=384, d_ff=64,
                             beta=256, P=2, s=1, kappas=(0,), cfg_id=13),
    "small_f32": Workload("small_f32", "f32", "f32", T=150, k=3, E=6, d=256, d_ff=128,
                          beta=16, P=2, s=1, kappas=(0,), cfg_id=14),
    "small_fp8": Workload("small_fp8", "bf16", "fp8", T=160, k=2, E=8, d=256, d_ff=256,
                          beta=128, P=4, s=2, kappas=(0,), cfg_id=15),
    # e4m3 weights off the 256 grid: the register-staged tile kernels
    "odd_fp8": Workload("odd_fp8", "bf16", "fp8", T=240, k=3, E=6, d=384, d_ff=128,
                        beta=64, P=2, s=1, kappas=(0,), cfg_id=17),
    # e4m3 weights on the stream kernels with several tiles each way and replicas
    "stream_fp8": Workload("stream_fp8", "bf16", "fp8", T=700, k=4, E=8, d=512, d_ff=512,
                           beta=128, P=8, s=4, kappas=(0,), cfg_id=18),
    # d and d_ff multiples of 256: the persistent 256 x 256 tile kernels, with
    # several tiles in both directions, ragged blocks and replicated experts
    "stream_bf16": Workload("stream_bf16", "bf16", "bf16", T=700, k=4, E=8, d=512, d_ff=256,
                            beta=128, P=8, s=4, kappas=(0,), cfg_id=16),
}


def _tol(w):
    return TOL["fp8"] if w.wdt == "fp8" else TOL[w.act]


def _run(case, s=None, P=None):
    r = case.runner
    r.status.zero_()
    r.step(case.x, case.gates, case.ids, s=s)
    torch.cuda.synchronize()
    return r.y.clone()


@pytest.mark.parametrize("name", ["tiny_f32", *SMALL])
def test_forward_full_parity(name):
    w = WORKLOADS.get(name) or SMALL[name]
    say(f"[fwd] {name}")
    c = Case(w, 0)
    y = _run(c)
    assert c.status() == 0
    x, w1, w2, ids, gates = c.oracle_inputs()
    ref = offn.forward(x, w1, w2, ids, gates)
    err = rel_l2(y.double().cpu().numpy(), ref)
    say(f"  rel_l2={err:.3e}")
    assert err <= _tol(w)


@pytest.mark.parametrize("name", ["tiny_f32", "small_bf16", "beta32_bf16", "stream_bf16", "odd_fp8",
                                  "stream_fp8"])
def test_forward_plan_invariance(name):
    w = WORKLOADS.get(name) or SMALL[name]
    say(f"[fwd-invariance] {name}")
    c = Case(w, 0)
    y_plan = _run(c)
    y_fixed = _run(c, s=0)
    assert torch.equal(y_plan, y_fixed)
    c1 = Case(w, 0, P=1, s=0)
    assert torch.equal(_run(c1), y_plan)
    c8 = Case(w, 0, P=8, s=8)
    assert torch.equal(_run(c8), y_plan)


def test_forward_saves_z():
    w = SMALL["small_bf16"]
    c = Case(w, 0, backward=True)       # a backward-capable runner keeps [G, U]
    _run(c)
    x, w1, w2, ids, gates = c.oracle_inputs()
    _, zs = offn.forward(x, w1, w2, ids, gates, return_z=True)
    rs = oracle_route(ids, w.E, w.beta)
    zg = c.runner.z.double().cpu().numpy()
    got, ref = [], []
    for e, (toks, j, z) in zs.items():
        slots = rs["row_to_slot"][toks * w.k + j]
        got.append(zg[slots])
        ref.append(z)
    err = rel_l2(np.concatenate(got), np.concatenate(ref))
    say(f"  z rel_l2={err:.3e}")
    assert err <= TOL["bf16"]


# every skew level each workload is run at
FULL = [(name, kappa) for name in ("olmoe_bf16", "qwen3_bf16", "dsv3_fp8")
        for kappa in WORKLOADS[name].kappas]


@pytest.mark.parametrize("name,kappa", FULL)
def test_forward_full_size_sampled(name, kappa):
    w = WORKLOADS[name]
    say(f"[fwd-full] {name} kappa={kappa}")
    c = Case(w, kappa)
    y = _run(c)
    assert c.status() == 0
    info = c.runner.plan_f["plan_info"].cpu().numpy()
    say(f"  plan_info={info.tolist()}")
    rng = np.random.default_rng(kappa)
    tok = np.sort(rng.choice(c.T, size=48, replace=False))
    x, w1, w2, ids, gates = c.oracle_inputs()
    ref = offn.forward(x, w1, w2, ids, gates, tokens=tok)
    err = rel_l2(y[tok].double().cpu().numpy(), ref)
    say(f"  rel_l2={err:.3e}")
    assert err <= _tol(w)
    assert torch.isfinite(y.float()).all()


def test_forward_status_bad_plan():
    w = SMALL["small_bf16"]
    c = Case(w, 0)
    r = c.runner
    r.route(c.ids)
    r.make_plan()
    bw = r.plan_f["block_worker"].clone()
    bw[0] = 9                                   # worker outside [0, P)
    r.status.zero_()
    r.forward(c.x, c.gates, c.ids, block_worker=bw)
    torch.cuda.synchronize()
    assert c.status() & B.DEV_BAD_PLAN
