"""GPU parity of the fp8 MFMA path (MOE_EXEC_FP8_ACT) and its activation
quantizer.

- The quantizer (moe_quantize_act_rows) is bit-exact against the oracle's
  power-of-two row blocks: codes and exponents.
- The forward (FC1 and FC2 on the fp8 MFMA) is checked two ways:
  - against the oracle's fp8-operand forward (x and A quantized the same
    way), where only accumulation order and the bf16 roundings differ: saved
    [G, U] within 1e-2, y within 2e-2;
  - against the exact oracle (bf16 x, dequantized weights) within the e4m3
    bar of 6e-2.
- Placement does not change a bit. A zero weight-scale block adds nothing.
- The backward (dA and dX on the fp8 MFMA, dy and dZ quantized per row
  block) against the oracle's fp8-operand backward, which decides the e4m3
  codes on the same bf16 values the layer stores: dx, dW1 and dW2 within
  2e-2; against the exact backward within 3 * 2^-4, the bound the oracle's
  own pin uses for three quantizations.
"""
import numpy as np
import pytest
import torch

from moe_expert_ffn_amd import binding as B
from moe_expert_ffn_amd.inputs import WORKLOADS, Workload
from oracle import ffn as offn
from oracle.fp8 import quantize_row_blocks_pow2
from oracle.route import route_stats as oracle_route
from tests.conftest import rel_l2
from tests.gpu_util import Case, say

pytestmark = pytest.mark.gpu

TOL_MODEL_Z = 1e-2      # [G, U] against the fp8-operand oracle (bf16 storage)
TOL_MODEL_Y = 2e-2      # y against the same
TOL_EXACT = 6e-2        # y against the exact oracle (the e4m3 bar)
TOL_MODEL_DX = 2e-2     # dx against the fp8-operand backward oracle
TOL_MODEL_DW = 2e-2     # dW1, dW2 against the same
TOL_EXACT_BWD = 3 * 2.0 ** -4   # dx, dW against the exact backward

SMALL = {
    # one tile each way, ragged blocks
    "small_fp8": Workload("small_fp8", "bf16", "fp8", T=160, k=2, E=8, d=256, d_ff=256,
                          beta=128, P=4, s=2, kappas=(0,), cfg_id=15),
    # several tiles each way, replicas, a K loop of 4 steps
    "stream_fp8": Workload("stream_fp8", "bf16", "fp8", T=700, k=4, E=8, d=512, d_ff=512,
                           beta=128, P=8, s=4, kappas=(0,), cfg_id=18),
}


def _run(c, fp8_act=True, s=None):
    r = c.runner
    r.fp8_act = fp8_act
    r.status.zero_()
    r.step(c.x, c.gates, c.ids, s=s)
    torch.cuda.synchronize()
    assert c.status() == 0
    return r.y.clone()


def test_quantize_act_rows_matches_oracle():
    g = torch.Generator(device="cuda").manual_seed(5)
    rows, cols = 300, 1024
    x = torch.randn(rows, cols, device="cuda", generator=g)
    x *= torch.pow(10.0, torch.empty(rows, 1, device="cuda").uniform_(-6, 6, generator=g))
    x[7, 256:384] = 0.0                                  # a zero block
    x[9] = 0.0                                           # a zero row
    x[11, :128] *= 1e-3
    x[11, 5] = 448.0 * 2.0 ** 3                          # amax exactly on a binade edge
    x[12, 130] = -3.0e38                                 # near the top of the range
    xb = x.to(torch.bfloat16).contiguous()
    codes = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    exps = torch.empty(cols // 128, rows, dtype=torch.int32, device="cuda")
    B.quantize_act_rows(xb, codes, exps)
    torch.cuda.synchronize()
    rc, re = quantize_row_blocks_pow2(xb.float().cpu().numpy())
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    np.testing.assert_array_equal(exps.cpu().numpy(), re.T)
    assert int(exps[2, 7]) == -127 and int(exps[0, 11]) == 3


def _z_check(c, zg):
    """Saved [G, U] of every routed row against the fp8-operand oracle."""
    x, w1, w2, ids, gates = c.oracle_inputs()
    _, zs = offn.forward_fp8act(x, w1, w2, ids, gates, return_z=True)
    rs = oracle_route(ids, c.w.E, c.w.beta)
    got, ref = [], []
    for e, (toks, j, z) in zs.items():
        got.append(zg[rs["row_to_slot"][toks * c.w.k + j]])
        ref.append(z)
    return rel_l2(np.concatenate(got), np.concatenate(ref))


@pytest.mark.parametrize("name", list(SMALL))
def test_fp8_act_forward_parity(name):
    w = SMALL[name]
    say(f"[fp8-act] {name}")
    c = Case(w, 0, backward=True)          # a backward-capable runner keeps [G, U]
    y0 = _run(c, fp8_act=False)
    y = _run(c)
    x, w1, w2, ids, gates = c.oracle_inputs()
    ez = _z_check(c, c.runner.z.double().cpu().numpy())
    ym = rel_l2(y.double().cpu().numpy(), offn.forward_fp8act(x, w1, w2, ids, gates))
    ye = rel_l2(y.double().cpu().numpy(), offn.forward(x, w1, w2, ids, gates))
    moved = rel_l2(y.double().cpu().numpy(), y0.double().cpu().numpy())
    say(f"  z vs fp8-operand oracle {ez:.3e}, y {ym:.3e}; y vs exact {ye:.3e}; "
        f"vs the bf16-x path {moved:.3e}")
    assert ez <= TOL_MODEL_Z and ym <= TOL_MODEL_Y and ye <= TOL_EXACT
    assert moved > 1e-4                    # the flag took the fp8 path
    assert torch.isfinite(y.float()).all()


def test_fp8_act_plan_invariance():
    w = SMALL["stream_fp8"]
    say("[fp8-act] plan invariance")
    c = Case(w, 0)
    y_plan = _run(c)
    assert torch.equal(_run(c, s=0), y_plan)
    assert torch.equal(_run(Case(w, 0, P=1, s=0)), y_plan)


def test_fp8_act_zero_scale_block():
    """A weight block whose scale is 0 contributes nothing; the blocks after
    it keep their own scales."""
    w = SMALL["stream_fp8"]
    say("[fp8-act] zero weight-scale blocks")
    c = Case(w, 0, backward=True)
    c.w1s[1, 2, 0] = 0.0                   # expert 1, G rows 256..383, K 0..127
    c.w1s[3, 5, 3] = 0.0                   # expert 3, U rows, the last K block
    c.w1s[3, 5, 1] = 0.0
    _run(c)
    ez = _z_check(c, c.runner.z.double().cpu().numpy())
    say(f"  z vs fp8-operand oracle {ez:.3e}")
    assert ez <= TOL_MODEL_Z


@pytest.mark.parametrize("kappa", [1, 8])
def test_fp8_act_full_size_sampled(kappa):
    w = WORKLOADS["dsv3_fp8"]
    say(f"[fp8-act] dsv3_fp8 kappa={kappa}")
    c = Case(w, kappa)
    y = _run(c)
    rng = np.random.default_rng(kappa + 100)
    tok = np.sort(rng.choice(c.T, size=48, replace=False))
    x, w1, w2, ids, gates = c.oracle_inputs()
    yt = y[tok].double().cpu().numpy()
    ym = rel_l2(yt, offn.forward_fp8act(x, w1, w2, ids, gates, tokens=tok))
    ye = rel_l2(yt, offn.forward(x, w1, w2, ids, gates, tokens=tok))
    say(f"  y vs fp8-operand oracle {ym:.3e}; vs exact {ye:.3e}")
    assert ym <= TOL_MODEL_Y and ye <= TOL_EXACT
    assert torch.isfinite(y.float()).all()


def test_fp8_act_rejected_where_unsupported():
    """bf16 weights and the two-phase launch refuse the flag, in the forward
    and the backward."""
    say("[fp8-act] refusals")
    c = Case(SMALL["small_fp8"], 0)
    r = c.runner
    r.route(c.ids)
    r.make_plan()
    with pytest.raises(B.MoeError):
        B.forward(r.layer, c.x, c.gates, c.ids, r.beta, r.P, r.rs, r.plan_f["block_worker"], r.y,
                  r.z, r.ws, r.status, two_phase=True, fp8_act=True)
    cb = Case(WORKLOADS["tiny_f32"], 0)
    rb = cb.runner
    rb.route(cb.ids)
    rb.make_plan()
    with pytest.raises(B.MoeError):
        B.forward(rb.layer, cb.x, cb.gates, cb.ids, rb.beta, rb.P, rb.rs, rb.plan_f["block_worker"],
                  rb.y, rb.z, rb.ws, rb.status, fp8_act=True)
    cw = Case(SMALL["small_fp8"], 0, backward=True)
    rw = cw.runner
    rw.step(cw.x, cw.gates, cw.ids)
    rw.make_plan(B.PLAN_BWD, None, rw.plan_b)
    with pytest.raises(B.MoeError):
        B.backward(rw.layer, cw.x, cw.gates, cw.dy, rw.z, cw.ids, rw.beta, rw.P, rw.s, rw.rs,
                   rw.owner, rw.plan_b["block_worker"], rw.dx, rw.dw1, rw.dw2, rw.ws, rw.status,
                   two_phase=True, fp8_act=True)


def _run_bwd(c, fp8_act=True, s=None):
    r = c.runner
    r.fp8_act = fp8_act
    r.status.zero_()
    r.step(c.x, c.gates, c.ids, dy=c.dy, s=s)
    torch.cuda.synchronize()
    assert c.status() == 0
    return r.dx.clone(), r.dw1.clone(), r.dw2.clone()


def _bwd_errs(dx, dw1, dw2, o, tokens=None, experts=None):
    """rel-L2 of dx (the tokens given) and of the worst expert's dW1 and dW2,
    each expert on its own."""
    ex = range(dw1.shape[0]) if experts is None else experts
    dxs = dx if tokens is None else dx[tokens]

    def worst(dw, ref):
        return max(rel_l2(dw[e].double().cpu().numpy(), ref[e]) for e in ex)
    return rel_l2(dxs.double().cpu().numpy(), o["dx"]), worst(dw1, o["dw1"]), worst(dw2, o["dw2"])


@pytest.mark.parametrize("name", list(SMALL))
def test_fp8_act_backward_parity(name):
    w = SMALL[name]
    say(f"[fp8-act-bwd] {name}")
    c = Case(w, 0, backward=True)
    dx0, _, _ = _run_bwd(c, fp8_act=False)
    dx, dw1, dw2 = _run_bwd(c)
    x, w1, w2, ids, gates = c.oracle_inputs()
    dy = c.dy.double().cpu().numpy()
    e8 = _bwd_errs(dx, dw1, dw2, offn.backward_fp8act(x, w1, w2, ids, gates, dy, w.beta))
    e0 = _bwd_errs(dx, dw1, dw2, offn.backward(x, w1, w2, ids, gates, dy))
    moved = rel_l2(dx.double().cpu().numpy(), dx0.double().cpu().numpy())
    say(f"  vs fp8-operand oracle dx={e8[0]:.3e} dw1={e8[1]:.3e} dw2={e8[2]:.3e}; "
        f"vs exact dx={e0[0]:.3e} dw1={e0[1]:.3e} dw2={e0[2]:.3e}; dx vs the bf16-operand path "
        f"{moved:.3e}")
    assert e8[0] <= TOL_MODEL_DX and max(e8[1:]) <= TOL_MODEL_DW
    assert max(e0) <= TOL_EXACT_BWD
    assert moved > 1e-4                    # the flag took the fp8 path


def test_fp8_act_backward_plan_invariance():
    w = SMALL["stream_fp8"]
    say("[fp8-act-bwd] plan invariance")
    c = Case(w, 0, backward=True)
    dx_p, dw1_p, dw2_p = _run_bwd(c)
    dx_f, dw1_f, dw2_f = _run_bwd(c, s=0)
    assert torch.equal(dx_p, dx_f)
    assert rel_l2(dw1_p.double().cpu().numpy(), dw1_f.double().cpu().numpy()) < 1e-6
    assert rel_l2(dw2_p.double().cpu().numpy(), dw2_f.double().cpu().numpy()) < 1e-6


@pytest.mark.parametrize("kappa", [1, 8])
def test_fp8_act_backward_full_size_sampled(kappa):
    w = WORKLOADS["dsv3_fp8_fwdbwd"]
    say(f"[fp8-act-bwd] dsv3_fp8_fwdbwd kappa={kappa}")
    c = Case(w, kappa, backward=True)
    dx, dw1, dw2 = _run_bwd(c)
    counts = np.bincount(c.ids_np[c.ids_np >= 0], minlength=w.E)
    held = [e for e in range(w.E) if counts[e] > 0]
    experts = sorted({int(np.argmax(counts)), min(held, key=lambda e: (counts[e], e))})
    rng = np.random.default_rng(kappa + 200)
    tok = np.sort(rng.choice(c.T, size=32, replace=False))
    x, w1, w2, ids, gates = c.oracle_inputs()
    o = offn.backward_fp8act(x, w1, w2, ids, gates, c.dy.double().cpu().numpy(), w.beta,
                             tokens=tok, experts=experts)
    e = _bwd_errs(dx, dw1, dw2, o, tokens=tok, experts=experts)
    say(f"  experts={experts} rows={counts[experts].tolist()} dx={e[0]:.3e} dw1={e[1]:.3e} "
        f"dw2={e[2]:.3e}")
    assert e[0] <= TOL_MODEL_DX and max(e[1:]) <= TOL_MODEL_DW
    assert torch.isfinite(dx.float()).all()


def test_fp8_act_nothing_routed_writes_zeros():
    """Every id -1: the quantizers see no rows in use and the fp8 MFMA
    kernels no items; y, dx and the weight gradients are still written, as
    zeros."""
    w = SMALL["stream_fp8"]
    say("[fp8-act] nothing routed")
    T = 64
    ids = np.full((T, w.k), -1, dtype=np.int32)
    gates = np.zeros((T, w.k), dtype=np.float32)
    c = Case(w, 0, backward=True, ids=ids, gates=gates)
    r = c.runner
    for t in (r.y, r.dx, r.dw1, r.dw2):
        t.fill_(float("nan"))
    dx, dw1, dw2 = _run_bwd(c)
    for name, t in (("y", r.y), ("dx", dx), ("dw1", dw1), ("dw2", dw2)):
        assert not torch.isnan(t).any(), f"{name} left unwritten"
        assert torch.count_nonzero(t) == 0, f"{name} not zero"


def test_fp8_act_backward_two_workers_quota_plans():
    """Two workers with quota plans (the partition count the cost model picks
    for the DeepSeek-V3 share at high kappa), replicas in both directions:
    the same parity as with the default plans."""
    w = SMALL["stream_fp8"]
    say("[fp8-act-bwd] P=2, quota plans")
    c = Case(w, 0, P=2, backward=True)
    c.runner.quota_umin = 1
    dx, dw1, dw2 = _run_bwd(c)
    say(f"  plans fwd={c.runner.plan_f['plan_info'].cpu().numpy().tolist()} "
        f"bwd={c.runner.plan_b['plan_info'].cpu().numpy().tolist()}")
    x, w1, w2, ids, gates = c.oracle_inputs()
    dy = c.dy.double().cpu().numpy()
    e8 = _bwd_errs(dx, dw1, dw2, offn.backward_fp8act(x, w1, w2, ids, gates, dy, w.beta))
    ym = rel_l2(c.runner.y.double().cpu().numpy(), offn.forward_fp8act(x, w1, w2, ids, gates))
    say(f"  y {ym:.3e}; dx={e8[0]:.3e} dw1={e8[1]:.3e} dw2={e8[2]:.3e}")
    assert ym <= TOL_MODEL_Y and e8[0] <= TOL_MODEL_DX and max(e8[1:]) <= TOL_MODEL_DW
