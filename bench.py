"""Benchmark of the skew-aware MoE expert layer on one MI355X.

One step = the whole path over one batch of synthetic routed tokens:
route statistics -> forward plan -> forward (FC1+SwiGLU, FC2, combine) ->
backward plan (reduction-aware) -> backward (dA, dX, combine, weight
gradients, replica reduction).  Inputs and weights are resident in HBM before
timing starts.  The workload is the Qwen3-30B-A3B-shaped layer (T=8192,
d=2048, d_ff=768, E=128, top-8, beta=128, P=8 CU partitions, s=4) at skew
kappa=1 by default.

Prints one JSON line.  `value` is useful TFLOP/s: (6 + 12) * d * d_ff * R per
step (R = routed rows; padding rows, SwiGLU, combine not counted), divided by
the measured step time.  The same line carries `kappa_sweep`: every skew level
of the workload (kappa 1, 4, 8 for the fwd+bwd layer) under fixed placement
(s = 0), the pages' planner (lambda = 12), the planner with lambda = 1 (the
measured price of a replica on one GPU) and the quota planner, in ms and
useful TFLOP/s, and the latency ratio kappa=8 / kappa=1 of each arm (`skew`);
and `two_phase`: the same steps with FC1+FC2 and dA+dX in one launch each.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer useful TFLOP/s (fwd,bwd) at κ=1/2/4/8; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 4096 flop/clk x 2.4 GHz, dense
PEAK_FP8_TFLOPS = 5033.2       # twice the bf16 rate on the fp8 MFMA, dense
PEAK_HBM_GBS = 8000.0

# stage names between consecutive stage events, keyed by the two-phase launch
# (FC1 and FC2, dA and dX in one kernel), which records its two events back to
# back (None: that interval holds no work)
FWD_STAGES = {False: ["sched", "fc1", "fc2", "combine"], True: ["sched", "fc1+fc2", None, "combine"]}
BWD_STAGES = {False: ["sched", "dA", "dX", "combine", "dW", "reduce"],
              True: ["sched", "dA+dX", None, "combine", "dW", "reduce"]}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_bf16_fwdbwd")
    ap.add_argument("--kappa", type=float, default=1)
    ap.add_argument("--fixed", action="store_true", help="fixed placement (s = 0)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the default kappa sweep (fixed vs planned at every kappa)")
    ap.add_argument("--sweep-steps", type=int, default=10,
                    help="timed steps per arm of the default kappa sweep")
    ap.add_argument("--sweep", action="store_true",
                    help="the long sweep instead: every kappa of the workload under fixed "
                         "placement, the bounded greedy planner (lambda 12 and 1), the quota "
                         "planner and the quota planner with P chosen by the cost model, and "
                         "the two planners compared")
    ap.add_argument("--gate-sweep", action="store_true",
                    help="time near-balanced kappas: fixed placement, the planner, and the "
                         "planner behind the replication gate")
    ap.add_argument("--gate-rho", type=int, default=1000,
                    help="replication gate price per replica, thousandths of a block")
    ap.add_argument("--size-sweep", action="store_true",
                    help="time every CU partition count P at every kappa next to the "
                         "wave-quantized cost model's prediction, and report the selector's regret")
    ap.add_argument("--split-sweep", action="store_true",
                    help="time the two-launch, one-launch and producer/consumer-split modes of "
                         "the FC1 -> FC2 and dA -> dX pairs at every kappa next to "
                         "moe_predict_split's prediction, and report its choice's regret")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens of the workload in the CPU oracle sample (0: all)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the CPU oracle sample until this much time has passed")
    return ap.parse_args()


def flops_per_row(w):
    return 6 * w.d * w.d_ff, 12 * w.d * w.d_ff


def build_case(w, kappa, fixed, dev, quota_umin=None, gate_rho=None, lam=12, P=None, lay=None,
               routing=None):
    """One timed configuration.  `lay` (the layer's weights, which do not depend
    on kappa) and `routing` (make_routing's ids and gates) may be shared
    between arms."""
    import torch

    from moe_expert_ffn_amd.inputs import contiguous_owners, make_dy, make_layer, make_routing, make_x
    from moe_expert_ffn_amd.runner import LayerRunner
    ids, gates = make_routing(w, kappa) if routing is None else routing
    T = ids.shape[0]
    lay = make_layer(w, dev) if lay is None else lay
    x = lay["x"] if "x" in lay and lay["x"].shape[0] == T else make_x(w, T, dev)
    act = torch.float32 if w.act == "f32" else torch.bfloat16
    dy = make_dy(w, T, dev) if w.backward else None
    r = LayerRunner(lay["w1"], lay["w2"], lay.get("w1_scale"), lay.get("w2_scale"), act_dtype=act,
                    T=T, k=w.k, beta=w.beta, P=P or w.P, s=0 if fixed else w.s,
                    owner=torch.from_numpy(contiguous_owners(w.E, P or w.P)), with_backward=w.backward,
                    quota_umin=quota_umin, gate_rho=gate_rho, lam=lam)
    return dict(runner=r, x=x, gates=torch.from_numpy(gates).to(dev), ids=torch.from_numpy(ids).to(dev),
                dy=dy, ids_np=ids, gates_np=gates, lay=lay, T=T,
                owner_np=contiguous_owners(w.E, P or w.P))


def predicted_cost(case, w, P):
    """moe_predict_cost of the case's current plans, thousandths of a step."""
    import torch

    from moe_expert_ffn_amd import binding as B
    r = case["runner"]
    cost = torch.zeros(1, dtype=torch.int64, device=r.owner.device)
    bw_b = r.plan_b["block_worker"] if w.backward else r.plan_f["block_worker"]
    B.predict_cost(r.rs["counts"], r.rs["block_offsets"], r.plan_f["block_worker"], bw_b, r.owner,
                   w.beta, P, w.d, w.d_ff, cost, r.status)
    return int(cost.item())


def predicted_split(case, w, backward):
    """moe_predict_split of the case's current plan for one direction: the
    predicted time of every mode (dict mode -> thousandths of a step) and the
    chosen mode."""
    import torch

    from moe_expert_ffn_amd import binding as B
    r = case["runner"]
    G = B.device_info()["num_cus"]
    costs = torch.zeros(G // w.P + 1, dtype=torch.int64, device=r.owner.device)
    choice = torch.zeros(1, dtype=torch.int32, device=r.owner.device)
    bw = r.plan_b["block_worker"] if backward else r.plan_f["block_worker"]
    B.predict_split(r.rs["counts"], r.rs["block_offsets"], bw, w.beta, w.P, w.d, w.d_ff, backward,
                    costs, choice, r.status)
    c = costs.cpu().tolist()
    return {m - 1: v for m, v in enumerate(c)}, int(choice.item())


def split_sweep(w, dev, lay, steps):
    """Every kappa: the pair times (FC1 -> FC2, dA -> dX, from the stage
    events) under two launches (-1), one launch (0) and producer counts n1,
    each next to its prediction; the model's choice, the measured best and
    the choice's regret per direction."""
    import torch

    from moe_expert_ffn_amd import binding as B
    n = B.device_info()["num_cus"] // w.P
    rows, regrets = [], []
    for kap in w.kappas:
        c = build_case(w, kap, False, dev, lay=lay)
        r = c["runner"]
        time_steps(c, 1, 0, with_events=False)                  # route and plan once
        pred_f, ch_f = predicted_split(c, w, False)
        pred_b, ch_b = predicted_split(c, w, True) if w.backward else ({}, None)
        modes = sorted({-1, 0, n // 4, n // 2, (2 * n) // 3, (3 * n) // 4, n - 1, ch_f,
                        ch_b if ch_b is not None else -1})
        meas = {}
        for m in modes:
            r.two_phase = m >= 0
            r.split_fwd = r.split_bwd = max(m, 0)
            ms, st = time_steps(c, steps, 2)
            fwd = sum(v for k, v in st.items() if k in ("fwd.fc1", "fwd.fc2", "fwd.fc1+fc2"))
            bwd = sum(v for k, v in st.items() if k in ("bwd.dA", "bwd.dX", "bwd.dA+dX"))
            meas[m] = (ms, fwd * 1e3, bwd * 1e3)
        r.two_phase, r.split_fwd, r.split_bwd = False, 0, 0
        row = {"kappa": kap, "n": n, "chosen_fwd": ch_f, "chosen_bwd": ch_b, "modes": {}}
        for m, (ms, fu, bu) in meas.items():
            row["modes"][m] = {"ms": round(ms, 4), "fwd_pair_us": round(fu, 1),
                               "bwd_pair_us": round(bu, 1),
                               "pred_fwd_steps": round(pred_f[m] / 1000, 1),
                               **({"pred_bwd_steps": round(pred_b[m] / 1000, 1)} if pred_b else {})}
        best_f = min(meas, key=lambda m: meas[m][1])
        row["best_fwd"] = best_f
        row["regret_fwd"] = round(meas[ch_f][1] / meas[best_f][1] - 1, 4)
        regrets.append(row["regret_fwd"])
        if w.backward:
            best_b = min(meas, key=lambda m: meas[m][2])
            row["best_bwd"] = best_b
            row["regret_bwd"] = round(meas[ch_b][2] / meas[best_b][2] - 1, 4)
            regrets.append(row["regret_bwd"])
        rows.append(row)
        del c
        torch.cuda.empty_cache()
    return {"runs": rows, "mean_regret": round(sum(regrets) / len(regrets), 4)}


def time_steps(case, steps, warmup, with_events=True):
    """Times `steps` full steps with nothing but the layer's own launches
    between the two synchronisations (wall ms/step).  With `with_events`, the
    same number of steps is run again with HIP events recorded around every
    stage for the per-stage mean ms: each recorded event holds the stream for
    a few microseconds (about 6 us measured between kernels), so those steps
    are longer and are not the step time."""
    import torch

    from moe_expert_ffn_amd import binding as B
    r = case["runner"]
    bwd = case["dy"] is not None

    def one(evf=None, evb=None, es=None, ep=None):
        r.route(case["ids"])
        if es:
            es.record(1)
        if bwd:               # the backward plan on the runner's side stream
            r.plan_bwd_async(events=ep)
        r.make_plan(B.PLAN_FWD)
        if es:
            es.record(2)
        r.forward(case["x"], case["gates"], case["ids"], events=evf)
        if bwd:
            r.join_bwd_plan()
            r.backward(case["x"], case["gates"], case["dy"], case["ids"], events=evb)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    evs = []
    if with_events:
        for _ in range(steps):
            evs.append((B.Events(5), B.Events(7) if bwd else None, B.Events(6),
                        B.Events(2) if bwd else None))
        torch.cuda.synchronize()
        for i in range(steps):
            ef, eb, es, ep = evs[i]
            es.record(0)
            one(ef.ev, eb.ev if eb else None, es, ep)
            es.record(5)
        torch.cuda.synchronize()
    stages = {}
    if with_events:
        acc = {}
        two = r.two_phase
        for ef, eb, es, ep in evs:
            for j, nm in enumerate(FWD_STAGES[two]):
                if nm:
                    acc.setdefault("fwd." + nm, []).append(ef.elapsed_ms(j, j + 1))
            if eb:
                for j, nm in enumerate(BWD_STAGES[two]):
                    if nm:
                        acc.setdefault("bwd." + nm, []).append(eb.elapsed_ms(j, j + 1))
            acc.setdefault("route", []).append(es.elapsed_ms(0, 1))
            acc.setdefault("plan.fwd", []).append(es.elapsed_ms(1, 2))
            if ep:            # on the side stream, next to the forward plan
                acc.setdefault("plan.bwd", []).append(ep.elapsed_ms(0, 1))
            acc.setdefault("step", []).append(es.elapsed_ms(0, 5))
        stages = {k: sum(v) / len(v) for k, v in acc.items()}
        steps_sorted = sorted(acc["step"])

        def pct(q):
            return steps_sorted[min(len(steps_sorted) - 1, int(q * len(steps_sorted)))]
        stages["step_p10"], stages["step_median"], stages["step_p90"] = pct(0.1), pct(0.5), pct(0.9)
    assert int(r.status.item()) == 0, "device status word set"
    return wall_ms, stages


def kernel_model(w, R, T, e_act, replicas, red_bytes=0, slots_used=0):
    """Algorithmic flops and HBM bytes of one launch of each kernel: every
    operand read once from HBM and every output written once (weights of the
    experts that have rows, gathered activations counted once per token, the
    fp32 weight gradients of owners and replicas; the replica reduction's
    bytes come from the backward plan, see reduce_bytes).  The routing
    statistics (histogram, scan, slotting) read the T k ids and write
    row_to_slot (T k) and slot_to_row over the slots in use, int32 each."""
    d, f, ab = w.d, w.d_ff, 2
    wb = 1 if w.wdt == "fp8" else 2
    w1 = 2 * f * d * wb * e_act
    w2 = d * f * wb * e_act
    x = T * d * ab
    m = {
        "fwd.fc1": (4 * d * f * R, w1 + x + R * f * ab + (R * 2 * f * ab if w.backward else 0)),
        "fwd.fc2": (2 * d * f * R, w2 + R * f * ab + R * d * ab),
        "fwd.combine": (0, R * d * ab + x),
        "route": (0, 4 * (2 * T * w.k + slots_used)),
    }
    if w.backward:
        m.update({
            "bwd.dA": (2 * d * f * R, w2 + x + 2 * R * 2 * f * ab + R * f * ab),
            "bwd.dX": (4 * d * f * R, w1 + R * 2 * f * ab + R * d * ab),
            "bwd.combine": (0, R * d * ab + x),
            "bwd.dW": (6 * d * f * R, 2 * x + R * 2 * f * ab + R * f * ab + 3 * d * f * 4 * (e_act + replicas)),
        })
        if red_bytes > 0:
            m["bwd.reduce"] = (0, red_bytes)
    # the two-phase launches: both products, their rows written and read back
    for a, b, k in (("fwd.fc1", "fwd.fc2", "fwd.fc1+fc2"), ("bwd.dA", "bwd.dX", "bwd.dA+dX")):
        if a in m:
            m[k] = (m[a][0] + m[b][0], m[a][1] + m[b][1])
    return m


def reduce_bytes(case, w):
    """Bytes the replica reduction moves under the backward plan: for every
    expert with a replica partial, or with no owner partial, the owner
    partial (if any) and each replica partial are read and the owner slot is
    written, 3 * d * d_ff fp32 values each."""
    q = case["runner"].plan_b["q"].cpu().numpy()
    own = case["owner_np"]
    per = 3 * w.d * w.d_ff * 4
    total = 0
    for e in range(w.E):
        has_own = q[e, own[e]] > 0
        nrep = int((q[e] > 0).sum()) - int(has_own)
        if nrep > 0 or not has_own:
            total += (int(has_own) + nrep + 1) * per
    return total


# HBM traffic of the dominant kernel from rocprofv3 counters (FETCH_SIZE and
# WRITE_SIZE per dispatch, scaled by the reading of a plain copy kernel of
# known size), valid only for the kernel sources it was measured on.
PROFILED_TRAFFIC = {"kernel": "bwd.dW", "workload": "qwen3_bf16_fwdbwd", "kappa": 1.0, "fixed": False,
                    "source": "4928bdf5712c7e12", "bytes": 3335867346,
                    "summary": "profiles/k_stream_SrcDwT_qwen3_bf16_fwdbwd_hbm_traffic.md"}


def source_hash():
    import hashlib
    h = hashlib.sha256()
    src = os.path.join(ROOT, "moe_expert_ffn_amd", "csrc")
    for name in sorted(os.listdir(src)):
        with open(os.path.join(src, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def roofline(w, stages, R, T, e_act, replicas, red_bytes=0, run=None, slots_used=0):
    model = kernel_model(w, R, T, e_act, replicas, red_bytes, slots_used)
    # every contraction runs on bf16 MFMA (e4m3 weights are widened to bf16
    # between LDS and the matrix cores), so the bf16 peak bounds it
    peak_f = PEAK_BF16_TFLOPS
    rows = {}
    for k, (fl, by) in model.items():
        if k not in stages:
            continue
        t = stages[k] * 1e-3
        tf, tb = fl / (peak_f * 1e12), by / (PEAK_HBM_GBS * 1e9)
        if tf >= tb:
            rows[k] = {"bound": "mfma", "achieved": fl / t / 1e12, "peak": peak_f, "unit": "TFLOP/s"}
        else:
            rows[k] = {"bound": "hbm", "achieved": by / t / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
        rows[k].update(frac=rows[k]["achieved"] / rows[k]["peak"], launch_us=stages[k] * 1e3,
                       flops=fl, bytes=by)
    dom = max(rows, key=lambda k: rows[k]["launch_us"])
    r = rows[dom]
    traffic = None
    # the counters belong to one kernel on one workload, kappa and placement
    if PROFILED_TRAFFIC and PROFILED_TRAFFIC.get("kernel") == dom and run is not None and \
            run == (PROFILED_TRAFFIC["workload"], PROFILED_TRAFFIC["kappa"], PROFILED_TRAFFIC["fixed"]) and \
            PROFILED_TRAFFIC.get("source") == source_hash():
        traffic = PROFILED_TRAFFIC["bytes"]
    out = {"kernel": dom, "bound": r["bound"], "achieved": round(r["achieved"], 2), "peak": r["peak"],
           "unit": r["unit"], "frac": round(r["frac"], 4), "traffic": traffic,
           "launch_us": round(r["launch_us"], 2), "algorithmic_flops": r["flops"],
           "algorithmic_bytes": r["bytes"]}
    per = {k: {"bound": v["bound"], "frac": round(v["frac"], 4), "us": round(v["launch_us"], 1),
               "achieved": round(v["achieved"], 1), "unit": v["unit"]}
           for k, v in rows.items()}
    return out, per


def compare_planners(case, w, n=50):
    """Both planners on this case's route statistics: objective (max blocks per
    worker), replicas and mean on-device time of one moe_plan call."""
    import torch

    from moe_expert_ffn_amd import binding as B
    r = case["runner"]
    r.route(case["ids"])
    out = {}
    for name, mode, lam in (("greedy_fwd", B.PLAN_FWD, r.lam), ("quota_umin1", B.PLAN_QUOTA, 1)):
        plan = B.alloc_plan(r.E, r.P, B.max_blocks(r.T, r.k, r.E, r.beta), r.dev)
        args = (r.rs["block_counts"], r.rs["block_offsets"], r.owner, r.P, w.s, mode, lam, plan,
                r.ws, r.status)
        for _ in range(5):
            B.plan(*args)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            B.plan(*args)
        e1.record()
        torch.cuda.synchronize()
        info = plan["plan_info"].cpu().tolist()
        out[name] = {"objective": info[0], "replicas": info[2], "tau": info[3],
                     "us": round(e0.elapsed_time(e1) * 1e3 / n, 2)}
    return out


# (name, fixed placement, lambda, quota floor u_min or None): the pages'
# bounded greedy at its lambda = 12 and at lambda = 1 (a replica's price on one
# GPU), and the quota planner (every plan, forward and backward)
SWEEP_ARMS = (("fixed", True, 12, None), ("planned", False, 12, None),
              ("planned-lambda1", False, 1, None), ("planned-quota", False, 12, 1))
TL_NAMES = ("fc1", "fc2", "dA", "dX", "dW")


def worker_spread(tl, P):
    """Per phase of one step's timeline: each worker's finish (its last
    workgroup's end, from the phase's first start) over the mean finish of the
    P workers; 1.0 is perfectly balanced.  Workgroup g belongs to worker
    (g % 8) * P / 8."""
    import numpy as np
    out = {}
    for ph, name in enumerate(TL_NAMES):
        st, en = tl[ph, :, 0], tl[ph, :, 1]
        n = int((st > 0).sum())
        if n == 0:
            continue
        g = np.arange(n)
        w = (g % 8) * P // 8
        t0 = st[:n].min()
        fin = np.array([en[:n][w == r].max() - t0 for r in range(P)], dtype=np.float64)
        out[name] = round(float(fin.max() / fin.mean()), 3)
    return out


def timeline_step(case):
    """One more step of the case with the library's per-workgroup timeline."""
    import torch

    from moe_expert_ffn_amd import binding as B
    r = case["runner"]
    tl = B.alloc_timeline(r.owner.device)
    r.route(case["ids"])
    r.make_plan(B.PLAN_FWD)
    r.forward(case["x"], case["gates"], case["ids"], timeline=tl)
    if case["dy"] is not None:
        r.make_plan(B.PLAN_BWD, out=r.plan_b)
        r.backward(case["x"], case["gates"], case["dy"], case["ids"], timeline=tl)
    torch.cuda.synchronize()
    return tl.cpu().numpy()


def kappa_sweep(w, dev, lay, steps, warmup=3):
    """Every kappa of the workload under each arm of SWEEP_ARMS: ms per step
    (wall clock over `steps` steps, no stage events), useful TFLOP/s and its share of the
    bf16 peak, the forward and backward stage sums, and the plans' objectives.
    Returns (rows, skew) with skew[arm] = ms(max kappa) / ms(kappa 1)."""
    import torch

    from moe_expert_ffn_amd.inputs import make_routing, realised_kappa
    f_fwd, f_bwd = flops_per_row(w)
    rows = []
    for kap in w.kappas:
        routing = make_routing(w, kap)
        R = int((routing[0] >= 0).sum())
        useful = (f_fwd + (f_bwd if w.backward else 0)) * R
        for arm, fixed, lam, umin in SWEEP_ARMS:
            c = build_case(w, kap, fixed, dev, lam=lam, lay=lay, routing=routing, quota_umin=umin)
            ms, st = time_steps(c, steps, warmup)
            spread = worker_spread(timeline_step(c), c["runner"].P)
            pf = c["runner"].plan_f["plan_info"].cpu().tolist()
            pb = c["runner"].plan_b["plan_info"].cpu().tolist() if w.backward else None
            rows.append({"kappa": kap, "kappa_realised": round(realised_kappa(routing[0], w.E), 3),
                         "placement": arm, "lambda": lam if umin is None else None,
                         "quota_umin": umin, "ms": round(ms, 4),
                         "tflops": round(useful / (ms * 1e-3) / 1e12, 2),
                         "pct_bf16_peak": round(100 * useful / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                         "fwd_us": round(sum(v for k_, v in st.items() if k_.startswith("fwd.")) * 1e3, 1),
                         "bwd_us": round(sum(v for k_, v in st.items() if k_.startswith("bwd.")) * 1e3, 1),
                         "objective_fwd": pf[0], "replicas_fwd": pf[2],
                         **({"objective_bwd": pb[0], "replicas_bwd": pb[2]} if pb else {}),
                         "worker_spread": spread})
            del c
            torch.cuda.empty_cache()
    skew = {}
    k_lo, k_hi = min(w.kappas), max(w.kappas)
    for arm, *_ in SWEEP_ARMS:
        t = {r["kappa"]: r["ms"] for r in rows if r["placement"] == arm}
        skew[arm] = round(t[k_hi] / t[k_lo], 4)
    return rows, {"kappa_hi": k_hi, "kappa_lo": k_lo, "ratio": skew}


def cpu_baseline(case, w, tokens, min_seconds):
    """The oracle, untuned, on the first `tokens` tokens (0: all) of the same
    workload: forward of those tokens plus their dx, and dW of every expert
    over their rows, in passes until at least `min_seconds` have elapsed.
    Useful TFLOP/s of those passes."""
    import numpy as np

    from oracle import ffn as offn
    from oracle.fp8 import dequant_blocks
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    n = case["T"] if tokens <= 0 else min(tokens, case["T"])
    ids = case["ids_np"][:n]
    gates = case["gates_np"][:n].astype(np.float64)
    lay = case["lay"]
    x = case["x"][:n].double().cpu().numpy()
    if w.wdt == "fp8":        # the oracle takes the dequantized weights
        w1 = dequant_blocks(lay["w1"].cpu().numpy(), lay["w1_scale"].cpu().numpy())
        w2 = dequant_blocks(lay["w2"].cpu().numpy(), lay["w2_scale"].cpu().numpy())
    else:
        w1 = lay["w1"].double().cpu().numpy()
        w2 = lay["w2"].double().cpu().numpy()
    dy = case["dy"][:n].double().cpu().numpy() if case["dy"] is not None else None
    rows = int((ids >= 0).sum())
    f_fwd, f_bwd = flops_per_row(w)
    passes, flops = 0, 0.0
    t_fwd, t_bwd = [], []
    t0 = time.perf_counter()
    while True:
        ta = time.perf_counter()
        offn.forward(x, w1, w2, ids, gates)
        t_fwd.append(time.perf_counter() - ta)
        flops += f_fwd * rows
        if dy is not None:
            ta = time.perf_counter()
            offn.backward(x, w1, w2, ids, gates, dy)
            t_bwd.append(time.perf_counter() - ta)
            flops += f_bwd * rows
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= 10:
            break
    what = "all" if n == case["T"] else f"first {n} of"
    out = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
           "sample": f"{what} {case['T']} tokens ({rows} routed rows), {passes} pass"
                     f"{'es' if passes > 1 else ''}: dense fp64 forward"
                     f"{' + backward (dx, dW)' if dy is not None else ''}, numpy",
           "seconds": dt}
    out["stages_ms"] = cpu_stages(case, w, ids, t_fwd, t_bwd)
    out["cpu_model"] = cpu_model()
    return out


def cpu_stages(case, w, ids, t_fwd, t_bwd):
    """Median milliseconds of each oracle stage on the same sample: routing
    statistics and the two plans (pure Python, one thread; three runs each),
    and the forward and backward passes timed above (numpy on the BLAS
    threads)."""
    import numpy as np

    from oracle import plan as oplan
    from oracle import route as oroute

    def med3(f):
        ts = []
        for _ in range(3):
            ta = time.perf_counter()
            res = f()
            ts.append(time.perf_counter() - ta)
        return float(np.median(ts)) * 1e3, res

    t_route, rs = med3(lambda: oroute.route_stats(ids, w.E, w.beta))
    own = case["owner_np"]
    t_pf, _ = med3(lambda: oplan.plan(rs["block_counts"], own, w.P, w.s, oplan.FWD))
    t_pb, _ = med3(lambda: oplan.plan(rs["block_counts"], own, w.P, w.s, oplan.BWD, 12))
    st = {"route_1thread": round(t_route, 2), "plan_fwd_1thread": round(t_pf, 3),
          "plan_bwd_1thread": round(t_pb, 3), "forward": round(float(np.median(t_fwd)) * 1e3, 1)}
    if t_bwd:
        st["backward"] = round(float(np.median(t_bwd)) * 1e3, 1)
    return st


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the layer's P workers are CU partitions of a single "
              f"MI355X; --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import torch

    from moe_expert_ffn_amd import binding as B
    from moe_expert_ffn_amd.inputs import WORKLOADS, realised_kappa
    B.load()
    dev = torch.device("cuda:0")
    w = WORKLOADS[args.workload]
    from moe_expert_ffn_amd.inputs import make_layer
    lay = make_layer(w, dev)                        # weights do not depend on kappa: shared
    case = build_case(w, args.kappa, args.fixed, dev, lay=lay)
    R = int((case["ids_np"] >= 0).sum())
    ms, stages = time_steps(case, args.steps, args.warmup)
    # the same steps with FC1 / FC2 and dA / dX in one two-phase launch each
    case["runner"].two_phase = True
    ms_two, stages_two = time_steps(case, args.steps, args.warmup)
    case["runner"].two_phase = False
    f_fwd, f_bwd = flops_per_row(w)
    useful = (f_fwd + (f_bwd if w.backward else 0)) * R
    value = useful / (ms * 1e-3) / 1e12

    import numpy as np
    e_act = int((np.bincount(case["ids_np"][case["ids_np"] >= 0].ravel(), minlength=w.E) > 0).sum())
    replicas = int(case["runner"].plan_b["plan_info"][2].item()) if w.backward else 0
    red_bytes = reduce_bytes(case, w) if w.backward else 0
    cnt = np.bincount(case["ids_np"][case["ids_np"] >= 0].ravel(), minlength=w.E)
    slots_used = int((-(-cnt // w.beta)).sum() * w.beta)
    roof, per_kernel = roofline(w, stages, R, case["T"], e_act, replicas, red_bytes,
                                run=(w.name, float(args.kappa), bool(args.fixed)),
                                slots_used=slots_used)
    _, per_two = roofline(w, stages_two, R, case["T"], e_act, replicas, red_bytes,
                          slots_used=slots_used)
    for k in ("fwd.fc1+fc2", "bwd.dA+dX"):
        if k in per_two:
            per_kernel[k + " (two-phase launch)"] = per_two[k]

    plan_f = case["runner"].plan_f["plan_info"].cpu().tolist()
    plan_b = case["runner"].plan_b["plan_info"].cpu().tolist() if w.backward else None
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded routing, random-init weights)",
        "config": {"workload": f"{w.name}: T={case['T']} d={w.d} d_ff={w.d_ff} E={w.E} top-{w.k} "
                               f"beta={w.beta} P={w.P} s={0 if args.fixed else w.s} "
                               f"kappa={args.kappa:g} ({'fwd+bwd' if w.backward else 'fwd'})",
                   "kappa_realised": round(realised_kappa(case["ids_np"], w.E), 4),
                   "routed_rows": R, "placement": "fixed" if args.fixed else "planned",
                   "plan_info_fwd": plan_f,
                   **({"plan_info_bwd": plan_b, "reduce_bytes": red_bytes} if w.backward else {})},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        # per-stage means from a second pass of the same steps with HIP events
        # around every stage (each event holds the stream a few microseconds,
        # so "step" there is above ms_per_step)
        "stages_us": {k: round(v * 1e3, 2) for k, v in stages.items()},
        # FC1 / FC2 and dA / dX in one two-phase launch each (MOE_EXEC_TWO_PHASE)
        "two_phase": {"ms_per_step": round(ms_two, 4),
                      "stages_us": {k: round(v * 1e3, 2) for k, v in stages_two.items()}},
        "roofline": roof,
        "kernels": per_kernel,
    }
    if w.wdt == "fp8":
        # the same steps with FC1, FC2 (and with a backward dA, dX) on the fp8
        # MFMA (MOE_EXEC_FP8_ACT: x, A, dy and dZ quantized per row block of
        # 128 features), each of those stages priced against the fp8 peak; the
        # fc1 stage includes the quantization of x and A, the dA stage that of
        # dy, the requantization of D and the SwiGLU gradient pass that
        # quantizes dZ
        case["runner"].fp8_act = True
        ms_f8, st_f8 = time_steps(case, args.steps, args.warmup)
        case["runner"].fp8_act = False
        gemm = {"fwd.fc1": 4 * w.d * w.d_ff * R, "fwd.fc2": 2 * w.d * w.d_ff * R,
                "bwd.dA": 2 * w.d * w.d_ff * R, "bwd.dX": 4 * w.d * w.d_ff * R}
        out["fp8_act"] = {
            "ms_per_step": round(ms_f8, 4),
            "tflops": round(useful / (ms_f8 * 1e-3) / 1e12, 3),
            "stages_us": {k: round(v * 1e3, 2) for k, v in st_f8.items()},
        }
        for k, fl in gemm.items():
            us = st_f8.get(k, 0.0) * 1e3
            if us:
                tf = fl / (us * 1e-6) / 1e12
                out["fp8_act"][k] = {"tflops": round(tf, 1),
                                     "pct_fp8_peak": round(100 * tf / PEAK_FP8_TFLOPS, 2)}
    if not args.sweep and not args.no_sweep and len(w.kappas) > 1:
        out["kappa_sweep"], out["skew"] = kappa_sweep(w, dev, lay, args.sweep_steps)
    if args.sweep:
        sweep, planners = [], []
        arms = [("fixed", True, None, 12, False), ("planned", False, None, 12, False),
                ("planned-lambda1", False, None, 1, False), ("planned-quota", False, 1, 12, False)]
        if w.wdt == "fp8":      # the same quota plans with the products on the fp8 MFMA
            arms.append(("planned-quota-fp8-mfma", False, 1, 12, True))
        for kap in w.kappas:
            for arm, fixed, umin, lam, f8 in arms:
                c = build_case(w, kap, fixed, dev, quota_umin=umin, lam=lam, lay=lay)
                c["runner"].fp8_act = f8
                Rk = int((c["ids_np"] >= 0).sum())
                msk, st = time_steps(c, max(5, args.steps // 2), 2)
                uk = (f_fwd + (f_bwd if w.backward else 0)) * Rk
                sweep.append({"kappa": kap, "placement": arm,
                              "ms": round(msk, 4), "tflops": round(uk / (msk * 1e-3) / 1e12, 2),
                              "fwd_us": round(sum(v for k_, v in st.items() if k_.startswith("fwd.")) * 1e3, 1),
                              "bwd_us": round(sum(v for k_, v in st.items() if k_.startswith("bwd.")) * 1e3, 1)})
                if arm == "planned":
                    planners.append({"kappa": kap, **compare_planners(c, w)})
                del c
                torch.cuda.empty_cache()
            # quota planner with the partition count P picked by the cost model
            chosen = None
            for P in (1, 2, 4, 8):
                c = build_case(w, kap, False, dev, quota_umin=1, P=P, lay=lay)
                time_steps(c, 1, 0, with_events=False)          # route and plan once
                cost = predicted_cost(c, w, P)
                if chosen is None or (cost, -P) < (chosen[1], -chosen[2]):
                    chosen = (c, cost, P)
                else:
                    del c
                torch.cuda.empty_cache()
            c, _, P = chosen
            Rk = int((c["ids_np"] >= 0).sum())
            msk, st = time_steps(c, max(5, args.steps // 2), 2)
            uk = (f_fwd + (f_bwd if w.backward else 0)) * Rk
            sweep.append({"kappa": kap, "placement": f"planned-quota-sized (P={P})",
                          "ms": round(msk, 4), "tflops": round(uk / (msk * 1e-3) / 1e12, 2),
                          "fwd_us": round(sum(v for k_, v in st.items() if k_.startswith("fwd.")) * 1e3, 1),
                          "bwd_us": round(sum(v for k_, v in st.items() if k_.startswith("bwd.")) * 1e3, 1)})
            del c, chosen
            torch.cuda.empty_cache()
        out["kappa_sweep"] = sweep
        out["planners"] = planners
    if args.gate_sweep:
        gs = []
        for kap in (1.05, 1.1, 1.25, 1.5, 2.0):
            for arm, fixed, rho in (("fixed", True, None), ("planned", False, None),
                                    ("planned-gated", False, args.gate_rho)):
                c = build_case(w, kap, fixed, dev, gate_rho=rho, lay=lay)
                msk, _ = time_steps(c, max(5, args.steps // 2), 2)
                pf = c["runner"].plan_f["plan_info"].cpu().tolist()
                pb = c["runner"].plan_b["plan_info"].cpu().tolist() if w.backward else None
                gs.append({"kappa": kap, "placement": arm, "ms": round(msk, 4),
                           "plan_info_fwd": pf, "plan_info_bwd": pb})
                del c
                torch.cuda.empty_cache()
        out["gate_sweep"] = {"rho_milli": args.gate_rho, "runs": gs}
    if args.size_sweep:
        rows, regrets = [], []
        for kap in w.kappas:
            per = {}
            for P in (1, 2, 4, 8):
                c = build_case(w, kap, False, dev, P=P, lay=lay)
                msk, _ = time_steps(c, max(5, args.steps // 2), 2)
                per[P] = (msk, predicted_cost(c, w, P))
                del c
                torch.cuda.empty_cache()
            chosen = min(per, key=lambda p: (per[p][1], -p))
            best = min(per, key=lambda p: per[p][0])
            regret = per[chosen][0] / per[best][0] - 1
            regrets.append(regret)
            rows.append({"kappa": kap, "chosen_P": chosen, "best_P": best, "regret": round(regret, 4),
                         "per_P": {p: {"ms": round(v[0], 4), "predicted_steps": round(v[1] / 1000, 1)}
                                   for p, v in per.items()}})
        out["size_sweep"] = {"runs": rows, "mean_regret": round(sum(regrets) / len(regrets), 4)}
    if args.split_sweep:
        out["split_sweep"] = split_sweep(w, dev, lay, max(5, args.steps // 2))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(case, w, args.cpu_tokens, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
