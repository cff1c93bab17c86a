"""Chains the library's calls for one expert layer over preallocated buffers:
route statistics -> plan -> forward (-> backward plan -> backward).

Buffers come from torch (device memory); every computation is a library call.
"""
from __future__ import annotations

import torch

from . import binding as B


class LayerRunner:
    def __init__(self, w1, w2, w1_scale=None, w2_scale=None, *, act_dtype, T, k, beta, P, s,
                 owner, lam=12, with_backward=False, save_z=None, quota_umin=None,
                 gate_rho=None, two_phase=False):
        dev = w1.device
        self.dev = dev
        self.layer = B.make_layer(w1, w2, w1_scale, w2_scale, act_dtype)
        self.keep = (w1, w2, w1_scale, w2_scale)
        self.E, self.d, self.dff = self.layer.E, self.layer.d, self.layer.d_ff
        self.T, self.k, self.beta, self.P, self.s, self.lam = T, k, beta, P, s, lam
        # quota_umin set: every plan (forward and backward) comes from the
        # quota-driven solver with that quota floor
        self.quota_umin = quota_umin
        # gate_rho set: every plan passes the replication gate with that price
        # per replica (thousandths of a block)
        self.gate_rho = gate_rho
        self.act_dtype = act_dtype
        # two_phase: FC1 / FC2 (dA / dX) in one two-phase launch instead of two
        self.two_phase = two_phase
        # producer workgroups per worker of the forward / backward two-phase
        # launch (0: every workgroup runs both phases)
        self.split_fwd = 0
        self.split_bwd = 0
        # e4m3 weights: every product but the weight gradients on the fp8 MFMA
        # (x, A, dy and dZ quantized per row block of 128 features)
        self.fp8_act = False
        self.owner = owner.to(device=dev, dtype=torch.int32).contiguous()
        self.with_backward = with_backward
        self.ws = B.workspace(self.layer, T, k, beta, P, s, with_backward, dev)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.rs = B.alloc_route(T, k, self.E, beta, dev)
        nbc = B.max_blocks(T, k, self.E, beta)
        self.plan_f = B.alloc_plan(self.E, P, nbc, dev)
        self.plan_b = B.alloc_plan(self.E, P, nbc, dev) if with_backward else None
        # the backward plan needs only the routing statistics: it runs on this
        # stream (default priority) while the forward plan and the forward run
        self.side = torch.cuda.Stream(device=dev) if with_backward and dev.type == "cuda" else None
        self.y = torch.empty((T, self.d), dtype=act_dtype, device=dev)
        need_z = with_backward if save_z is None else save_z
        ms = max(B.max_slots(T, k, self.E, beta), 1)
        self.z = torch.empty((ms, 2 * self.dff), dtype=act_dtype, device=dev) if need_z else None
        if with_backward:
            self.dx = torch.empty((T, self.d), dtype=act_dtype, device=dev)
            self.dw1 = torch.empty((self.E, 2 * self.dff, self.d), dtype=torch.float32, device=dev)
            self.dw2 = torch.empty((self.E, self.d, self.dff), dtype=torch.float32, device=dev)

    def route(self, topk_ids):
        return B.route_stats(topk_ids, self.E, self.beta, self.rs, self.ws, self.status)

    def make_plan(self, mode=B.PLAN_FWD, s=None, out=None):
        if s is not None and s > self.s:
            raise B.MoeError(f"replica budget s={s} above the runner's s={self.s}")
        out = self.plan_f if out is None else out
        lam = self.lam
        if self.quota_umin is not None:
            mode, lam = B.PLAN_QUOTA, self.quota_umin
        B.plan(self.rs["block_counts"], self.rs["block_offsets"], self.owner, self.P,
               self.s if s is None else s, mode, lam, out, self.ws, self.status)
        if self.gate_rho is not None:
            B.plan_gate(self.rs["block_counts"], self.rs["block_offsets"], self.owner, self.P,
                        self.gate_rho, out, self.status)
        return out

    def forward(self, x, gates, topk_ids, block_worker=None, events=None, timeline=None):
        bw = self.plan_f["block_worker"] if block_worker is None else block_worker
        B.forward(self.layer, x, gates, topk_ids, self.beta, self.P, self.rs, bw, self.y, self.z,
                  self.ws, self.status, events, timeline, self.two_phase, self.split_fwd,
                  self.fp8_act)
        return self.y

    def backward(self, x, gates, dy, topk_ids, block_worker=None, events=None, timeline=None):
        bw = self.plan_b["block_worker"] if block_worker is None else block_worker
        B.backward(self.layer, x, gates, dy, self.z, topk_ids, self.beta, self.P, self.s, self.rs,
                   self.owner, bw, self.dx, self.dw1, self.dw2, self.ws, self.status, events,
                   timeline, self.two_phase, self.split_bwd, self.fp8_act)
        return self.dx, self.dw1, self.dw2

    def step(self, x, gates, topk_ids, dy=None, s=None, timeline=None):
        """One pass of the whole path: route -> plan -> forward [-> plan(bwd) -> backward].

        s (default: the runner's s) is the replica budget of both plans; it may
        not exceed the runner's, whose replica slots the backward provides."""
        if s is not None and s > self.s:
            raise B.MoeError(f"replica budget s={s} above the runner's s={self.s}")
        self.route(topk_ids)
        if dy is not None:
            self.plan_bwd_async(s)
        self.make_plan(B.PLAN_FWD, s)
        self.forward(x, gates, topk_ids, timeline=timeline)
        if dy is not None:
            self.join_bwd_plan()
            self.backward(x, gates, dy, topk_ids, timeline=timeline)
        return self.y

    def plan_bwd_async(self, s=None, events=None):
        """The backward plan on the side stream, after the work already queued
        on the current stream (the routing statistics); `events` (optional,
        a B.Events of 2) brackets it there."""
        main = torch.cuda.current_stream(self.dev)
        self.side.wait_stream(main)
        with torch.cuda.stream(self.side):
            if events is not None:
                events.record(0)
            self.make_plan(B.PLAN_BWD, s, self.plan_b)
            if events is not None:
                events.record(1)

    def join_bwd_plan(self):
        """The current stream waits for the backward plan."""
        torch.cuda.current_stream(self.dev).wait_stream(self.side)
