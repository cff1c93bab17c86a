"""Helpers shared by the GPU parity tests: build a workload on the device, run
the library through the C ABI, and hand the same inputs to the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

from moe_expert_ffn_amd import binding as B
from moe_expert_ffn_amd.inputs import (Workload, contiguous_owners, make_dy, make_layer,
                                       make_routing, make_x)
from moe_expert_ffn_amd.runner import LayerRunner
from oracle.fp8 import dequant_blocks


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class LazyWeights:
    """Expert weights as fp64 numpy, converted one expert at a time."""

    def __init__(self, w, scale=None):
        self.w, self.scale = w, scale
        self.shape = tuple(w.shape)

    def __getitem__(self, e):
        e = int(e)
        if self.scale is not None:
            return dequant_blocks(self.w[e].cpu().numpy(), self.scale[e].cpu().numpy())
        return self.w[e].double().cpu().numpy()


class Case:
    def __init__(self, w: Workload, kappa, device="cuda", P=None, s=None, backward=False, salt=0,
                 ids=None, gates=None, lam=12):
        self.w = w
        self.P = w.P if P is None else P
        self.s = w.s if s is None else s
        if ids is None:
            ids, gates = make_routing(w, kappa, salt)
        self.ids_np, self.gates_np = ids, gates
        T = ids.shape[0]
        self.T = T
        lay = make_layer(w, device, salt)
        self.x = lay["x"] if "x" in lay and lay["x"].shape[0] == T else make_x(w, T, device, salt)
        self.w1, self.w2 = lay["w1"], lay["w2"]
        self.w1s, self.w2s = lay.get("w1_scale"), lay.get("w2_scale")
        self.ids = torch.from_numpy(ids).to(device)
        self.gates = torch.from_numpy(gates).to(device)
        self.owner_np = contiguous_owners(w.E, self.P)
        self.act = torch.float32 if w.act == "f32" else torch.bfloat16
        self.dy = make_dy(w, T, device, salt) if backward else None
        self.runner = LayerRunner(self.w1, self.w2, self.w1s, self.w2s, act_dtype=self.act, T=T,
                                  k=w.k, beta=w.beta, P=self.P, s=self.s,
                                  owner=torch.from_numpy(self.owner_np), with_backward=backward,
                                  lam=lam)

    def oracle_inputs(self):
        return (self.x.double().cpu().numpy(), LazyWeights(self.w1, self.w1s),
                LazyWeights(self.w2, self.w2s), self.ids_np, self.gates_np.astype(np.float64))

    def status(self):
        return int(self.runner.status.item())
