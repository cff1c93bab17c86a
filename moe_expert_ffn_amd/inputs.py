"""Seeded synthetic workloads for the skew-aware MoE expert layer.

This module only *draws inputs*: router top-k ids and gates, activations,
expert weights (optionally stored as e4m3 with 128x128 block scales) and the
upstream gradient.  It holds none of the layer's arithmetic: no counting into
blocks, no planning, no FFN.  Both the HIP path and the CPU oracle are fed
from here, and nothing here depends on either of them.

Shapes follow the workloads the MegaFlux summary (picx.dev/p/e4jAzZ,
"Problem Formulation", "Backward" equations) is stated for; the routing
distributions are synthetic stand-ins for the captured Qwen3/OLMoE routes the
pages measure on (those traces are not available).

Skew is controlled through the routing distribution.  To hit a requested skew
level the generator measures the realised skew with the plain definition
E * sum_e (c_e / sum c)^2 via ``numpy.bincount``; this only shapes inputs and
never produces an expected value.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make_routing", "make_layer", "make_dy",
           "seed_for", "realised_kappa"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    act: str          # activation / output dtype: "f32" or "bf16"
    wdt: str          # weight storage: "f32", "bf16" or "fp8"
    T: int            # tokens (source tokens for the one-GPU EP share)
    k: int            # router top-k
    E: int            # experts held by this GPU
    d: int            # model width
    d_ff: int         # expert hidden width (SwiGLU: W1 has 2*d_ff rows)
    beta: int         # block rows
    P: int            # workers (CU partitions)
    s: int            # replica budget per worker
    kappas: tuple     # skew levels the workload is run at
    backward: bool = False
    rows: int = 0     # fixed routed-row count (EP share); 0 = T*k
    cfg_id: int = 0   # seed namespace

    @property
    def routed_rows(self) -> int:
        return self.rows if self.rows else self.T * self.k


WORKLOADS = {
    # small correctness workload: fp32, Zipf(1.0) router bias
    "tiny_f32": Workload("tiny_f32", "f32", "f32", T=256, k=2, E=8, d=128, d_ff=64,
                         beta=16, P=4, s=1, kappas=(0,), cfg_id=1),
    # OLMoE-shaped forward
    "olmoe_bf16": Workload("olmoe_bf16", "bf16", "bf16", T=4096, k=8, E=64, d=2048,
                           d_ff=1024, beta=128, P=8, s=2, kappas=(1, 2, 4, 8), cfg_id=2),
    # Qwen3-30B-A3B-shaped forward
    "qwen3_bf16": Workload("qwen3_bf16", "bf16", "bf16", T=8192, k=8, E=128, d=2048,
                           d_ff=768, beta=128, P=8, s=4, kappas=(1, 2, 4, 8), cfg_id=3),
    # DeepSeek-V3 one-GPU EP share: 32 of 256 experts, e4m3 weights
    "dsv3_fp8": Workload("dsv3_fp8", "bf16", "fp8", T=0, k=8, E=32, d=7168, d_ff=2048,
                         beta=128, P=8, s=4, kappas=(1, 4, 8), rows=16384, cfg_id=4),
    # the same DeepSeek-V3 share, forward + backward (fp8 backward with token-axis requantization)
    "dsv3_fp8_fwdbwd": Workload("dsv3_fp8_fwdbwd", "bf16", "fp8", T=0, k=8, E=32, d=7168,
                                d_ff=2048, beta=128, P=8, s=4, kappas=(1, 4, 8), rows=16384,
                                backward=True, cfg_id=4),
    # Qwen3-shaped forward + backward
    "qwen3_bf16_fwdbwd": Workload("qwen3_bf16_fwdbwd", "bf16", "bf16", T=8192, k=8, E=128,
                                  d=2048, d_ff=768, beta=128, P=8, s=4, kappas=(1, 4, 8),
                                  backward=True, cfg_id=5),
}

STREAM_X, STREAM_W1, STREAM_W2, STREAM_LOGITS, STREAM_DY, STREAM_PERM = range(6)


def seed_for(w: Workload, kappa: float, stream: int, salt: int = 0) -> int:
    return 1000 * w.cfg_id + 10 * int(round(kappa)) + stream + 100000 * salt


def realised_kappa(ids: np.ndarray, E: int) -> float:
    c = np.bincount(ids[ids >= 0].reshape(-1), minlength=E).astype(np.float64)
    s = c.sum()
    return 1.0 if s == 0 else float(E * (c * c).sum() / (s * s))


def _softmax_rows(z: np.ndarray) -> np.ndarray:
    z = z - z.max(axis=1, keepdims=True)
    ez = np.exp(z)
    return ez / ez.sum(axis=1, keepdims=True)


def _topk_rows(logits: np.ndarray, k: int):
    """Top-k per row; ties go to the smaller expert id (stable sort on -logit)."""
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    chosen = np.take_along_axis(logits, order, axis=1)
    return order.astype(np.int32), chosen


def _route_from_logits(logits: np.ndarray, k: int):
    ids, chosen = _topk_rows(logits, k)
    gates = _softmax_rows(chosen).astype(np.float32)
    return ids, gates


def _uniform_exact(T, k, E, rng):
    """Every expert receives exactly T*k/E rows; ids distinct within a token."""
    perm = rng.permutation(E)
    flat = perm[np.arange(T * k) % E]
    ids = flat.reshape(T, k).astype(np.int32)
    gates = _softmax_rows(rng.standard_normal((T, k))).astype(np.float32)
    return ids, gates


def _hot_exact(T, k, E, rng):
    """k hot experts receive every token: the largest skew possible (E/k)."""
    hot = rng.choice(E, size=k, replace=False)
    ids = np.stack([rng.permutation(hot) for _ in range(T)]).astype(np.int32)
    gates = _softmax_rows(rng.standard_normal((T, k))).astype(np.float32)
    return ids, gates


def _zipf_popularity(E, a, rank_perm):
    ranks = np.empty(E, dtype=np.int64)
    ranks[rank_perm] = np.arange(E)
    return (ranks + 1.0) ** (-a)


def _tune(kappa_target, build, lo, hi, increasing=True, iters=40):
    """Bisect a scalar knob so that the realised skew of build(knob) is close to the
    target; returns the best (ids, gates, knob) seen."""
    best = None
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        ids, gates, kap = build(mid)
        err = abs(kap - kappa_target) / kappa_target
        if best is None or err < best[0]:
            best = (err, ids, gates, mid)
        if err < 0.005:
            break
        if (kap < kappa_target) == increasing:
            lo = mid
        else:
            hi = mid
    return best[1], best[2], best[3]


def make_routing(w: Workload, kappa: float, salt: int = 0):
    """Top-k expert ids int32 [T, k] (-1 = no local expert) and gates fp32 [T, k]."""
    rng = np.random.default_rng(seed_for(w, kappa, STREAM_LOGITS, salt))
    T, k, E = w.T, w.k, w.E
    if w.name == "tiny_f32" or kappa == 0:
        bias = -1.0 * np.log(np.arange(E) + 1.0)       # Zipf(1.0) per-expert bias
        logits = rng.standard_normal((T, E)) + bias[None, :]
        return _route_from_logits(logits, k)
    if w.wdt == "fp8":
        return _route_ep_share(w, kappa, rng)
    if kappa == 1:
        return _uniform_exact(T, k, E, rng)
    if abs(kappa - E / k) < 1e-9:
        return _hot_exact(T, k, E, rng)
    base = rng.standard_normal((T, E))
    if w.name.startswith("olmoe"):
        # Dirichlet(alpha) expert popularity; alpha tuned in log space
        gam_u = rng.random(E)

        def build(log_alpha):
            alpha = math.exp(log_alpha)
            g = np.random.default_rng(seed_for(w, kappa, STREAM_PERM, salt)).gamma(alpha, size=E)
            theta = np.maximum(g / g.sum(), 1e-30) * (1.0 + 1e-9 * gam_u)
            ids, gates = _route_from_logits(base + np.log(theta)[None, :], k)
            return ids, gates, realised_kappa(ids, E)
        ids, gates, _ = _tune(kappa, build, math.log(1e-3), math.log(1e3), increasing=False)
        return ids, gates
    rank_perm = rng.permutation(E)

    def build(a):
        pop = _zipf_popularity(E, a, rank_perm)
        ids, gates = _route_from_logits(base + np.log(pop)[None, :], k)
        return ids, gates, realised_kappa(ids, E)
    ids, gates, _ = _tune(kappa, build, 0.0, 8.0, increasing=True)
    return ids, gates


def _route_ep_share(w: Workload, kappa, rng):
    """One GPU's share of a top-8-of-256 layer holding 32 experts: each source token
    has m ~ Binomial(8, 32/256) | m >= 1 local slots; rows stop at exactly w.rows."""
    k, E, R = w.k, w.E, w.rows
    m_list = []
    total = 0
    while total < R:
        m = 0
        while m == 0:
            m = int(rng.binomial(k, E / 256.0))
        m = min(m, R - total)
        m_list.append(m)
        total += m
    T = len(m_list)
    ids = np.full((T, k), -1, dtype=np.int32)
    slot_pos = [rng.permutation(k)[:m] for m in m_list]
    gates = _softmax_rows(rng.standard_normal((T, k))).astype(np.float32)
    if kappa == 1:
        perm = rng.permutation(E)
        n = 0
        for t, m in enumerate(m_list):
            for jj in range(m):
                ids[t, slot_pos[t][jj]] = perm[n % E]
                n += 1
        return ids, gates
    rank_perm = rng.permutation(E)
    # m distinct experts per token by Gumbel-top-m over log popularity, with a fixed
    # noise table so the draw varies smoothly with the Zipf exponent
    noise = -np.log(-np.log(np.clip(np.random.default_rng(rng.integers(1 << 62)).random((T, E)),
                                    1e-300, 1 - 1e-16)))

    def build(a):
        pop = _zipf_popularity(E, a, rank_perm)
        score = np.log(pop)[None, :] + noise
        order = np.argsort(-score, axis=1, kind="stable")
        out = np.full((T, k), -1, dtype=np.int32)
        for t, m in enumerate(m_list):
            out[t, slot_pos[t]] = order[t, :m]
        return out, gates, realised_kappa(out, E)
    ids, gates, _ = _tune(kappa, build, 0.0, 8.0, increasing=True)
    return ids, gates


def _bf16_round(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.bfloat16)


def _quant_e4m3_blocks(wf: torch.Tensor):
    """e4m3fn codes (uint8) with one fp32 scale per 128x128 block: scale = amax/448,
    code = RNE(w/scale) saturated to +-448.  A storage format of the inputs."""
    E, N, K = wf.shape
    wb = wf.reshape(E, N // 128, 128, K // 128, 128)
    amax = wb.abs().amax(dim=(2, 4)).clamp_min(1e-30)
    scale = (amax / 448.0).to(torch.float32)
    qv = (wb / scale[:, :, None, :, None]).clamp(-448.0, 448.0)
    codes = qv.reshape(E, N, K).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.contiguous()


def make_layer(w: Workload, device="cpu", salt: int = 0):
    """x [T, d] and expert weights.  W1 [E, 2*d_ff, d] (rows 0..d_ff-1 = gate G,
    d_ff..2d_ff-1 = up U), W2 [E, d, d_ff]; both ~ N(0, 1/d) (literal reading of the
    tiny workload's W ~ N(0, 1/d), reused for every workload).

    Returns a dict of torch tensors on `device`.  For fp8 workloads, w1/w2 are uint8
    e4m3fn codes and w1_scale/w2_scale fp32 [E, N/128, K/128]."""
    dev = torch.device(device)
    act = torch.float32 if w.act == "f32" else torch.bfloat16

    def gen(stream):
        g = torch.Generator(device=dev)
        g.manual_seed(seed_for(w, 0, stream, salt))
        return g
    T = w.T if w.T else None
    out = {}
    if T is not None:
        out["x"] = torch.randn((T, w.d), generator=gen(STREAM_X), device=dev).to(act)
    std = 1.0 / math.sqrt(w.d)
    w1 = torch.randn((w.E, 2 * w.d_ff, w.d), generator=gen(STREAM_W1), device=dev) * std
    w2 = torch.randn((w.E, w.d, w.d_ff), generator=gen(STREAM_W2), device=dev) * std
    if w.wdt == "fp8":
        out["w1"], out["w1_scale"] = _quant_e4m3_blocks(w1)
        out["w2"], out["w2_scale"] = _quant_e4m3_blocks(w2)
    else:
        wdt = torch.float32 if w.wdt == "f32" else torch.bfloat16
        out["w1"], out["w2"] = w1.to(wdt).contiguous(), w2.to(wdt).contiguous()
    return out


def make_x(w: Workload, T: int, device="cpu", salt: int = 0):
    """Activations for a workload whose token count is only known after routing."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed_for(w, 0, STREAM_X, salt))
    act = torch.float32 if w.act == "f32" else torch.bfloat16
    return torch.randn((T, w.d), generator=g, device=dev).to(act)


def make_dy(w: Workload, T: int, device="cpu", salt: int = 0):
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed_for(w, 0, STREAM_DY, salt))
    act = torch.float32 if w.act == "f32" else torch.bfloat16
    return torch.randn((T, w.d), generator=g, device=dev).to(act)


def contiguous_owners(E: int, P: int) -> np.ndarray:
    """h(e) = floor(e*P/E): contiguous expert-parallel ownership."""
    return (np.arange(E) * P // E).astype(np.int32)
