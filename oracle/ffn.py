"""Oracle: dense per-token SwiGLU expert FFN and its gradients, fp64 --
TEST INFRASTRUCTURE ONLY.

MegaFlux summary (picx.dev/p/e4jAzZ), "Backward" section:
* expert computation: Z_e = X_e W_1,e ; Z_e = [G_e, U_e] ;
  A_e = SiLU(G_e) * U_e ; O_e = A_e W_2,e ; y_t = sum_{e in S_t} p_te O_e[t];
* gradients: dA_e = D_e W_2,e^T ; dX_e = dZ_e W_1,e^T ; dW_2,e = A_e^T D_e ;
  dW_1,e = X_e^T dZ_e.

Storage convention (matches the library): w1 is [E, 2*d_ff, d] with rows
0..d_ff-1 producing G and rows d_ff..2*d_ff-1 producing U, i.e. it holds
W_1,e transposed; w2 is [E, d, d_ff], i.e. W_2,e transposed.  So for one row
x (length d): z = w1[e] @ x, o = w2[e] @ a.

Readings (the pages are silent): D_e = dL/dO_e, which through
y_t = sum p O carries the gate, D[t] = p_te * dy_t; SiLU(g) = g * sigmoid(g);
expert slots with id < 0 contribute nothing.  There are no blocks and no
plan here: every routed (token, slot) pair is computed on its own and the k
contributions of a token are added in slot order.
"""
from __future__ import annotations

import numpy as np


def sigmoid(g):
    return 1.0 / (1.0 + np.exp(-g))


def silu(g):
    return g * sigmoid(g)


def _pairs_by_expert(ids, tokens):
    """{e: (positions into `tokens`, slot j)} for every routed pair."""
    sub = ids[tokens]
    out = {}
    for e in np.unique(sub[sub >= 0]):
        ti, j = np.nonzero(sub == e)
        out[int(e)] = (ti, j)
    return out


def forward(x, w1, w2, topk_ids, gates, tokens=None, return_z=False):
    """y [n, d] for the given token subset (default: all tokens), fp64."""
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(topk_ids)
    p = np.asarray(gates, dtype=np.float64)
    T, k = ids.shape
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    F = w1.shape[1] // 2
    contrib = np.zeros((len(tokens), k, x.shape[1]))
    zs = {}
    for e, (ti, j) in _pairs_by_expert(ids, tokens).items():
        xe = x[tokens[ti]]
        w1e = np.asarray(w1[e], dtype=np.float64)
        w2e = np.asarray(w2[e], dtype=np.float64)
        z = xe @ w1e.T
        a = silu(z[:, :F]) * z[:, F:]
        o = a @ w2e.T
        contrib[ti, j] = p[tokens[ti], j][:, None] * o
        if return_z:
            zs[e] = (tokens[ti], j, z)
    y = np.zeros((len(tokens), x.shape[1]))
    for j in range(k):
        y += contrib[:, j]
    return (y, zs) if return_z else y


def round_bf16(v) -> np.ndarray:
    """fp32 values rounded to bfloat16 (8 significant bits, nearest, ties to
    even), returned as fp32; finite inputs only."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def forward_fp8act(x, w1, w2, topk_ids, gates, tokens=None, return_z=False):
    """The forward of an e4m3-weight layer whose two products run on fp8
    operands (reading of "per-1x128 e4m3 activations"): each row of x and each
    row of A = SiLU(G) U is quantized in blocks of 128 features with
    power-of-two scales (oracle.fp8.quantize_row_blocks_pow2) before the
    product that reads it; the weights are as given (dequantized).  A is
    formed from Z and stored in the activation dtype, bf16 (round to nearest
    even from its fp32 value), before its quantization, as the layer keeps
    A between the two products.  The gated combine is forward's."""
    from oracle.fp8 import dequant_row_blocks_pow2, quantize_row_blocks_pow2
    x = np.asarray(x, dtype=np.float64)
    xh = dequant_row_blocks_pow2(*quantize_row_blocks_pow2(x.astype(np.float32)))
    ids = np.asarray(topk_ids)
    p = np.asarray(gates, dtype=np.float64)
    T, k = ids.shape
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    F = w1.shape[1] // 2
    contrib = np.zeros((len(tokens), k, x.shape[1]))
    zs = {}
    for e, (ti, j) in _pairs_by_expert(ids, tokens).items():
        z = xh[tokens[ti]] @ np.asarray(w1[e], dtype=np.float64).T
        a = round_bf16((silu(z[:, :F]) * z[:, F:]).astype(np.float32))
        ah = dequant_row_blocks_pow2(*quantize_row_blocks_pow2(a))
        o = ah @ np.asarray(w2[e], dtype=np.float64).T
        contrib[ti, j] = p[tokens[ti], j][:, None] * o
        if return_z:
            zs[e] = (tokens[ti], j, z)
    y = np.zeros((len(tokens), x.shape[1]))
    for j in range(k):
        y += contrib[:, j]
    return (y, zs) if return_z else y


def backward(x, w1, w2, topk_ids, gates, dy, tokens=None, experts=None):
    """Gradients of L = sum_t dy_t . y_t.

    Returns dict with dx [n, d] for the token subset `tokens` (default all) and,
    for each expert in `experts` (default all), dw1 [2*d_ff, d] and dw2 [d, d_ff]
    in the library's storage layout (gradient of w1/w2 as stored).  dW of an
    expert sums over *all* of its routed rows, whatever `tokens` is.
    """
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    ids = np.asarray(topk_ids)
    p = np.asarray(gates, dtype=np.float64)
    T, k = ids.shape
    d = x.shape[1]
    E = w1.shape[0]
    F = w1.shape[1] // 2
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    experts = range(E) if experts is None else experts
    tok_pos = {int(t): i for i, t in enumerate(tokens)}
    all_pairs = _pairs_by_expert(ids, np.arange(T))

    dx_contrib = np.zeros((len(tokens), k, d))
    dw1, dw2 = {}, {}
    want_w = set(int(e) for e in experts)
    for e in range(E):
        need_rows = e in want_w
        ti, j = all_pairs.get(e, (np.zeros(0, int), np.zeros(0, int)))
        if not need_rows:
            keep = np.array([t in tok_pos for t in ti], dtype=bool)
            ti, j = ti[keep], j[keep]
        w1e = np.asarray(w1[e], dtype=np.float64)
        w2e = np.asarray(w2[e], dtype=np.float64)
        xe = x[ti]
        D = p[ti, j][:, None] * dy[ti]                 # dL/dO_e
        z = xe @ w1e.T
        g, u = z[:, :F], z[:, F:]
        sg = sigmoid(g)
        a = g * sg * u
        dA = D @ w2e                                  # D_e W_2,e^T in math layout
        dG = dA * u * sg * (1.0 + g * (1.0 - sg))
        dU = dA * g * sg
        dZ = np.concatenate([dG, dU], axis=1)
        dX = dZ @ w1e                                 # dZ_e W_1,e^T
        for r in range(len(ti)):
            pos = tok_pos.get(int(ti[r]))
            if pos is not None:
                dx_contrib[pos, j[r]] = dX[r]
        if need_rows:
            dw2[e] = D.T @ a                          # [d, d_ff] = (A^T D)^T
            dw1[e] = dZ.T @ xe                        # [2 d_ff, d] = (X^T dZ)^T
    dx = np.zeros((len(tokens), d))
    for jj in range(k):
        dx += dx_contrib[:, jj]
    return {"dx": dx, "dw1": dw1, "dw2": dw2}


def backward_fp8(x, w1, w2, topk_ids, gates, dy, beta, tokens=None, experts=None):
    """The backward of an fp8-weight layer with token-axis requantization
    (MegaFlux summary, "Backward": overlapped requantization of D_e and dZ_e).

    Reading: dA, dZ and dx use the exact D = p * dy and the dequantized
    weights (w1, w2 as given, already dequantized); the weight gradients take
    D and dZ requantized to e4m3 in blocks of beta consecutive slots of the
    expert (its rows in flat (token, slot) order, which is the slot order)
    times one column (oracle.fp8.quantize_token_blocks), with x and
    A = SiLU(G) U unquantized:  dW2 = Dq^T A,  dW1 = dZq^T X.  D is formed in
    fp32 as p * dy (the value the device quantizes); dZ enters the
    quantizer as fp32.
    """
    from oracle.fp8 import dequant_token_blocks, quantize_token_blocks
    out = backward(x, w1, w2, topk_ids, gates, dy, tokens=tokens, experts=experts)
    x = np.asarray(x, dtype=np.float64)
    dy32 = np.asarray(dy, dtype=np.float32)
    ids = np.asarray(topk_ids)
    p32 = np.asarray(gates, dtype=np.float32)
    T, k = ids.shape
    E = w1.shape[0]
    F = w1.shape[1] // 2
    experts = range(E) if experts is None else experts
    all_pairs = _pairs_by_expert(ids, np.arange(T))
    for e in experts:
        e = int(e)
        ti, j = all_pairs.get(e, (np.zeros(0, int), np.zeros(0, int)))
        w1e = np.asarray(w1[e], dtype=np.float64)
        w2e = np.asarray(w2[e], dtype=np.float64)
        if len(ti) == 0:
            out["dw1"][e] = np.zeros((2 * F, x.shape[1]))
            out["dw2"][e] = np.zeros((w2e.shape[0], F))
            continue
        xe = x[ti]
        D32 = (p32[ti, j][:, None] * dy32[ti]).astype(np.float32)
        D = D32.astype(np.float64)
        z = xe @ w1e.T
        g, u = z[:, :F], z[:, F:]
        sg = sigmoid(g)
        a = g * sg * u
        dA = D @ w2e
        dZ = np.concatenate([dA * u * sg * (1.0 + g * (1.0 - sg)), dA * g * sg], axis=1)
        Dq = dequant_token_blocks(*quantize_token_blocks(D32, beta), beta)
        dZq = dequant_token_blocks(*quantize_token_blocks(dZ.astype(np.float32), beta), beta)
        out["dw2"][e] = Dq.T @ a
        out["dw1"][e] = dZq.T @ xe
    return out


def backward_fp8act(x, w1, w2, topk_ids, gates, dy, beta, tokens=None, experts=None):
    """The backward of an e4m3-weight layer whose products run on fp8 operands
    in both directions (the reading of "per-1x128 e4m3 activations" that
    forward_fp8act follows, carried to dA and dX):

    * [G, U] are what the fp8-operand forward saves: Z = Q(x) W1 stored in
      bf16 (Q: each row in blocks of 128 features with power-of-two scales,
      oracle.fp8.quantize_row_blocks_pow2);
    * dA = p * (Q(dy_t) W2): the token's dy row is quantized, once for all of
      its k slots, the gate is applied to the product, and dA is stored in
      bf16 before the SwiGLU gradient;
    * dZ = [dG, dU] from dA, G and U as in backward, stored in bf16; the row's
      dX contribution is Q(dZ) W1, and dx adds a token's k contributions in
      slot order;
    * the weight gradients are backward_fp8's: dW2 = Dq^T A with D = p * dy
      (dy as given) and A from the saved Z, dW1 = dZq^T X with this dZ and X
      as given; Dq and dZq are the token-axis requantizations.
    The e4m3 codes of dZ (both quantizations) are integers decided by floating
    point, so they are decided on the values the layer stores (bf16 Z, dA and
    dZ), as the layer decides them.
    """
    from oracle.fp8 import (dequant_row_blocks_pow2, dequant_token_blocks,
                            quantize_row_blocks_pow2, quantize_token_blocks)

    def q_rows(v):
        return dequant_row_blocks_pow2(*quantize_row_blocks_pow2(np.asarray(v, dtype=np.float32)))

    def bf16(v):
        return round_bf16(np.asarray(v, dtype=np.float32)).astype(np.float64)

    x = np.asarray(x, dtype=np.float64)
    xh = q_rows(x)
    dy32 = np.asarray(dy, dtype=np.float32)
    dyh = q_rows(dy32)
    ids = np.asarray(topk_ids)
    p32 = np.asarray(gates, dtype=np.float32)
    p = p32.astype(np.float64)
    T, k = ids.shape
    d = x.shape[1]
    E = w1.shape[0]
    F = w1.shape[1] // 2
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    experts = range(E) if experts is None else experts
    tok_pos = {int(t): i for i, t in enumerate(tokens)}
    all_pairs = _pairs_by_expert(ids, np.arange(T))

    dx_contrib = np.zeros((len(tokens), k, d))
    dw1, dw2 = {}, {}
    want_w = set(int(e) for e in experts)
    for e in range(E):
        need_rows = e in want_w
        ti, j = all_pairs.get(e, (np.zeros(0, int), np.zeros(0, int)))
        if not need_rows:
            keep = np.array([t in tok_pos for t in ti], dtype=bool)
            ti, j = ti[keep], j[keep]
        w1e = np.asarray(w1[e], dtype=np.float64)
        w2e = np.asarray(w2[e], dtype=np.float64)
        if len(ti) == 0:
            if need_rows:
                dw1[e] = np.zeros((2 * F, d))
                dw2[e] = np.zeros((d, F))
            continue
        z = bf16(xh[ti] @ w1e.T)
        g, u = z[:, :F], z[:, F:]
        sg = sigmoid(g)
        a = g * sg * u
        dA = bf16(p[ti, j][:, None] * (dyh[ti] @ w2e))
        dZ = bf16(np.concatenate([dA * u * sg * (1.0 + g * (1.0 - sg)), dA * g * sg], axis=1))
        dX = q_rows(dZ) @ w1e
        for r in range(len(ti)):
            pos = tok_pos.get(int(ti[r]))
            if pos is not None:
                dx_contrib[pos, j[r]] = dX[r]
        if need_rows:
            D32 = (p32[ti, j][:, None] * dy32[ti]).astype(np.float32)
            Dq = dequant_token_blocks(*quantize_token_blocks(D32, beta), beta)
            dZq = dequant_token_blocks(*quantize_token_blocks(dZ.astype(np.float32), beta), beta)
            dw2[e] = Dq.T @ a
            dw1[e] = dZq.T @ x[ti]
    dx = np.zeros((len(tokens), d))
    for jj in range(k):
        dx += dx_contrib[:, jj]
    return {"dx": dx, "dw1": dw1, "dw2": dw2}
