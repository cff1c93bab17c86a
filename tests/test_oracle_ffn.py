"""Pins for the dense FFN oracle (oracle/ffn.py).

The forward follows the expert-computation equation of the MegaFlux summary
("Backward" section): Z = X W1, Z = [G, U], A = SiLU(G) * U, O = A W2,
y_t = sum_e p_te O_e[t].  Pinned by
* a closed form: permutation-shaped weights turn every matrix product into an
  index lookup, so a transposed operand or a swapped G/U half fails;
* SiLU special values (sigmoid(ln 3) = 3/4);
* brute force with scalar loops on a tiny case;
* invariants: linear in the gates, id < 0 contributes nothing, relabelling
  experts changes nothing.
The backward (gradient equations of the same section) is pinned by central
finite differences of L = sum_t dy_t . y_t in fp64.
"""
import math

import numpy as np
import pytest

from oracle import ffn
from oracle import ffn as offn
from oracle.fp8 import decode_e4m3


def _rand_case(rng, T=6, k=2, E=3, d=5, F=3, neg=False):
    x = rng.standard_normal((T, d))
    w1 = rng.standard_normal((E, 2 * F, d)) / math.sqrt(d)
    w2 = rng.standard_normal((E, d, F)) / math.sqrt(d)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    if neg:
        ids[0, 1] = -1
        ids[3, 0] = -1
    gates = rng.random((T, k))
    return x, w1, w2, ids, gates


def test_silu_special_values():
    assert ffn.silu(np.array(0.0)) == 0.0
    assert abs(ffn.silu(np.array(math.log(3.0))) - 0.75 * math.log(3.0)) < 1e-15
    assert abs(ffn.silu(np.array(-math.log(3.0))) + 0.25 * math.log(3.0)) < 1e-15


def test_permutation_weights_closed_form():
    rng = np.random.default_rng(0)
    n = 6                                   # d = d_ff = n
    E, T, k = 2, 5, 2
    x = rng.standard_normal((T, n))
    w1 = np.zeros((E, 2 * n, n))
    w2 = np.zeros((E, n, n))
    perms = {}
    for e in range(E):
        p1, p2, p3 = rng.permutation(n), rng.permutation(n), rng.permutation(n)
        g, u, w = rng.random(n) + 0.5, rng.random(n) + 0.5, rng.random(n) + 0.5
        for i in range(n):
            w1[e, i, p1[i]] = g[i]          # G_i = g_i * x[p1(i)]
            w1[e, n + i, p2[i]] = u[i]      # U_i = u_i * x[p2(i)]
            w2[e, i, p3[i]] = w[i]          # O_i = w_i * A[p3(i)]
        perms[e] = (p1, p2, p3, g, u, w)
    ids = np.array([[0, 1], [1, 0], [0, -1], [1, 1 - 1], [0, 1]])
    gates = rng.random((T, k))
    y = ffn.forward(x, w1, w2, ids, gates)
    for t in range(T):
        for i in range(n):
            want = 0.0
            for j in range(k):
                e = ids[t, j]
                if e < 0:
                    continue
                p1, p2, p3, g, u, w = perms[e]
                m = p3[i]
                G = g[m] * x[t, p1[m]]
                U = u[m] * x[t, p2[m]]
                want += gates[t, j] * w[i] * (G / (1.0 + math.exp(-G))) * U
            assert abs(y[t, i] - want) < 1e-12


def test_scalar_loop_brute_force():
    rng = np.random.default_rng(1)
    x, w1, w2, ids, gates = _rand_case(rng, neg=True)
    T, d = x.shape
    F = w1.shape[1] // 2
    y = ffn.forward(x, w1, w2, ids, gates)
    for t in range(T):
        want = [0.0] * d
        for j in range(ids.shape[1]):
            e = ids[t, j]
            if e < 0:
                continue
            a = []
            for f in range(F):
                gv = sum(w1[e, f, c] * x[t, c] for c in range(d))
                uv = sum(w1[e, F + f, c] * x[t, c] for c in range(d))
                a.append(gv / (1.0 + math.exp(-gv)) * uv)
            for i in range(d):
                want[i] += gates[t, j] * sum(w2[e, i, f] * a[f] for f in range(F))
        np.testing.assert_allclose(y[t], want, rtol=1e-12, atol=1e-14)


def test_invariants():
    rng = np.random.default_rng(2)
    x, w1, w2, ids, gates = _rand_case(rng, T=8, k=3, E=5)
    y = ffn.forward(x, w1, w2, ids, gates)
    np.testing.assert_allclose(ffn.forward(x, w1, w2, ids, 2.5 * gates), 2.5 * y, rtol=1e-13)
    assert np.abs(ffn.forward(x, w1, w2, ids, 0 * gates)).max() == 0.0
    ids2 = ids.copy()
    ids2[:, 2] = -1
    y2 = ffn.forward(x, w1, w2, ids2, gates)
    gates3 = gates.copy()
    gates3[:, 2] = 0
    np.testing.assert_allclose(y2, ffn.forward(x, w1, w2, ids, gates3), rtol=1e-13, atol=1e-15)
    relabel = rng.permutation(5)
    inv = np.argsort(relabel)
    y3 = ffn.forward(x, w1[inv], w2[inv], relabel[ids], gates)
    np.testing.assert_allclose(y3, y, rtol=1e-13)
    sub = np.array([5, 1, 6])
    np.testing.assert_allclose(ffn.forward(x, w1, w2, ids, gates, tokens=sub), y[sub], rtol=1e-13)


def test_backward_finite_differences():
    rng = np.random.default_rng(3)
    x, w1, w2, ids, gates = _rand_case(rng, T=5, k=2, E=3, d=4, F=3, neg=True)
    dy = rng.standard_normal(x.shape)
    g = ffn.backward(x, w1, w2, ids, gates, dy)

    def loss(x_, w1_, w2_):
        return float((ffn.forward(x_, w1_, w2_, ids, gates) * dy).sum())
    h = 1e-6
    for name, arr in (("x", x), ("w1", w1), ("w2", w2)):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            args_p = {"x": x, "w1": w1, "w2": w2}
            args_m = dict(args_p)
            args_p[name], args_m[name] = ap, am
            num[idx] = (loss(args_p["x"], args_p["w1"], args_p["w2"])
                        - loss(args_m["x"], args_m["w1"], args_m["w2"])) / (2 * h)
        if name == "x":
            got = g["dx"]
        elif name == "w1":
            got = np.stack([g["dw1"][e] for e in range(3)])
        else:
            got = np.stack([g["dw2"][e] for e in range(3)])
        np.testing.assert_allclose(got, num, rtol=1e-6, atol=1e-8, err_msg=name)


def test_backward_subsets_and_linearity():
    rng = np.random.default_rng(4)
    x, w1, w2, ids, gates = _rand_case(rng, T=9, k=2, E=4, d=5, F=2)
    dy = rng.standard_normal(x.shape)
    full = ffn.backward(x, w1, w2, ids, gates, dy)
    sub = ffn.backward(x, w1, w2, ids, gates, dy, tokens=np.array([2, 7]), experts=[1, 3])
    np.testing.assert_allclose(sub["dx"], full["dx"][[2, 7]], rtol=1e-13)
    for e in (1, 3):
        np.testing.assert_allclose(sub["dw1"][e], full["dw1"][e], rtol=1e-13)
        np.testing.assert_allclose(sub["dw2"][e], full["dw2"][e], rtol=1e-13)
    twice = ffn.backward(x, w1, w2, ids, gates, 2 * dy)
    np.testing.assert_allclose(twice["dx"], 2 * full["dx"], rtol=1e-13)
    zero = ffn.backward(x, w1, w2, ids, gates, 0 * dy)
    assert all(np.abs(v).max() == 0 for v in zero["dw2"].values())


# ---- fp8 backward with token-axis requantization ----------------------------

def _fp8_case(seed, T=96, k=2, E=3, d=16, F=8):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    w1 = rng.standard_normal((E, 2 * F, d)) / np.sqrt(d)
    w2 = rng.standard_normal((E, d, F)) / np.sqrt(F)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    g = rng.random((T, k)).astype(np.float32)
    dy = rng.standard_normal((T, d)).astype(np.float32).astype(np.float64)
    return x, w1, w2, ids, g, dy


def test_fp8_backward_dx_is_the_exact_one():
    x, w1, w2, ids, g, dy = _fp8_case(1)
    a = offn.backward(x, w1, w2, ids, g, dy)
    b = offn.backward_fp8(x, w1, w2, ids, g, dy, beta=16)
    np.testing.assert_array_equal(a["dx"], b["dx"])


def test_fp8_backward_dw_within_the_e4m3_bound():
    x, w1, w2, ids, g, dy = _fp8_case(2)
    a = offn.backward(x, w1, w2, ids, g, dy)
    b = offn.backward_fp8(x, w1, w2, ids, g, dy, beta=16)
    for key in ("dw1", "dw2"):
        A = np.stack([a[key][e] for e in range(3)])
        Bq = np.stack([b[key][e] for e in range(3)])
        err = np.linalg.norm(Bq - A) / np.linalg.norm(A)
        assert 1e-4 < err < 2.0 ** -4, (key, err)        # quantized, within half an e4m3 step


def test_fp8_backward_exact_when_D_is_representable():
    # gates 1 and dy drawn from e4m3 codes times 2^-3 with each block column's
    # largest magnitude 448 * 2^-3: every D value is code * scale exactly, so
    # dW2 equals the unquantized one
    rng = np.random.default_rng(5)
    T, k, E, d, F, beta = 64, 1, 2, 8, 4, 16
    x = rng.standard_normal((T, d))
    w1 = rng.standard_normal((E, 2 * F, d)) / 3
    w2 = rng.standard_normal((E, d, F)) / 3
    ids = (np.arange(T) % E)[:, None]
    g = np.ones((T, k), dtype=np.float32)
    grid = decode_e4m3(np.arange(0, 0x7F, dtype=np.uint8))
    dy = rng.choice(np.concatenate([grid, -grid]), size=(T, d)) * 2.0 ** -3
    for e in range(E):                 # every beta-row block of each expert gets a 448
        rows = np.nonzero(ids[:, 0] == e)[0]
        for b0 in range(0, len(rows), beta):
            dy[rows[b0], :] = 448 * 2.0 ** -3
    a = offn.backward(x, w1, w2, ids, g, dy)
    b = offn.backward_fp8(x, w1, w2, ids, g, dy, beta=beta)
    for e in range(E):
        np.testing.assert_allclose(b["dw2"][e], a["dw2"][e], rtol=1e-12, atol=1e-12)


# ---- the requantized operands, row by row -------------------------------------
# With x_t the unit vector e_t (d >= T), column t of dW1_e = dZq^T X is the
# requantized dZ row of token t in expert e; with A_t = a e_t (one-hot), column
# t of dW2_e = Dq^T A is a times the requantized D row.  The exact rows come
# from the unquantized backward (pinned above by finite differences and the
# closed forms).  What the pages fix (MegaFlux summary, "Backward": D_e and
# dZ_e requantized along the tokens; readings F1-F4: blocks of beta
# consecutive slots of one expert, counted from its first slot, times one
# column; scale = amax / 448) then gives three properties per block column,
# checked without re-running the quantizer:
#   * its largest magnitude survives (code 448 times the scale);
#   * every value is an e4m3 value times that scale (scale = largest / 448);
#   * every value is within half an e4m3 step of the exact one.

def _grid_units(r):
    """Distance of |r| (<= 448) from the nearest e4m3 value, in steps of the
    grid there: 3 mantissa bits above 2^-6, steps of 2^-9 below."""
    a = np.abs(np.asarray(r, dtype=np.float64))
    m, _ = np.frexp(a)                                  # a = m 2^e, 1/2 <= m < 1
    normal = np.abs(m * 16 - np.rint(m * 16))
    sub = np.abs(a / 2.0 ** -9 - np.rint(a / 2.0 ** -9))
    return np.where(a >= 2.0 ** -6, normal, sub)


def _tokens_of(ids, e):
    """Tokens of expert e's rows in slot order (flat (token, slot) order)."""
    flat = np.asarray(ids).ravel()
    return np.nonzero(flat == e)[0] // ids.shape[1]


def _check_token_blocks(q_rows, true_rows, beta):
    n = q_rows.shape[0]
    assert n > beta                                     # several blocks, the last one ragged
    for b0 in range(0, n, beta):
        q, v = q_rows[b0:b0 + beta], true_rows[b0:b0 + beta]
        vmax = np.abs(v).max(axis=0)
        zero = vmax == 0
        assert np.all(q[:, zero] == 0)
        q, v, vmax = q[:, ~zero], v[:, ~zero], vmax[~zero]
        m = np.abs(q).max(axis=0)
        assert np.all(np.abs(m - vmax) <= 2.0 ** -21 * vmax), "block column maximum not kept"
        s = m / 448.0
        assert np.all(_grid_units(q / s) <= 1e-6), "values off the block column's e4m3 grid"
        err = np.abs(q - v)
        assert np.all(err <= 2.0 ** -4 * np.abs(v) + 2.0 ** -10 * s + 2.0 ** -21 * np.abs(v)), \
            "a value moved by more than half an e4m3 step"


def _onehot_case(seed, T=48, k=2, E=3, d=64, F=8):
    rng = np.random.default_rng(seed)
    x = np.eye(T, d)                                    # x_t = e_t
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    g = rng.uniform(0.1, 1.0, (T, k)).astype(np.float32)   # gates != 1
    dy = rng.standard_normal((T, d)).astype(np.float32).astype(np.float64)
    return rng, x, ids, g, dy


def test_fp8_backward_dz_rows_are_token_axis_blocks():
    beta = 8
    rng, x, ids, g, dy = _onehot_case(11)
    E, d, F = 3, x.shape[1], 8
    w1 = rng.standard_normal((E, 2 * F, d))
    w2 = rng.standard_normal((E, d, F)) / np.sqrt(F)
    a = offn.backward(x, w1, w2, ids, g, dy)
    b = offn.backward_fp8(x, w1, w2, ids, g, dy, beta=beta)
    for e in range(E):
        t = _tokens_of(ids, e)
        _check_token_blocks(b["dw1"][e][:, t].T, a["dw1"][e][:, t].T, beta)


def test_fp8_backward_d_rows_are_token_axis_blocks_with_gates():
    # G = 1 everywhere and U_t = e_t, so A_t = SiLU(1) e_t
    beta = 8
    rng, x, ids, g, dy = _onehot_case(12)
    E, d, T = 3, x.shape[1], x.shape[0]
    F = T
    w1 = np.zeros((E, 2 * F, d))
    w1[:, :F, :] = 1.0
    w1[:, F + np.arange(T), np.arange(T)] = 1.0
    w2 = rng.standard_normal((E, d, F)) / np.sqrt(F)
    b = offn.backward_fp8(x, w1, w2, ids, g, dy, beta=beta)
    silu1 = 1.0 / (1.0 + np.exp(-1.0))
    for e in range(E):
        t = _tokens_of(ids, e)
        j = np.nonzero(ids[t] == e)[1]                  # slot of expert e in each token
        d_exact = g[t, j].astype(np.float64)[:, None] * dy[t]     # D = p dy
        _check_token_blocks(b["dw2"][e][:, t].T / silu1, d_exact, beta)


# ---- the fp8-operand forward (x and A quantized per row block of 128) ----------

def _fp8act_identity_case():
    """One token, one expert, d = d_ff = 128, where both quantizations are the
    identity: x = 448 at feature 0 (a block maximum exactly 448 * 2^0) and
    e4m3 values below it; G rows pick features so G = x[1..], U rows read
    x[0] scaled so that A = SiLU(G) U lands exactly on chosen e4m3 values with
    a block maximum of 448 * 2^-2."""
    from oracle.fp8 import decode_e4m3
    rng = np.random.default_rng(21)
    grid = decode_e4m3(np.arange(0x08, 0x76, dtype=np.uint8))       # normal codes below 448
    x = np.zeros((1, 128))
    x[0, 0] = 448.0
    x[0, 1:] = rng.choice(grid, 127) * rng.choice([-1, 1], 127)
    w1 = np.zeros((1, 256, 128))
    for jj in range(128):
        w1[0, jj, 1 + jj % 127] = 1.0                               # G_j = x[1 + j % 127]
    g = x[0, 1 + np.arange(128) % 127]
    a_want = rng.choice(grid, 128) * 0.25
    a_want[7] = 448.0 * 0.25                                        # the block maximum
    sil = offn.silu(g)
    for jj in range(128):
        w1[0, 128 + jj, 0] = a_want[jj] / sil[jj] / 448.0           # U_j = a_j / SiLU(G_j)
    w2 = rng.standard_normal((1, 128, 128))
    return x, w1, w2, np.zeros((1, 1), dtype=np.int64), np.ones((1, 1)), a_want


def test_forward_fp8act_is_forward_where_quantization_is_exact():
    x, w1, w2, ids, gates, a_want = _fp8act_identity_case()
    y8 = offn.forward_fp8act(x, w1, w2, ids, gates)
    y = offn.forward(x, w1, w2, ids, gates)
    np.testing.assert_allclose(y8, y, rtol=1e-12, atol=1e-9)
    np.testing.assert_allclose(y8[0], w2[0] @ a_want, rtol=1e-12, atol=1e-9)


def test_forward_fp8act_quantizes_a_per_block():
    """Moving one A value off the e4m3 grid changes y by the rounding of that
    value alone (its block's scale is unchanged), within half an e4m3 step;
    the exact forward moves by the full offset."""
    x, w1, w2, ids, gates, a_want = _fp8act_identity_case()
    j = 40
    v = a_want[j]
    w1b = w1.copy()
    off = abs(v) * 2.0 ** -6                                        # a sixteenth of v's own step
    w1b[0, 128 + j, 0] *= (v + off) / v
    y8 = offn.forward_fp8act(x, w1b, w2, ids, gates)
    y = offn.forward(x, w1b, w2, ids, gates)
    base = w2[0] @ a_want
    np.testing.assert_allclose(y8[0], base, rtol=1e-12, atol=1e-9)   # rounded back onto the grid
    np.testing.assert_allclose(y[0] - base, w2[0][:, j] * off, rtol=1e-6, atol=1e-9)


def test_forward_fp8act_error_bound():
    """On random data the fp8-operand forward stays within the e4m3
    quantization bound of the exact one (two roundings of at most 2^-4
    relative per value, plus one through SiLU)."""
    rng = np.random.default_rng(22)
    T, d, F, E, k = 40, 256, 128, 3, 2
    x = rng.standard_normal((T, d))
    w1 = rng.standard_normal((E, 2 * F, d)) / np.sqrt(d)
    w2 = rng.standard_normal((E, d, F)) / np.sqrt(F)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    gates = rng.random((T, k))
    y8 = offn.forward_fp8act(x, w1, w2, ids, gates)
    y = offn.forward(x, w1, w2, ids, gates)
    err = np.linalg.norm(y8 - y) / np.linalg.norm(y)
    assert 1e-3 < err < 3 * 2.0 ** -4


def test_round_bf16_matches_torch():
    import torch
    rng = np.random.default_rng(23)
    v = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-30, 30, 200000)).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(offn.round_bf16(v), ref)


# ---- the fp8-operand backward (dy and dZ quantized per row block of 128) -------

def _q_rows(v):
    from oracle.fp8 import dequant_row_blocks_pow2, quantize_row_blocks_pow2
    return dequant_row_blocks_pow2(*quantize_row_blocks_pow2(np.asarray(v, dtype=np.float32)))


def _check_row_blocks_pow2(q, v):
    """q holds v (bf16 values) quantized per row and block of 128 features with
    a power-of-two scale 2^e, e the smallest integer with amax <= 448 * 2^e:
    every value is an e4m3 value times 2^e, within half an e4m3 step of v."""
    rows, cols = v.shape
    for b0 in range(0, cols, 128):
        vb, qb = v[:, b0:b0 + 128], q[:, b0:b0 + 128]
        amax = np.abs(vb).max(axis=1)
        m, E = np.frexp(amax / 448.0)
        e = np.where(m == 0.5, E - 1, E)[:, None].astype(np.float64)
        s = np.power(2.0, e)
        assert np.all(amax[:, None] <= 448.0 * s) and np.all(amax[:, None] > 224.0 * s)
        assert np.all(_grid_units(qb / s) <= 1e-6), "values off the row block's e4m3 grid"
        assert np.all(np.abs(qb - vb) <= 2.0 ** -4 * np.abs(vb) + 2.0 ** -10 * s), \
            "a value moved by more than half an e4m3 step"


# Gates with at most four significant bits, off powers of two: p times an e4m3
# value is then exact in bf16.
_GATES4 = np.array([0.375, 0.625, 0.75, 0.875, 0.3125, 0.5625, 0.6875, 0.8125], dtype=np.float32)


def _fp8act_bwd_case(seed, T=24, k=1, E=2, F=128):
    """d = 2 F, W1 = I and W2 picking dy's first F features, so that
    G, U = the halves of Q(x), dA = p Q(dy)[:F] and dX = dZ; Z and dA are then
    exact in bf16 and the exact backward's dx is dZ itself."""
    rng = np.random.default_rng(seed)
    d = 2 * F
    x = rng.standard_normal((T, d))
    w1 = np.repeat(np.eye(d)[None], E, axis=0)
    w2 = np.repeat(np.eye(d, F)[None], E, axis=0)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    g = rng.choice(_GATES4, (T, k))
    dy = rng.standard_normal((T, d)).astype(np.float32).astype(np.float64)
    return x, w1, w2, ids, g, dy


def test_backward_fp8act_dx_is_the_dz_rows_quantized():
    """dX = Q(dZ) W1 with dZ (bf16) from dA = p Q(dy) W2 and Z = Q(x) W1: the
    exact backward on Q(x) and Q(dy) gives that dZ (W1 = I exposes it in dx;
    Z and dA are exact in bf16 here), and the fp8-operand dx must be it,
    rounded to bf16 and quantized per row block.  Quantizing D = p dy instead
    of dy, dA instead of dZ, blocks along the wrong axis, or no dZ
    quantization, each fail it."""
    x, w1, w2, ids, g, dy = _fp8act_bwd_case(31)
    dz = offn.backward(_q_rows(x), w1, w2, ids, g, _q_rows(dy))["dx"]
    got = offn.backward_fp8act(x, w1, w2, ids, g, dy, beta=8)["dx"]
    v = offn.round_bf16(dz.astype(np.float32)).astype(np.float64)
    _check_row_blocks_pow2(got, v)
    assert np.abs(got - v).max() > 0                   # something was rounded


def test_backward_fp8act_dw2_takes_z_of_the_quantized_x():
    """dW2 = Dq^T A with A from the fp8-operand forward's Z = Q(x) W1 (W1 = I:
    Z exact in bf16) and D from dy as given: it is backward_fp8's dW2 on
    Q(x), and not the one on x."""
    rng = np.random.default_rng(32)
    T, k, E, F = 40, 2, 3, 128
    d = 2 * F
    x = rng.standard_normal((T, d))
    w1 = np.repeat(np.eye(d)[None], E, axis=0)
    w2 = rng.standard_normal((E, d, F)) / np.sqrt(F)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    g = rng.uniform(0.2, 0.9, (T, k)).astype(np.float32)
    dy = rng.standard_normal((T, d)).astype(np.float32).astype(np.float64)
    b = offn.backward_fp8act(x, w1, w2, ids, g, dy, beta=16)
    ref = offn.backward_fp8(_q_rows(x), w1, w2, ids, g, dy, beta=16)
    plain = offn.backward_fp8(x, w1, w2, ids, g, dy, beta=16)
    for e in range(E):
        np.testing.assert_allclose(b["dw2"][e], ref["dw2"][e], rtol=1e-12, atol=1e-12)
        assert np.abs(b["dw2"][e] - plain["dw2"][e]).max() > 1e-6


def test_backward_fp8act_dw1_takes_dz_of_the_quantized_dy():
    """With x_t = e_t (on the e4m3 grid, so Q(x) = x) column t of dW1_e is the
    token-axis requantized dZ row of token t, whose dZ (bf16) comes from
    dA = p Q(dy) W2: each block of beta slots times one column keeps its
    maximum, lies on that column's e4m3 grid and stays within half a step of
    the exact backward's dZ on Q(dy), rounded to bf16 (W1 exact in bf16 and W2
    picking features keep Z and dA exact in bf16)."""
    beta = 8
    rng, x, ids, g, dy = _onehot_case(33)
    g = rng.choice(_GATES4, g.shape)
    E, d, F = 3, x.shape[1], 64                        # dZ rows: one block of 128
    pad = ((0, 0), (0, 128 - d))
    xp, dyp = np.pad(x, pad), np.pad(dy, pad)          # feature blocks of 128
    assert np.array_equal(_q_rows(xp), xp)
    w1 = offn.round_bf16(rng.standard_normal((E, 2 * F, 128)).astype(np.float32)).astype(np.float64)
    w2 = np.repeat(np.eye(128, F)[None], E, axis=0)
    a = offn.backward(xp, w1, w2, ids, g, _q_rows(dyp))
    b = offn.backward_fp8act(xp, w1, w2, ids, g, dyp, beta=beta)
    plain = offn.backward_fp8(xp, w1, w2, ids, g, dyp, beta=beta)
    for e in range(E):
        t = _tokens_of(ids, e)
        ref = offn.round_bf16(a["dw1"][e][:, t].T.astype(np.float32)).astype(np.float64)
        _check_token_blocks(b["dw1"][e][:, t].T, ref, beta)
        assert np.abs(b["dw1"][e] - plain["dw1"][e]).max() > 0


def test_backward_fp8act_error_bound():
    """dx and the weight gradients stay within the e4m3 bound of the exact
    backward (a few roundings of at most 2^-4 relative per value)."""
    rng = np.random.default_rng(34)
    T, k, E, d, F = 40, 2, 3, 256, 128
    x = rng.standard_normal((T, d))
    w1 = rng.standard_normal((E, 2 * F, d)) / np.sqrt(d)
    w2 = rng.standard_normal((E, d, F)) / np.sqrt(F)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    g = rng.uniform(0.2, 0.9, (T, k)).astype(np.float32)
    dy = rng.standard_normal((T, d)).astype(np.float32).astype(np.float64)
    a = offn.backward(x, w1, w2, ids, g, dy)
    b = offn.backward_fp8act(x, w1, w2, ids, g, dy, beta=16)
    err = np.linalg.norm(b["dx"] - a["dx"]) / np.linalg.norm(a["dx"])
    assert 1e-3 < err < 3 * 2.0 ** -4, err
    for key in ("dw1", "dw2"):
        A = np.stack([a[key][e] for e in range(E)])
        Bq = np.stack([b[key][e] for e in range(E)])
        err = np.linalg.norm(Bq - A) / np.linalg.norm(A)
        assert 1e-4 < err < 3 * 2.0 ** -4, (key, err)
