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
