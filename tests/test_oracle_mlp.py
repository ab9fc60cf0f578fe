"""Pins of the oracle's shared dense MLP.

Checked against a scalar-loop evaluation written out element by element
(non-square shapes, so a transposed operand fails), closed forms (a zero
gate or up projection gives zero; one hidden unit by hand) and exact
invariants (linearity in W_d, token permutation).
"""

import math

import numpy as np

from oracle import omni_oracle as O


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def loops(x, Wg, Wu, Wd):
    L, d = x.shape
    F = Wg.shape[0]
    out = np.zeros((L, Wd.shape[0]))
    for t in range(L):
        a = []
        for j in range(F):
            g = sum(x[t, c] * Wg[j, c] for c in range(d))
            u = sum(x[t, c] * Wu[j, c] for c in range(d))
            a.append(g / (1.0 + math.exp(-g)) * u)
        for i in range(Wd.shape[0]):
            out[t, i] = sum(a[j] * Wd[i, j] for j in range(F))
    return out


def test_matches_scalar_loops():
    r = rng(1)
    L, d, F = 3, 5, 7
    x, Wg, Wu, Wd = r.normal(size=(L, d)), r.normal(size=(F, d)), r.normal(size=(F, d)), r.normal(size=(d, F))
    np.testing.assert_allclose(O.shared_mlp(x, Wg, Wu, Wd), loops(x, Wg, Wu, Wd), rtol=1e-12, atol=1e-12)


def test_closed_forms():
    r = rng(2)
    L, d, F = 4, 6, 8
    x, Wg, Wu, Wd = r.normal(size=(L, d)), r.normal(size=(F, d)), r.normal(size=(F, d)), r.normal(size=(d, F))
    assert np.all(O.shared_mlp(x, np.zeros_like(Wg), Wu, Wd) == 0.0)  # SiLU(0) = 0
    assert np.all(O.shared_mlp(x, Wg, np.zeros_like(Wu), Wd) == 0.0)
    # one token, one hidden unit: x = (1, 2), w_g = (log 3, 0) so g = log 3 and
    # SiLU(g) = (3/4) log 3; w_u = (0, 1) so u = 2; W_d = (1, -1)^T
    x1 = np.array([[1.0, 2.0]])
    out = O.shared_mlp(x1, np.array([[math.log(3), 0.0]]), np.array([[0.0, 1.0]]),
                       np.array([[1.0], [-1.0]]))
    a = 0.75 * math.log(3) * 2.0
    np.testing.assert_allclose(out, [[a, -a]], rtol=1e-14)


def test_invariants():
    r = rng(3)
    L, d, F = 9, 4, 6
    x, Wg, Wu, Wd = r.normal(size=(L, d)), r.normal(size=(F, d)), r.normal(size=(F, d)), r.normal(size=(d, F))
    base = O.shared_mlp(x, Wg, Wu, Wd)
    np.testing.assert_allclose(O.shared_mlp(x, Wg, Wu, 3.0 * Wd), 3.0 * base, rtol=1e-12)
    pi = r.permutation(L)
    np.testing.assert_allclose(O.shared_mlp(x[pi], Wg, Wu, Wd), base[pi], rtol=1e-12)
    # permuting the hidden units (rows of W_g, W_u with columns of W_d) changes nothing
    h = r.permutation(F)
    np.testing.assert_allclose(O.shared_mlp(x, Wg[h], Wu[h], Wd[:, h]), base, rtol=1e-12, atol=1e-14)


def test_layer_is_the_sum_of_the_branches():
    r = rng(4)
    L, d, Nr, Nc, K, F = 6, 8, 4, 5, 3, 16
    x = r.normal(size=(L, d))
    Wr, Wc = r.normal(size=(Nr, d)), r.normal(size=(Nc, d))
    W, V = r.normal(size=(Nr * Nc, d)), r.normal(size=(Nr * Nc, d))
    Wg, Wu, Wd = r.normal(size=(F, d)), r.normal(size=(F, d)), r.normal(size=(d, F))
    out = O.layer_forward(x, Wr, Wc, W, V, K, 2, Wg, Wu, Wd)
    np.testing.assert_allclose(out["layer"], loops(x, Wg, Wu, Wd) + out["y"], rtol=1e-12, atol=1e-12)
