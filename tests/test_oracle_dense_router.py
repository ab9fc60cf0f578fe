"""Pins of the oracle's dense (fully connected) router.

Checked against Python's sorted() over every expert, against the Cartesian
router when the dense weights are the sums W_r[i] + W_c[j] (then the
LogSoftmax over all N experts factorises into p_r[i] + p_c[j] exactly, so
the two routers must select the same experts with the same scores), and
special cases (K = N, K = 1).
"""

import math

import numpy as np
import pytest

from oracle import omni_oracle as O


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def test_matches_python_sorted():
    r = rng(1)
    L, d, N, K = 5, 7, 40, 6
    x, Wn = r.normal(size=(L, d)), r.normal(size=(N, d))
    idx, score, gate = O.dense_route(x, Wn, K)
    for t in range(L):
        s = [sum(x[t, c] * Wn[n, c] for c in range(d)) for n in range(N)]
        m = max(s)
        lse = m + math.log(sum(math.exp(v - m) for v in s))
        want = sorted(range(N), key=lambda n: (-(s[n] - lse), n))[:K]
        assert idx[t].tolist() == want
        np.testing.assert_allclose(score[t], [s[n] - lse for n in want], rtol=0, atol=1e-12)
        np.testing.assert_allclose(gate[t].sum(), 1.0, rtol=1e-14)


@pytest.mark.parametrize("seed", [2, 3, 4])
def test_factorised_weights_reproduce_the_cartesian_router(seed):
    r = rng(seed)
    L, d, Nr, Nc, K = 6, 9, 7, 5, 8
    x, Wr, Wc = r.normal(size=(L, d)), r.normal(size=(Nr, d)), r.normal(size=(Nc, d))
    Wn = (Wr[:, None, :] + Wc[None, :, :]).reshape(Nr * Nc, d)  # row n = i*Nc + j
    idx_d, score_d, gate_d = O.dense_route(x, Wn, K)
    idx_c, score_c, gate_c, _, _ = O.route(x, Wr, Wc, K)
    np.testing.assert_array_equal(idx_d, idx_c)
    np.testing.assert_allclose(score_d, score_c, rtol=0, atol=1e-12)
    np.testing.assert_allclose(gate_d, gate_c, rtol=0, atol=1e-12)


def test_special_cases():
    r = rng(5)
    L, d, N = 4, 3, 9
    x, Wn = r.normal(size=(L, d)), r.normal(size=(N, d))
    idx, _, gate = O.dense_route(x, Wn, N)
    assert all(sorted(row) == list(range(N)) for row in idx.tolist())
    idx1, _, gate1 = O.dense_route(x, Wn, 1)
    np.testing.assert_array_equal(idx1[:, 0], np.argmax(x @ Wn.T, axis=1))
    assert np.all(gate1 == 1.0)
