"""Pins of the backward oracle.

The gradients are checked against central finite differences of the forward
oracle (itself pinned by brute force and closed forms), so a dropped term, a
wrong sign or a transposed operand anywhere in the chain rule fails here.
Further pins: the per-group matrix form of the expert backward against the
per-task sums, K = 1 (a single selected expert has gate 1, so the router
receives no gradient), the exact vanishing of sum_k dS_k, token permutation
and linearity in the upstream gradient.
"""

import numpy as np
import pytest

from oracle import omni_backward_oracle as BO
from oracle import omni_oracle as O


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def problem(seed, L=5, d=10, Nr=5, Nc=6, K=4, scale=1.0):
    r = rng(seed)
    N = Nr * Nc
    return dict(
        x=r.normal(size=(L, d)) * scale,
        Wr=r.normal(size=(Nr, d)) / np.sqrt(d) * 3.0,
        Wc=r.normal(size=(Nc, d)) / np.sqrt(d) * 3.0,
        W=r.normal(size=(N, d)) / np.sqrt(d),
        V=r.normal(size=(N, d)) / np.sqrt(d),
        dy=r.normal(size=(L, d)),
        K=K,
    )


def loss(P, **override):
    q = dict(P)
    q.update(override)
    out = O.routed_forward(q["x"], q["Wr"], q["Wc"], q["W"], q["V"], q["K"], B=4)
    return float((q["dy"] * out["y"]).sum()), out["idx"]


def fd(P, name, coord, eps=1e-6):
    base_idx = loss(P)[1]
    plus, minus = P[name].copy(), P[name].copy()
    plus[coord] += eps
    minus[coord] -= eps
    lp, ip = loss(P, **{name: plus})
    lm, im = loss(P, **{name: minus})
    assert np.array_equal(ip, base_idx) and np.array_equal(im, base_idx), "selection moved"
    return (lp - lm) / (2 * eps)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_gradients_match_finite_differences(seed):
    P = problem(seed)
    G = BO.routed_backward(P["x"], P["Wr"], P["Wc"], P["W"], P["V"], P["K"], P["dy"])
    uniq = list(G["uniq"])
    r = rng(100 + seed)
    N, d = P["W"].shape
    unused = sorted(set(range(N)) - set(uniq))

    def grad_of(name, coord):
        if name == "x":
            return G["dx"][coord]
        if name == "Wr":
            return G["dWr"][coord]
        if name == "Wc":
            return G["dWc"][coord]
        e, c = coord
        if e not in uniq:
            return 0.0
        return G["d" + name][uniq.index(e), c]

    coords = []
    for name, shape in (("x", P["x"].shape), ("Wr", P["Wr"].shape), ("Wc", P["Wc"].shape)):
        for _ in range(6):
            coords.append((name, tuple(int(v) for v in (r.integers(shape[0]), r.integers(shape[1])))))
    for name in ("W", "V"):
        for _ in range(6):
            coords.append((name, (int(r.choice(uniq)), int(r.integers(d)))))
        if unused:
            coords.append((name, (int(unused[0]), int(r.integers(d)))))
    for name, coord in coords:
        want = fd(P, name, coord)
        got = grad_of(name, coord)
        assert abs(got - want) <= 1e-6 * (1.0 + abs(want)), (name, coord, got, want)


def test_dgate_and_dscore_match_finite_differences():
    """dgate = a u and dS (softmax Jacobian), each against differences of y."""
    P = problem(7, L=3, K=5)
    idx, score, gate, _, _ = O.route(P["x"], P["Wr"], P["Wc"], P["K"])
    terms = BO.task_terms(P["x"], P["W"], P["V"], idx, gate, P["dy"])
    dgate = terms["dgate"].reshape(idx.shape)
    dS = BO.score_grad(gate, dgate)
    eps = 1e-6

    def loss_of_gate(gt):
        y = O.assemble_token_centric(P["x"], P["W"], P["V"], idx, gt)
        return float((P["dy"] * y).sum())

    def loss_of_score(sc):
        return loss_of_gate(O.gate_softmax(sc))

    for t in range(idx.shape[0]):
        for k in range(idx.shape[1]):
            for f, arg, want in ((loss_of_gate, gate, dgate), (loss_of_score, score, dS)):
                p, m = arg.copy(), arg.copy()
                p[t, k] += eps
                m[t, k] -= eps
                num = (f(p) - f(m)) / (2 * eps)
                assert abs(num - want[t, k]) <= 1e-7 * (1 + abs(num))


@pytest.mark.parametrize("B", [1, 3, 8, 1000])
def test_grouped_matrix_form_equals_per_task_sums(B):
    """Few experts, many tasks: experts repeat across tokens and groups."""
    r = rng(B)
    L, d, N, K = 23, 9, 14, 5
    x, W, V, dy = (r.normal(size=s) for s in ((L, d), (N, d), (N, d), (L, d)))
    idx = np.stack([r.choice(N, size=K, replace=False) for _ in range(L)])
    gate = r.dirichlet(np.ones(K), size=L)
    perm, off = O.schedule(idx, N, B)
    e_g, dW_g, dV_g, dx_g = BO.expert_grads_grouped(x, W, V, idx, gate, dy, perm, off)
    terms = BO.task_terms(x, W, V, idx, gate, dy)
    uniq = np.unique(idx)
    dW, dV = BO.expert_grads(x, dy, idx, terms, uniq)
    dx = BO.input_grad_expert(W, idx, terms["dh"])
    assert np.array_equal(e_g, uniq)
    np.testing.assert_allclose(dW_g, dW, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dV_g, dV, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dx_g, dx, rtol=1e-12, atol=1e-12)


def test_k1_router_gets_no_gradient():
    P = problem(3, K=1)
    G = BO.routed_backward(P["x"], P["Wr"], P["Wc"], P["W"], P["V"], 1, P["dy"])
    assert np.all(G["dS"] == 0.0)
    assert np.all(G["dWr"] == 0.0) and np.all(G["dWc"] == 0.0)
    np.testing.assert_array_equal(G["dx"], G["dx_expert"])


def test_score_gradient_sums_to_zero_and_logsoftmax_term_vanishes():
    P = problem(4, L=8, Nr=7, Nc=9, K=6)
    idx, score, gate, _, _ = O.route(P["x"], P["Wr"], P["Wc"], P["K"])
    dgate = BO.task_terms(P["x"], P["W"], P["V"], idx, gate, P["dy"])["dgate"].reshape(idx.shape)
    dS = BO.score_grad(gate, dgate)
    assert np.all(np.abs(dS.sum(axis=1)) <= 1e-15 * (1 + np.abs(dS).sum(axis=1)))
    ds_r, ds_c = BO.logit_grads(P["x"], P["Wr"], P["Wc"], idx, dS)
    # without the LogSoftmax mean term the raw logit gradient is dp itself
    Nc = P["Wc"].shape[0]
    dp_r = np.zeros_like(ds_r)
    np.add.at(dp_r, (np.repeat(np.arange(idx.shape[0]), idx.shape[1]), idx.reshape(-1) // Nc),
              dS.reshape(-1))
    assert np.max(np.abs(ds_r - dp_r)) <= 1e-14 * max(1.0, np.max(np.abs(dp_r)))


def test_token_permutation_and_linearity():
    P = problem(5, L=7)
    G = BO.routed_backward(P["x"], P["Wr"], P["Wc"], P["W"], P["V"], P["K"], P["dy"])
    pi = rng(9).permutation(P["x"].shape[0])
    Gp = BO.routed_backward(P["x"][pi], P["Wr"], P["Wc"], P["W"], P["V"], P["K"], P["dy"][pi])
    np.testing.assert_allclose(Gp["dx"], G["dx"][pi], rtol=1e-12, atol=1e-12)
    for k in ("dW", "dV", "dWr", "dWc"):
        np.testing.assert_allclose(Gp[k], G[k], rtol=1e-11, atol=1e-12)
    G2 = BO.routed_backward(P["x"], P["Wr"], P["Wc"], P["W"], P["V"], P["K"], 2.5 * P["dy"])
    for k in ("dx", "dW", "dV", "dWr", "dWc", "dgate"):
        np.testing.assert_allclose(G2[k], 2.5 * G[k], rtol=1e-12, atol=1e-12)


def test_single_task_closed_form():
    """L = 1, K = 1: gate 1, y = SiLU(h) v, so dV = SiLU(h) dy, dW = u SiLU'(h) x."""
    r = rng(12)
    d = 6
    x, w, v, dy = (r.normal(size=d) for _ in range(4))
    h = float(x @ w)
    sig = 1 / (1 + np.exp(-h))
    u = float(v @ dy)
    terms = BO.task_terms(x[None], w[None], v[None], np.zeros((1, 1), int), np.ones((1, 1)), dy[None])
    dW, dV = BO.expert_grads(x[None], dy[None], np.zeros((1, 1), int), terms, [0])
    np.testing.assert_allclose(dV[0], h * sig * dy, rtol=1e-14)
    np.testing.assert_allclose(dW[0], u * (sig + h * sig * (1 - sig)) * x, rtol=1e-14)
    dx = BO.input_grad_expert(w[None], np.zeros((1, 1), int), terms["dh"])
    np.testing.assert_allclose(dx[0], u * (sig + h * sig * (1 - sig)) * w, rtol=1e-14)
