"""CPU oracle of the OmniMoE routed-branch backward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite uses it.  It shares no code with the
HIP library and imports nothing from the package; it builds on the forward
oracle (omni_oracle), whose definitions it differentiates.

Everything is float64 from the exact input values, written as the plain
chain rule of the forward definitions:

  forward, per token t  [digest (paper.rainbus.top), method paragraph,
  steps 1-3; gist.science resume sections 2.1-2.2]
    s_r = x_t W_r^T, s_c = x_t W_c^T, p = LogSoftmax(s)
    S_k = p_r[i_k] + p_c[j_k] over the selected ids n_k = i_k N_c + j_k
    g = softmax(S)
    y_t = sum_k g_k SiLU(x_t . W[n_k]) V[n_k]

  backward of a scalar loss with upstream gradient dy = dLoss/dy
    per task (t, k), e = n_k:  h = x_t . W[e], a = SiLU(h), u = V[e] . dy_t
      dgate_k = a u
      dh      = g_k u SiLU'(h),      SiLU'(h) = sig(h) (1 + h (1 - sig(h)))
      dV[e]  += g_k a dy_t,  dW[e] += dh x_t,  dx_t += dh W[e]
    router: dS = g * (dgate - sum_k g_k dgate_k)        (softmax Jacobian)
      dp_r[i_k] += dS_k, dp_c[j_k] += dS_k
      ds = dp - softmax(s) * sum(dp)                     (LogSoftmax Jacobian)
      dW_r = ds_r^T x, dW_c = ds_c^T x, dx += ds_r W_r + ds_c W_c

The top-K selection is piecewise constant in its inputs, so it contributes
no gradient: ids are fixed at their forward values (the gradient exists
wherever the selection is not at a tie).

Pinned by tests/test_oracle_backward.py: central finite differences of the
forward oracle, the per-group matrix form against the per-task sums, K = 1
(no router gradient), the vanishing of sum_k dS_k, and token permutation.
"""

from __future__ import annotations

import numpy as np

from oracle import omni_oracle as O

F64 = np.float64


def sigmoid(h):
    h = O.as_f64(h)
    return 1.0 / (1.0 + np.exp(-h))


def silu_grad(h):
    """d/dh of h * sigmoid(h) = sig(h) (1 + h (1 - sig(h)))."""
    h = O.as_f64(h)
    s = sigmoid(h)
    return s * (1.0 + h * (1.0 - s))


# ---------------------------------------------------------------------------
# Expert branch
# ---------------------------------------------------------------------------

def task_terms(x, W, V, idx, gate, dy, m=None):
    """Per-task scalars of the backward for task ids m (default: all).

    Returns dict of float64 arrays over the tasks: t, e, h, a, u,
    dgate (= a u), dh (= g u SiLU'(h)), ga (= g a).
    W and V may be any object supporting W[int array] -> [n, d] rows.
    """
    x, dy, gate = O.as_f64(x), O.as_f64(dy), O.as_f64(gate)
    idx = np.asarray(idx, np.int64)
    L, K = idx.shape
    if m is None:
        m = np.arange(L * K, dtype=np.int64)
    m = np.asarray(m, np.int64)
    t = m // K
    e = idx.reshape(-1)[m]
    g = gate.reshape(-1)[m]
    Wm = O.as_f64(W[e])
    Vm = O.as_f64(V[e])
    h = np.einsum("md,md->m", x[t], Wm)
    u = np.einsum("md,md->m", dy[t], Vm)
    a = O.silu(h)
    return dict(t=t, e=e, h=h, a=a, u=u, dgate=a * u, dh=g * u * silu_grad(h), ga=g * a)


def expert_grads(x, dy, idx, terms, experts):
    """dW[e] = sum of dh x_t and dV[e] = sum of g a dy_t over e's tasks.

    `terms` must cover every task of the listed experts (e.g. all tasks).
    Returns (dW [len(experts), d], dV [len(experts), d]) float64.
    """
    x, dy = O.as_f64(x), O.as_f64(dy)
    experts = np.asarray(experts, np.int64)
    d = x.shape[1]
    dW = np.zeros((experts.size, d), F64)
    dV = np.zeros((experts.size, d), F64)
    for r, ex in enumerate(experts):
        sel = terms["e"] == ex
        ts = terms["t"][sel]
        dW[r] = terms["dh"][sel] @ x[ts]
        dV[r] = terms["ga"][sel] @ dy[ts]
    return dW, dV


def input_grad_expert(W, idx, dh, tokens=None):
    """Expert part of dx: dx_t = sum_k dh_{t,k} W[idx[t,k]] (rows of `tokens`).

    dh is indexed by task id (shape [L*K] or [L, K]).
    """
    idx = np.asarray(idx, np.int64)
    L, K = idx.shape
    dh = O.as_f64(dh).reshape(L, K)
    if tokens is None:
        tokens = np.arange(L)
    rows = []
    for t in tokens:
        rows.append(dh[t] @ O.as_f64(W[idx[t]]))
    return np.stack(rows) if rows else np.zeros((0, 0), F64)


def expert_grads_grouped(x, W, V, idx, gate, dy, perm, group_off):
    """The expert backward as the per-group matrix product of the schedule.

    For group q (digest, step 3: O_q = (G_q . sigma(X_q W_q^T)) V_q with
    H_q = X_q W_q^T), with dO_q the rows of dy at the group's tokens:
      dA_q = dO_q V_q^T;  dV_q = (G_q . sigma(H_q))^T dO_q
      dH_q = G_q . sigma'(H_q) . dA_q;  dW_q = dH_q^T X_q;  dX_q = dH_q W_q
    Returns (uniq experts ascending, dW [U, d], dV [U, d], dx_expert [L, d]).
    """
    x, dy, gate = O.as_f64(x), O.as_f64(dy), O.as_f64(gate)
    idx = np.asarray(idx, np.int64)
    L, K = idx.shape
    d = x.shape[1]
    dx = np.zeros((L, d), F64)
    out_e, out_W, out_V = [], [], []
    for q in range(len(group_off) - 1):
        lo, hi = int(group_off[q]), int(group_off[q + 1])
        if lo == hi:
            continue
        ms = np.asarray(perm[lo:hi], np.int64)
        tok, tok_pos = np.unique(ms // K, return_inverse=True)
        ex, ex_pos = np.unique(idx.reshape(-1)[ms], return_inverse=True)
        Gq = np.zeros((tok.size, ex.size), F64)
        Gq[tok_pos, ex_pos] = gate.reshape(-1)[ms]
        Xq, dOq = x[tok], dy[tok]
        Wq, Vq = O.as_f64(W[ex]), O.as_f64(V[ex])
        Hq = Xq @ Wq.T
        dAq = dOq @ Vq.T
        dVq = (Gq * O.silu(Hq)).T @ dOq
        dHq = Gq * silu_grad(Hq) * dAq
        out_e.append(ex)
        out_W.append(dHq.T @ Xq)
        out_V.append(dVq)
        dx[tok] += dHq @ Wq
    e = np.concatenate(out_e) if out_e else np.zeros(0, np.int64)
    order = np.argsort(e, kind="stable")
    cat = lambda parts: np.concatenate(parts)[order] if parts else np.zeros((0, d), F64)
    return e[order], cat(out_W), cat(out_V), dx


# ---------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------

def score_grad(gate, dgate):
    """dS = g * (dgate - sum_k g_k dgate_k), the softmax Jacobian per token."""
    gate, dgate = O.as_f64(gate), O.as_f64(dgate)
    return gate * (dgate - (gate * dgate).sum(axis=-1, keepdims=True))


def logit_grads(x, Wr, Wc, idx, dS):
    """ds_r [L, N_r], ds_c [L, N_c]: the gradient of the raw row / column logits.

    dp_r[t, i] sums dS over the token's selected ids in row i (likewise
    columns); the LogSoftmax Jacobian then gives ds = dp - softmax(s) sum(dp).
    """
    idx = np.asarray(idx, np.int64)
    dS = O.as_f64(dS)
    Wr, Wc = O.as_f64(Wr), O.as_f64(Wc)
    L, K = idx.shape
    Nr, Nc = Wr.shape[0], Wc.shape[0]
    t = np.repeat(np.arange(L), K)
    rows, cols = idx.reshape(-1) // Nc, idx.reshape(-1) % Nc
    dp_r = np.zeros((L, Nr), F64)
    dp_c = np.zeros((L, Nc), F64)
    np.add.at(dp_r, (t, rows), dS.reshape(-1))
    np.add.at(dp_c, (t, cols), dS.reshape(-1))
    s_r, s_c = O.project(x, Wr, Wc)
    sm_r = np.exp(O.log_softmax(s_r))
    sm_c = np.exp(O.log_softmax(s_c))
    ds_r = dp_r - sm_r * dp_r.sum(axis=-1, keepdims=True)
    ds_c = dp_c - sm_c * dp_c.sum(axis=-1, keepdims=True)
    return ds_r, ds_c


def router_backward(x, Wr, Wc, idx, gate, dgate):
    """Router gradients: (dWr [N_r, d], dWc [N_c, d], dx_router [L, d], dS [L, K])."""
    x, Wr, Wc = O.as_f64(x), O.as_f64(Wr), O.as_f64(Wc)
    dS = score_grad(gate, dgate)
    ds_r, ds_c = logit_grads(x, Wr, Wc, idx, dS)
    return ds_r.T @ x, ds_c.T @ x, ds_r @ Wr + ds_c @ Wc, dS


# ---------------------------------------------------------------------------
# End to end
# ---------------------------------------------------------------------------

def routed_backward(x, Wr, Wc, W, V, K, dy):
    """Gradients of sum(dy * y) for the routed branch, all parameters.

    Returns dict: idx, gate (forward routing), dgate [L, K], uniq (used
    experts, ascending), dW [U, d], dV [U, d] (rows of uniq), dx [L, d]
    (expert + router parts), dx_expert, dWr, dWc.
    """
    idx, score, gate, _, _ = O.route(x, Wr, Wc, K)
    terms = task_terms(x, W, V, idx, gate, dy)
    uniq = np.unique(idx)
    dW, dV = expert_grads(x, dy, idx, terms, uniq)
    dx_e = input_grad_expert(W, idx, terms["dh"])
    dgate = terms["dgate"].reshape(idx.shape)
    dWr, dWc, dx_r, dS = router_backward(x, Wr, Wc, idx, gate, dgate)
    return dict(idx=idx, gate=gate, dgate=dgate, uniq=uniq, dW=dW, dV=dV,
                dx=dx_e + dx_r, dx_expert=dx_e, dWr=dWr, dWc=dWc, dS=dS)
