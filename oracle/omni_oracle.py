"""CPU oracle of the OmniMoE routed-branch forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the package's smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
and imports nothing from the package.

Everything is computed in float64 from the exact input values (bf16 and fp32
inputs are up-cast exactly, nothing is re-rounded).  The code is deliberately
plain: no blocking, fusion or reordering beyond what the definitions state.

Sources (web pages about "OmniMoE: An Efficient MoE by Orchestrating Atomic
Experts at Scale", arXiv 2602.05711):

* [digest]  paper.rainbus.top technical digest, method paragraph: step 1
  (atomic experts, global matrices W and V, retrieval and assembly),
  step 2 (Cartesian Product Router), step 3 (expert-centric scheduling and
  the per-group product).
* [resume-de]  gist.science (German) "Technisches Resümee", section 2.1
  (atomic experts, DEA) and section 2.2 (router; task collection,
  grouping by contiguous expert-id ranges, sub-sort by token id).
* [makerbund]  makerbund.cn article, section 五 (ablation: reverting the
  scheduling to token-centric leaves the quality unchanged).

Readings where the pages are silent (each also listed with its reason in the
design notes of the repository):

* sigma is SiLU, h / (1 + exp(-h)): each atomic expert has only an input and
  an output vector, so the "SwiGLU" remark of the digest has no gate vector
  to act on.
* the gate g_x is the softmax over the K selected scores S.
* expert id n <-> grid coordinate (i, j) is row-major: n = i * N_c + j.
* W_r and W_c are stored as [N_r, d] and [N_c, d] (one row per grid row /
  column), so s_r = x W_r^T in that storage.
* top-K uses the total order (S descending, n ascending); row and column
  pre-selection use (p descending, index ascending).
* group of expert e is floor(e / B) (B consecutive expert ids); the schedule
  is the task ids sorted by (group, token, task id).
* y starts at zero and receives every task's contribution (no bias, no
  capacity limit); the shared dense MLP is a separate branch (shared_mlp),
  read as a SwiGLU block, and layer_forward adds the two.

Pinned by the CPU tests (tests/test_oracle_*.py) against brute force, closed
forms and invariants; no function here is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

F64 = np.float64


def as_f64(a) -> np.ndarray:
    """Exact up-cast to float64 (numpy arrays or torch CPU tensors)."""
    if hasattr(a, "detach"):  # torch tensor: bf16 has no numpy dtype
        a = a.detach().to("cpu")
        import torch  # local: the oracle itself needs only numpy

        a = a.to(torch.float64).numpy()
    return np.asarray(a, dtype=F64)


# ---------------------------------------------------------------------------
# Cartesian Product Router  [digest, step 2; resume-de 2.2]
# ---------------------------------------------------------------------------

def project(x, Wr, Wc):
    """Row and column logits s_r = x W_r, s_c = x W_c  [digest, step 2].

    x [L, d]; Wr [N_r, d]; Wc [N_c, d] (row per grid row / column).
    Returns (s_r [L, N_r], s_c [L, N_c]) in float64.
    """
    x, Wr, Wc = as_f64(x), as_f64(Wr), as_f64(Wc)
    return x @ Wr.T, x @ Wc.T


def log_softmax(s):
    """LogSoftmax over the last axis: s - (max + log sum exp(s - max))."""
    s = as_f64(s)
    m = s.max(axis=-1, keepdims=True)
    return s - (m + np.log(np.exp(s - m).sum(axis=-1, keepdims=True)))


def expert_id(i, j, Nc):
    """Row-major reading of the grid coordinate (i, j) as an expert id."""
    return i * Nc + j


def _take_topk(S, n, K):
    """First K entries under the order (S desc, n asc).  S, n: 1-D."""
    order = np.lexsort((n, -S))  # last key is primary
    return n[order[:K]], S[order[:K]]


def topk_explicit(p_r, p_c, K):
    """Brute-force top-K over an explicitly built S [L, N_r*N_c].

    S_ij = p_r[i] + p_c[j]  [digest, step 2].  Only for small grids: this is
    the reference the implicit selection is checked against.
    Returns idx [L, K] int64 and score [L, K] float64, rows ordered by
    (S desc, n asc).
    """
    p_r, p_c = as_f64(p_r), as_f64(p_c)
    L, Nr = p_r.shape
    Nc = p_c.shape[1]
    if not 1 <= K <= Nr * Nc:
        raise ValueError("K must lie in [1, N_r*N_c]")
    S = (p_r[:, :, None] + p_c[:, None, :]).reshape(L, Nr * Nc)
    n_all = np.arange(Nr * Nc, dtype=np.int64)
    idx = np.empty((L, K), np.int64)
    score = np.empty((L, K), F64)
    for t in range(L):
        idx[t], score[t] = _take_topk(S[t], n_all, K)
    return idx, score


def preselect(p, Kx):
    """Indices of the first Kx entries of p under (p desc, index asc)."""
    p = as_f64(p)
    order = np.lexsort((np.arange(p.shape[0]), -p))
    return order[:Kx]


def topk_implicit(p_r, p_c, K):
    """Top-K over the implicit grid without building S  [digest, step 2].

    Any (i, j) in the top K under (S desc, n asc) has fewer than K rows that
    precede row i under (p_r desc, i asc) (each such row i' gives an (i', j)
    that precedes (i, j)), and likewise for its column.  So the top K lies in
    R x C, where R holds the first min(K, N_r) rows and C the first
    min(K, N_c) columns.  The selection is made over that K x K candidate
    set, scored with the same sums S = p_r[i] + p_c[j].
    Returns idx [L, K] int64 and score [L, K] float64 in (S desc, n asc)
    order.
    """
    p_r, p_c = as_f64(p_r), as_f64(p_c)
    L, Nr = p_r.shape
    Nc = p_c.shape[1]
    if not 1 <= K <= Nr * Nc:
        raise ValueError("K must lie in [1, N_r*N_c]")
    idx = np.empty((L, K), np.int64)
    score = np.empty((L, K), F64)
    for t in range(L):
        R = preselect(p_r[t], min(K, Nr))
        C = preselect(p_c[t], min(K, Nc))
        S = (p_r[t][R][:, None] + p_c[t][C][None, :]).ravel()
        n = expert_id(R[:, None].astype(np.int64), C[None, :].astype(np.int64), Nc).ravel()
        idx[t], score[t] = _take_topk(S, n, K)
    return idx, score


def gate_softmax(score):
    """Gate g_x = softmax over the K selected scores of each token."""
    score = as_f64(score)
    e = np.exp(score - score.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def route(x, Wr, Wc, K, method="implicit"):
    """Full router: projections, LogSoftmax, top-K, gate.

    Returns (idx [L,K] int64, score [L,K] f64, gate [L,K] f64,
    p_r [L,N_r] f64, p_c [L,N_c] f64).
    """
    s_r, s_c = project(x, Wr, Wc)
    p_r, p_c = log_softmax(s_r), log_softmax(s_c)
    if method == "implicit":
        idx, score = topk_implicit(p_r, p_c, K)
    elif method == "explicit":
        idx, score = topk_explicit(p_r, p_c, K)
    else:
        raise ValueError(method)
    return idx, score, gate_softmax(score), p_r, p_c


# ---------------------------------------------------------------------------
# Expert-centric scheduling  [digest, step 3; resume-de 2.2]
# ---------------------------------------------------------------------------

def num_groups(N, B):
    return -(-N // B)


def tasks(idx):
    """Task collection: task m = t*K + k is (token t, expert idx[t,k])."""
    idx = np.asarray(idx, np.int64)
    L, K = idx.shape
    m = np.arange(L * K, dtype=np.int64)
    return m, m // K, idx.reshape(-1)


def schedule(idx, N, B):
    """Sort the L*K tasks by (group, token, task id); group = expert // B.

    Groups are contiguous ranges of B expert ids [resume-de 2.2]; the
    primary key is the group id and the secondary key the token id
    [digest, step 3]; the task id breaks the remaining ties.
    Returns perm [L*K] int64 (task ids in schedule order) and
    group_off [G+1] int64, group_off[q] = #{tasks whose group < q}.
    """
    m, t, e = tasks(idx)
    if e.size and (e.min() < 0 or e.max() >= N):
        raise ValueError("expert id out of range")
    g = e // B
    perm = np.lexsort((m, t, g))  # primary g, then t, then m
    G = num_groups(N, B)
    counts = np.bincount(g, minlength=G)
    group_off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return perm.astype(np.int64), group_off


def token_order(idx, B):
    """Tokens sorted by the group of their first (highest-scoring) expert,
    ties by token id: tokens whose leading experts share a group come
    together.  A processing order for the per-token output sum (it changes
    which tokens run side by side, never a token's result).
    Returns order [L] int64.
    """
    idx = np.asarray(idx, np.int64)
    L = idx.shape[0]
    return np.lexsort((np.arange(L), idx[:, 0] // B)).astype(np.int64)


# ---------------------------------------------------------------------------
# Dynamic Expert Assembly  [digest, steps 1 and 3; resume-de 2.1]
# ---------------------------------------------------------------------------

def silu(h):
    """SiLU(h) = h * sigmoid(h) = h / (1 + exp(-h))."""
    h = as_f64(h)
    return h / (1.0 + np.exp(-h))


def assemble_expert_centric(x, W, V, idx, gate, perm, group_off):
    """y from the per-group products O_q = (G_q . sigma(X_q W_q^T)) V_q.

    [digest, step 3]: for each active group q (non-empty segment of the
    schedule), X_q stacks the distinct tokens of the group's tasks (in
    schedule order), W_q and V_q the rows of the distinct experts they use,
    and G_q [tokens x experts] holds each task's gate at its (token, expert)
    entry and zero elsewhere.  O_q's rows are added into y at their tokens.

    W and V may be any object supporting W[int array] -> [n, d] rows.
    """
    x = as_f64(x)
    idx = np.asarray(idx, np.int64)
    gate = as_f64(gate)
    L, K = idx.shape
    d = x.shape[1]
    y = np.zeros((L, d), F64)
    G = len(group_off) - 1
    for q in range(G):
        lo, hi = int(group_off[q]), int(group_off[q + 1])
        if lo == hi:
            continue  # inactive group
        ms = np.asarray(perm[lo:hi], np.int64)
        t_q = ms // K
        e_q = idx.reshape(-1)[ms]
        tok, tok_pos = np.unique(t_q, return_inverse=True)
        exp_ids, exp_pos = np.unique(e_q, return_inverse=True)
        Gq = np.zeros((tok.size, exp_ids.size), F64)
        # top-K ids of a token are distinct, so no (token, expert) entry repeats
        Gq[tok_pos, exp_pos] = gate.reshape(-1)[ms]
        Xq = x[tok]
        Wq = as_f64(W[exp_ids])
        Vq = as_f64(V[exp_ids])
        Oq = (Gq * silu(Xq @ Wq.T)) @ Vq
        y[tok] += Oq
    return y


def assemble_token_centric(x, W, V, idx, gate, tokens=None):
    """Plain token-centric definition y_t = (g_x . sigma(x w_x^T)) v_x.

    [digest, step 1]: w_x = W[I_x] and v_x = V[I_x] are the token's K rows.
    `tokens` restricts the computation to some token ids (rows of the
    result follow that list).
    """
    x = as_f64(x)
    idx = np.asarray(idx, np.int64)
    gate = as_f64(gate)
    if tokens is None:
        tokens = np.arange(idx.shape[0])
    y = np.zeros((len(tokens), x.shape[1]), F64)
    for r, t in enumerate(tokens):
        w_x = as_f64(W[idx[t]])
        v_x = as_f64(V[idx[t]])
        y[r] = (gate[t] * silu(w_x @ x[t])) @ v_x
    return y


def routed_forward(x, Wr, Wc, W, V, K, B):
    """Router, schedule and expert-centric assembly, end to end."""
    idx, score, gate, _, _ = route(x, Wr, Wc, K)
    Nr, Nc = as_f64(Wr).shape[0], as_f64(Wc).shape[0]
    perm, group_off = schedule(idx, Nr * Nc, B)
    y = assemble_expert_centric(x, W, V, idx, gate, perm, group_off)
    return dict(idx=idx, score=score, gate=gate, perm=perm,
                group_off=group_off, y=y)


# ---------------------------------------------------------------------------
# Shared dense MLP and the whole layer  [digest, step 1: y = ... + MLP(x);
# resume-de 2.1: a standard dense MLP branch active for every input]
# ---------------------------------------------------------------------------

def shared_mlp(x, Wg, Wu, Wd):
    """MLP(x) = (SiLU(x W_g^T) * (x W_u^T)) W_d^T, a SwiGLU feed-forward block.

    The pages name the branch and its role but not its shape; the digest's
    "SwiGLU" remark has no gate vector to act on in an atomic expert and is
    read as describing this branch.  Wg, Wu [d_ff, d]; Wd [d, d_ff] (one row
    per output, the layout of a linear layer's weight).
    """
    x, Wg, Wu, Wd = as_f64(x), as_f64(Wg), as_f64(Wu), as_f64(Wd)
    return (silu(x @ Wg.T) * (x @ Wu.T)) @ Wd.T


def layer_forward(x, Wr, Wc, W, V, K, B, Wg, Wu, Wd):
    """The whole layer: routed branch plus the shared dense MLP."""
    out = routed_forward(x, Wr, Wc, W, V, K, B)
    out["mlp"] = shared_mlp(x, Wg, Wu, Wd)
    out["layer"] = out["y"] + out["mlp"]
    return out


# ---------------------------------------------------------------------------
# Dense router  [makerbund, section 五: the ablation that replaces the
# Cartesian Product Router by a fully connected router over all N experts]
# ---------------------------------------------------------------------------

def dense_select(s, K):
    """The dense router's steps after the logits: p = LogSoftmax(s) over the
    N experts, top-K under (p desc, n asc), gate = softmax over the K
    selected scores.  s [L, N].  Returns (idx [L,K] int64, score, gate)."""
    s = as_f64(s)
    N = s.shape[1]
    if not 1 <= K <= N:
        raise ValueError("K must lie in [1, N]")
    p = log_softmax(s)
    n_all = np.arange(N, dtype=np.int64)
    idx = np.empty((s.shape[0], K), np.int64)
    score = np.empty((s.shape[0], K), F64)
    for t in range(s.shape[0]):
        idx[t], score[t] = _take_topk(p[t], n_all, K)
    return idx, score, gate_softmax(score)


def dense_route(x, Wn, K):
    """Fully connected router: s = x Wn^T over all N experts (Wn [N, d]),
    p = LogSoftmax(s) over the N experts, top-K under (p desc, n asc),
    gate = softmax over the K selected scores (the same conventions as the
    Cartesian router).  Returns (idx [L,K] int64, score [L,K], gate [L,K]).
    """
    return dense_select(as_f64(x) @ as_f64(Wn).T, K)
