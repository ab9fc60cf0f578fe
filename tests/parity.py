"""Comparison rules between the HIP path and the CPU oracle.

* top-K: every token's GPU id set holds K distinct ids in [0, N); ids in the
  symmetric difference with the oracle's set must score within TOPK_TOL of
  the oracle's K-th score (swaps of near-ties); the GPU score of each id must
  be within TOPK_TOL of the oracle's S for that id; the GPU rows must be
  ordered by (score desc, id asc); the GPU gate must be within TOPK_TOL of
  the softmax of the oracle's scores over the GPU's own selected set.
* schedule: perm and group_off bit-exact against the oracle's schedule of
  the same idx array.
* y: judged on identical routing (the oracle's assembly of the GPU's idx and
  gate), norm-wise: ||dy||_F <= rtol ||y*||_F and max|dy| <= rtol max|y*|.
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import omni_oracle as O

TOPK_TOL = 1e-5
RTOL = {"f32": 1e-4, "bf16": 2e-2}
# Every product and sum runs in fp32 for both dtypes (bf16 inputs are widened
# exactly), so fp32 rounding bounds the error of either path: the test also
# holds both to this tighter bound.
RTOL_FP32_ARITH = 1e-4


def to_np(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        t = t.detach().to("cpu")
        if t.dtype == torch.bfloat16:
            t = t.to(torch.float64)
        return t.numpy()
    return np.asarray(t)


class DeviceRows:
    """W[ids] for a device tensor: gathers only the requested rows (float64)."""

    def __init__(self, t: torch.Tensor):
        self.t = t

    def __getitem__(self, ids):
        ids = torch.as_tensor(np.asarray(ids, np.int64), device=self.t.device)
        return self.t.index_select(0, ids.reshape(-1)).to("cpu", torch.float64).numpy().reshape(
            tuple(np.shape(ids)) + (self.t.shape[1],))


def oracle_router_tokens(x_rows, Wr, Wc, K):
    """Oracle routing of some tokens (rows of x given as float64)."""
    return O.route(x_rows, Wr, Wc, K)


def check_topk(idx_g, score_g, gate_g, p_r, p_c, K, tol=TOPK_TOL):
    """Apply the top-K rule; returns the number of tolerated swaps."""
    idx_g, score_g, gate_g = to_np(idx_g), to_np(score_g), to_np(gate_g)
    p_r, p_c = np.asarray(p_r), np.asarray(p_c)
    L, Nr = p_r.shape
    Nc = p_c.shape[1]
    N = Nr * Nc
    idx_o, score_o = O.topk_implicit(p_r, p_c, K)
    swaps = 0
    for t in range(L):
        ids = idx_g[t].astype(np.int64)
        assert ids.min() >= 0 and ids.max() < N, f"token {t}: id out of range"
        assert len(set(ids.tolist())) == K, f"token {t}: repeated ids"
        S_at = p_r[t, ids // Nc] + p_c[t, ids % Nc]
        err = np.abs(score_g[t].astype(np.float64) - S_at).max()
        assert err <= tol, f"token {t}: score error {err:.3g}"
        # ordering by (score desc, id asc) of the GPU's own values
        for k in range(K - 1):
            a, b = score_g[t, k], score_g[t, k + 1]
            assert a > b or (a == b and ids[k] < ids[k + 1]), f"token {t}: order broken at {k}"
        s_star = score_o[t, K - 1]
        diff = set(ids.tolist()) ^ set(idx_o[t].tolist())
        for n in diff:
            S = p_r[t, n // Nc] + p_c[t, n % Nc]
            assert abs(S - s_star) <= tol, (
                f"token {t}: id {n} (S={S:.8f}) differs from the oracle set, "
                f"K-th score {s_star:.8f}")
        swaps += len(diff) // 2
        g_ref = O.gate_softmax(S_at[None])[0]
        gerr = np.abs(gate_g[t].astype(np.float64) - g_ref).max()
        assert gerr <= tol, f"token {t}: gate error {gerr:.3g}"
    return swaps


def check_schedule(idx, perm_g, off_g, N, B):
    perm_o, off_o = O.schedule(to_np(idx).astype(np.int64), N, B)
    np.testing.assert_array_equal(to_np(perm_g).astype(np.int64), perm_o)
    np.testing.assert_array_equal(to_np(off_g).astype(np.int64), off_o)


def y_errors(y_g, y_o):
    y_g = to_np(y_g).astype(np.float64)
    y_o = np.asarray(y_o, np.float64)
    dy = y_g - y_o
    nrm = np.linalg.norm(dy) / max(np.linalg.norm(y_o), 1e-300)
    mx = np.abs(dy).max() / max(np.abs(y_o).max(), 1e-300)
    return nrm, mx


def check_y(y_g, y_o, rtol):
    nrm, mx = y_errors(y_g, y_o)
    assert nrm <= rtol and mx <= rtol, f"y error: norm-wise {nrm:.3g}, max {mx:.3g} (rtol {rtol})"
    return nrm, mx
