"""GPU parity of the dense (fully connected) router against the oracle.

The same top-K rule as the Cartesian router: K distinct ids in [0, N); each
GPU score within 1e-5 of the oracle's LogSoftmax at that id; rows ordered by
(score desc, id asc); ids outside the oracle's set only as swaps within 1e-5
of the oracle's K-th score; gates within 1e-5 of the softmax of the oracle's
scores over the GPU's own ids.
"""

import numpy as np
import pytest
import torch

from atomic_expert_routing_amd import omni, synth
from oracle import omni_oracle as O
from parity import TOPK_TOL, to_np

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    omni.library()


def check_dense(idx_g, score_g, gate_g, s_oracle, K, tol=TOPK_TOL):
    """Compare with the oracle given its float64 logits s [L, N]; returns swaps."""
    idx_g, score_g, gate_g = to_np(idx_g), to_np(score_g), to_np(gate_g)
    p = O.log_softmax(s_oracle)
    idx_o, score_o, _ = O.dense_select(s_oracle, K)
    N = p.shape[1]
    swaps = 0
    for t in range(p.shape[0]):
        ids = idx_g[t].astype(np.int64)
        assert ids.min() >= 0 and ids.max() < N and len(set(ids.tolist())) == K, f"token {t}: ids"
        err = np.abs(score_g[t] - p[t, ids]).max()
        assert err <= tol, f"token {t}: score error {err:.3g}"
        for k in range(K - 1):
            a, b = score_g[t, k], score_g[t, k + 1]
            assert a > b or (a == b and ids[k] < ids[k + 1]), f"token {t}: order at {k}"
        s_star = score_o[t, K - 1]
        diff = set(ids.tolist()) ^ set(idx_o[t].tolist())
        for n in diff:
            assert abs(p[t, n] - s_star) <= tol, f"token {t}: id {n} not a near-tie swap"
        swaps += len(diff) // 2
        g_ref = O.gate_softmax(p[t, ids][None])[0]
        assert np.abs(gate_g[t] - g_ref).max() <= tol, f"token {t}: gate"
    return swaps


CASES = [
    (64, 64, 1024, 16, "f32"),
    (130, 128, 5000, 50, "bf16"),
    (40, 64, 150000, 128, "bf16"),   # three chunks, the last partial
    (16, 64, 65536 + 50, 100, "f32"),  # last chunk smaller than K
    (24, 64, 3000, 512, "bf16"),     # K at the limit
    (8, 64, 70000, 1, "bf16"),       # K = 1
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "L{}_d{}_N{}_K{}_{}".format(*c))
def test_dense_router_matches_oracle(case):
    L, d, N, K, dtype = case
    say(f"dense router case {case}")
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    x = synth.normal_rows("x", L, d, 1.0, 7, "cpu", dt)
    Wn = synth.normal_rows("W", N, d, 1.0 / np.sqrt(d) * 4, 7, "cpu", dt)
    idx, score, gate = omni.omni_dense_router(x.cuda(), Wn.cuda(), K)
    torch.cuda.synchronize()
    s = O.as_f64(x) @ O.as_f64(Wn).T
    swaps = check_dense(idx, score, gate, s, K)
    say(f"  swaps={swaps}")


def test_exact_ties_go_to_the_smaller_id():
    """All logits equal (x = 0): the K smallest ids, across chunk boundaries."""
    L, d, N, K = 6, 64, 70000, 300
    x = torch.zeros((L, d), dtype=torch.bfloat16, device="cuda")
    Wn = synth.normal_rows("W", N, d, 0.1, 3, "cuda", torch.bfloat16)
    idx, score, gate = omni.omni_dense_router(x, Wn, K)
    torch.cuda.synchronize()
    want = np.tile(np.arange(K), (L, 1))
    np.testing.assert_array_equal(to_np(idx), want)
    np.testing.assert_allclose(to_np(score), -np.log(N), rtol=0, atol=1e-5)
    np.testing.assert_allclose(to_np(gate), 1.0 / K, rtol=1e-5)


def test_full_size_dense_router_sampled():
    """4096 tokens over the 1.7M experts of the bench shape (d = 2048, K = 128):
    sampled tokens against the oracle, whose logits are formed from the
    weight rows streamed to the host in blocks."""
    w = synth.WORKLOADS[synth.HEADLINE]
    say("full-size dense router: inputs")
    x = synth.make_inputs(w, seed=0, device="cuda")["x"]
    Wn = synth.normal_rows("W", w.N, w.d, 1.0 / np.sqrt(w.d), 1, "cuda", torch.bfloat16)
    say("  dense router")
    idx, score, gate = omni.omni_dense_router(x, Wn, w.K)
    torch.cuda.synchronize()
    toks = np.array([0, 1234, w.L - 1])
    xs = to_np(x[torch.as_tensor(toks, device="cuda")]).astype(np.float64)
    s = np.empty((len(toks), w.N))
    for r0 in range(0, w.N, 65536):
        r1 = min(w.N, r0 + 65536)
        s[:, r0:r1] = xs @ to_np(Wn[r0:r1]).astype(np.float64).T
    swaps = check_dense(to_np(idx)[toks], to_np(score)[toks], to_np(gate)[toks], s, w.K)
    say(f"  swaps={swaps} over {len(toks)} tokens")
    del Wn
    torch.cuda.empty_cache()
