"""The routed forward captured as a HIP graph and replayed.

Each replay is checked bit for bit against an eager forward on the same
inputs (per-task assembly, with and without the token order, and the
blocked assembly); between replays the program runs its own eager work (a forward on
other inputs, which overwrites the shared buffers) and synchronises, so a
replay that relied on state left by the capture would fail.
"""

import pytest
import torch

from atomic_expert_routing_amd import omni, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    omni.library()


CASES = [
    ((256, 256, 40, 36, 32, 16, "bf16"), {}),
    ((64, 64, 32, 32, 16, 16, "f32"), {}),
    ((200, 256, 40, 36, 32, 16, "bf16"), {"token_order": True, "assembly": "expert_centric"}),
    ((200, 512, 40, 36, 48, 16, "bf16"), {"assembly": "blocked"}),
]


@pytest.mark.parametrize("case,opts", CASES,
                         ids=lambda c: "-".join(f"{k}={v}" for k, v in c.items()) if isinstance(c, dict)
                         else "L{}_d{}_{}x{}_K{}_B{}_{}".format(*c))
def test_graph_replays_match_eager(case, opts):
    L, d, Nr, Nc, K, B, dtype = case
    w, a_cpu = synth.make_case(L, d, Nr, Nc, K, B, dtype, seed=1)
    _, b_cpu = synth.make_case(L, d, Nr, Nc, K, B, dtype, seed=2)
    a = {k: v.cuda() for k, v in a_cpu.items()}
    b = {k: v.cuda() for k, v in b_cpu.items()}
    ref = omni.RoutedBranch(L, d, Nr, Nc, K, B, w.torch_dtype, **opts)
    ref.forward(a["x"], a["Wr"], a["Wc"], a["W"], a["V"])
    torch.cuda.synchronize()
    names = ["idx", "gate", "y"] + (["token_order"] if ref.token_order is not None else [])
    if ref.assembly == "expert_centric":  # the other forms keep the schedule to themselves
        names += ["perm", "group_off"]
    want = {k: getattr(ref, k).clone() for k in names}

    br = omni.RoutedBranch(L, d, Nr, Nc, K, B, w.torch_dtype, **opts)
    br.capture(a["x"], a["Wr"], a["Wc"], a["W"], a["V"])
    for rep in range(4):
        # eager work on other inputs through the same buffers, then replay
        br.forward(b["x"], b["Wr"], b["Wc"], b["W"], b["V"])
        torch.cuda.synchronize()
        assert not torch.equal(br.idx, want["idx"])
        br.replay()
        torch.cuda.synchronize()
        for k, v in want.items():
            assert torch.equal(getattr(br, k), v), (rep, k)
