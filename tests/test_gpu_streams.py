"""Two routed branches in flight on two streams.

Each branch has its own outputs and workspace and runs the whole path on
its own stream, on its own inputs; the launches of the two interleave on the
device.  Every branch's results must equal, bit for bit, those of the same
branch run alone: the library keeps no state between calls and the two
workspaces are disjoint.
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
    ((512, 256, 40, 36, 32, 16, "bf16"), {}),
    ((300, 512, 48, 48, 64, 32, "bf16"), {"token_order": True, "assembly": "expert_centric"}),
    ((128, 64, 32, 32, 16, 16, "f32"), {}),
]


@pytest.mark.parametrize("case,opts", CASES,
                         ids=lambda c: "-".join(f"{k}={v}" for k, v in c.items()) if isinstance(c, dict)
                         else "L{}_d{}_{}x{}_K{}_B{}_{}".format(*c))
def test_two_streams_match_one(case, opts):
    L, d, Nr, Nc, K, B, dtype = case
    print(f"two-stream case {case} {opts}", flush=True)
    ins = []
    for seed in (11, 12):
        w, cpu = synth.make_case(L, d, Nr, Nc, K, B, dtype, seed=seed)
        ins.append({k: v.cuda() for k, v in cpu.items()})
    want = []
    for inp in ins:
        ref = omni.RoutedBranch(L, d, Nr, Nc, K, B, w.torch_dtype, **opts)
        ref.forward(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"])
        torch.cuda.synchronize()
        names = ("idx", "gate", "y") + (("perm", "group_off") if ref.assembly != "auto" else ())
        want.append({k: getattr(ref, k).clone() for k in names})
    branches = [omni.RoutedBranch(L, d, Nr, Nc, K, B, w.torch_dtype, **opts) for _ in ins]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    start = torch.cuda.Event()
    start.record(torch.cuda.current_stream())
    for st in streams:
        st.wait_event(start)
    for step in range(6):
        i = step % 2
        with torch.cuda.stream(streams[i]):
            inp = ins[i]
            branches[i].forward(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"])
    torch.cuda.synchronize()
    for i, br in enumerate(branches):
        for k, v in want[i].items():
            assert torch.equal(getattr(br, k), v), (i, k)
    assert not torch.equal(branches[0].y, branches[1].y)
