"""GPU parity of omni_expert_forward_auto, the assembly whose form the device
chooses per call from the routing's reuse (tasks per distinct expert): the
per-task passes on spread-out routing, the blocked form where tokens pile
onto few experts.  Both choices are held to the oracle's assembly of the
same routing (fp32 arithmetic bound), and the choice itself is checked
against the device's rule replayed on the host from the ids.
"""

import zlib

import numpy as np
import pytest
import torch

from atomic_expert_routing_amd import omni, synth
from oracle import omni_oracle as O
from parity import RTOL_FP32_ARITH, check_y, to_np

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    omni.library()


SAMPLE, HASH = 65536, 2654435761


def expected_choice(idx, dt, d):
    """The rule the device applies: the blocked form when a fixed sample of the
    tasks (all of them up to 65536, else tasks i * 2654435761 mod L*K) holds
    each of its distinct experts twice or more on average; only for the
    inputs the blocked form takes (bf16, d % 256 == 0)."""
    ids = to_np(idx).reshape(-1).astype(np.int64)
    M = ids.size
    S = min(M, SAMPLE)
    m = np.arange(S, dtype=np.uint64)
    if M > S:
        m = (m * np.uint64(HASH)) % np.uint64(M)
    distinct = np.unique(ids[m.astype(np.int64)]).size
    blocked_ok = dt == "bf16" and d % 256 == 0
    return int(blocked_ok and S >= 2 * distinct)


CASES = [
    # L, d, Nr, Nc, K, B, dtype, x distribution
    (300, 256, 128, 128, 16, 16, "bf16", "normal"),     # spread out: per-task passes
    (300, 256, 40, 40, 32, 16, "bf16", "normal"),       # small grid: every expert reused
    (512, 256, 64, 64, 32, 16, "bf16", "clustered"),    # clustered: blocked form
    (200, 256, 3, 4, 12, 5, "bf16", "normal"),          # K = N: every token uses all 12
    (130, 512, 37, 29, 50, 7, "bf16", "clustered"),     # ragged blocks
    (256, 128, 32, 32, 16, 16, "bf16", "clustered"),    # d % 256 != 0: per-task only
    (256, 64, 32, 32, 16, 16, "f32", "clustered"),      # fp32: per-task only
    (1, 256, 4, 4, 3, 2, "bf16", "normal"),             # one token
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "L{}_d{}_{}x{}_K{}_B{}_{}_{}".format(*c))
def test_auto_matches_oracle_and_takes_the_expected_form(case):
    L, d, Nr, Nc, K, B, dt, dist = case
    w, inp_cpu = synth.make_case(L, d, Nr, Nc, K, B, dt, x_dist=dist,
                                 seed=zlib.crc32(repr(case).encode()) % 1000)
    inp = {k: v.cuda() for k, v in inp_cpu.items()}
    say(f"auto {w.name} ({dist})")
    br = omni.RoutedBranch(L, d, Nr, Nc, K, B, w.torch_dtype)  # assembly="auto"
    br.y.fill_(-5.0)
    br.forward(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"])
    torch.cuda.synchronize()
    want = expected_choice(br.idx, dt, d)
    assert int(br.chosen.item()) == want
    y_o = O.assemble_token_centric(inp_cpu["x"], inp_cpu["W"], inp_cpu["V"], to_np(br.idx),
                                   to_np(br.gate))
    nrm, mx = check_y(br.y, y_o, RTOL_FP32_ARITH)
    say(f"  chosen={want} y_err norm={nrm:.2e} max={mx:.2e}")
    # the per-task passes on the same routing: bit for bit when they were chosen
    perm, off = omni.omni_schedule(br.idx, w.N, B)
    y_pt = omni.omni_expert_forward(inp["x"], inp["W"], inp["V"], br.idx, br.gate, perm, off, B)
    torch.cuda.synchronize()
    if want == 0:
        assert torch.equal(br.y, y_pt)
    else:
        y_bl = omni.omni_expert_forward_blocked(
            inp["x"], inp["W"], inp["V"], br.idx, br.gate,
            omni.omni_schedule(br.idx, w.N, B, token_order=True, tasks=False)[2])
        torch.cuda.synchronize()
        assert torch.equal(br.y, y_bl)  # the blocked form over the schedule's token order


def test_choice_is_made_per_call():
    """One branch, spread-out then clustered then spread-out routing: the flag
    follows each call's routing and every y matches the oracle."""
    L, d, Nr, Nc, K, B = 512, 256, 128, 128, 16, 16
    br = omni.RoutedBranch(L, d, Nr, Nc, K, B, torch.bfloat16)
    for rep, dist in enumerate(("normal", "clustered", "normal")):
        w, inp_cpu = synth.make_case(L, d, Nr, Nc, K, B, "bf16", x_dist=dist, seed=40 + rep)
        inp = {k: v.cuda() for k, v in inp_cpu.items()}
        say(f"per-call choice: call {rep} ({dist})")
        br.forward(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"])
        torch.cuda.synchronize()
        assert int(br.chosen.item()) == expected_choice(br.idx, "bf16", d)
        assert int(br.chosen.item()) == (1 if dist == "clustered" else 0)
        y_o = O.assemble_token_centric(inp_cpu["x"], inp_cpu["W"], inp_cpu["V"],
                                       to_np(br.idx), to_np(br.gate))
        check_y(br.y, y_o, RTOL_FP32_ARITH)


def test_auto_graph_replays_switch_form_with_the_inputs():
    """A captured forward replays correctly on routing of either kind: the
    choice is data on the device, so one graph serves both."""
    L, d, Nr, Nc, K, B = 512, 256, 128, 128, 16, 16
    wa, a_cpu = synth.make_case(L, d, Nr, Nc, K, B, "bf16", x_dist="clustered", seed=51)
    wb, b_cpu = synth.make_case(L, d, Nr, Nc, K, B, "bf16", x_dist="normal", seed=52)
    a = {k: v.cuda() for k, v in a_cpu.items()}
    b = {k: v.cuda() for k, v in b_cpu.items()}
    want = {}
    for name, inp in (("a", a), ("b", b)):
        ref = omni.RoutedBranch(L, d, Nr, Nc, K, B, torch.bfloat16)
        ref.forward(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"])
        torch.cuda.synchronize()
        want[name] = (ref.y.clone(), int(ref.chosen.item()))
    assert want["a"][1] == 1 and want["b"][1] == 0
    # static input buffers: the graph reads whatever they hold at replay time
    x, Wr, Wc, W, V = (a[k].clone() for k in ("x", "Wr", "Wc", "W", "V"))
    br = omni.RoutedBranch(L, d, Nr, Nc, K, B, torch.bfloat16)
    br.capture(x, Wr, Wc, W, V)
    for rep in range(4):
        name = "a" if rep % 2 == 0 else "b"
        src = a if name == "a" else b
        for dst, k in zip((x, Wr, Wc, W, V), ("x", "Wr", "Wc", "W", "V")):
            dst.copy_(src[k])
        torch.cuda.synchronize()
        say(f"graph replay {rep} ({name})")
        br.replay()
        torch.cuda.synchronize()
        assert int(br.chosen.item()) == want[name][1], rep
        assert torch.equal(br.y, want[name][0]), rep
