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


BLK_BWD_MAX_L = 524288  # tokens the blocked backward's per-token bitmap holds


def _bwd_choice(idx, dt, d, L):
    """The backward's rule: the forward's, within the blocked backward's own
    limit on L."""
    return int(expected_choice(idx, dt, d) and L <= BLK_BWD_MAX_L)


def _assert_same_backward(got, ref, n):
    assert int(got[3].item()) == n and torch.equal(got[2][:n], ref[2][:n])
    for name, a, b in (("dx", got[0], ref[0]), ("dgate", got[1], ref[1]),
                       ("dW", got[4][:n], ref[4][:n]), ("dV", got[5][:n], ref[5][:n])):
        assert torch.equal(a, b), name


@pytest.mark.parametrize("case", CASES, ids=lambda c: "L{}_d{}_{}x{}_K{}_B{}_{}_{}".format(*c))
def test_auto_backward_takes_the_expected_form(case):
    """omni_expert_backward_auto on the oracle's routing: the flag follows the
    forward's rule, every output equals the chosen form's bit for bit, and
    the gradients meet the backward oracle (fp32-arithmetic bound)."""
    from oracle import omni_backward_oracle as BO
    L, d, Nr, Nc, K, B, dt, dist = case
    w, inp_cpu = synth.make_case(L, d, Nr, Nc, K, B, dt, x_dist=dist,
                                 seed=zlib.crc32(repr(case).encode()) % 1000)
    say(f"auto backward {w.name} ({dist})")
    idx_o, _, gate_o, _, _ = O.route(inp_cpu["x"], inp_cpu["Wr"], inp_cpu["Wc"], K)
    inp = {k: v.cuda() for k, v in inp_cpu.items()}
    idx = torch.as_tensor(idx_o, dtype=torch.int32).cuda()
    gate = torch.as_tensor(gate_o, dtype=torch.float32).cuda()
    dy = synth.upstream_grad(w, seed=3).cuda()
    chosen = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    got = omni.omni_expert_backward_auto(inp["x"], inp["W"], inp["V"], idx, gate, dy,
                                         chosen=chosen)
    torch.cuda.synchronize()
    want = _bwd_choice(idx, dt, d, L)
    assert int(chosen.item()) == want
    if want == 0:
        ref = omni.omni_expert_backward(inp["x"], inp["W"], inp["V"], idx, gate, dy)
    else:
        order = omni.omni_schedule(idx, w.N, 1, token_order=True, tasks=False)[2]
        ref = omni.omni_expert_backward_blocked(inp["x"], inp["W"], inp["V"], idx, gate, dy,
                                                order)
    torch.cuda.synchronize()
    n = int(ref[3].item())
    _assert_same_backward(got, ref, n)
    gate_f = to_np(gate).astype(np.float64)
    dy_c = to_np(dy).astype(np.float64)
    terms = BO.task_terms(inp_cpu["x"], inp_cpu["W"], inp_cpu["V"], idx_o, gate_f, dy_c)
    assert np.array_equal(to_np(got[2])[:n], np.unique(idx_o))
    dW_o, dV_o = BO.expert_grads(inp_cpu["x"], dy_c, idx_o, terms, np.unique(idx_o))
    dx_o = BO.input_grad_expert(inp_cpu["W"], idx_o, terms["dh"])
    errs = {"dgate": check_y(got[1], terms["dgate"].reshape(L, K), RTOL_FP32_ARITH),
            "dx": check_y(got[0], dx_o, RTOL_FP32_ARITH),
            "dW": check_y(to_np(got[4])[:n], dW_o, RTOL_FP32_ARITH),
            "dV": check_y(to_np(got[5])[:n], dV_o, RTOL_FP32_ARITH)}
    say(f"  chosen={want} " + " ".join(f"{k}={v[0]:.1e}" for k, v in errs.items()))


def test_auto_backward_one_workspace_serves_both_forms():
    """One workspace, clustered then spread-out then clustered routing: each
    call takes its own form and equals that form's output bit for bit."""
    L, d, Nr, Nc, K, B = 512, 256, 128, 128, 16, 16
    ws = torch.empty((omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_BACKWARD_AUTO, L=L, d=d,
                                                K=K, N=Nr * Nc),), dtype=torch.uint8,
                     device="cuda")
    chosen = torch.empty((1,), dtype=torch.int32, device="cuda")
    for rep, dist in enumerate(("clustered", "normal", "clustered")):
        w, inp_cpu = synth.make_case(L, d, Nr, Nc, K, B, "bf16", x_dist=dist, seed=60 + rep)
        inp = {k: v.cuda() for k, v in inp_cpu.items()}
        br = omni.RoutedBranch(L, d, Nr, Nc, K, B, torch.bfloat16)
        br.forward(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"])
        dy = synth.upstream_grad(w, seed=rep).cuda()
        say(f"auto backward, shared workspace: call {rep} ({dist})")
        got = omni.omni_expert_backward_auto(inp["x"], inp["W"], inp["V"], br.idx, br.gate, dy,
                                             ws=ws, chosen=chosen)
        torch.cuda.synchronize()
        assert int(chosen.item()) == int(br.chosen.item()) == (1 if dist == "clustered" else 0)
        if dist == "clustered":
            order = omni.omni_schedule(br.idx, w.N, 1, token_order=True, tasks=False)[2]
            ref = omni.omni_expert_backward_blocked(inp["x"], inp["W"], inp["V"], br.idx,
                                                    br.gate, dy, order)
        else:
            ref = omni.omni_expert_backward(inp["x"], inp["W"], inp["V"], br.idx, br.gate, dy)
        torch.cuda.synchronize()
        _assert_same_backward(got, ref, int(ref[3].item()))


@pytest.mark.parametrize("name", ["skewed_L16384_N1700416_d2048", synth.HEADLINE,
                                  "L4096_N1048576_d1024", "L4096_N280900_d768"])
def test_auto_backward_full_size(name):
    """The full-size workloads: the skewed one takes the blocked form, the
    spread-out ones the per-task form (at d = 768 the blocked form is not
    offered), each bit for bit."""
    w = synth.WORKLOADS[name]
    say(f"auto backward full-size {name}")
    inp = synth.make_inputs(w, seed=0, device="cuda")
    br = omni.RoutedBranch(w.L, w.d, w.Nr, w.Nc, w.K, w.B, w.torch_dtype)
    br.forward(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"])
    dy = synth.upstream_grad(w, seed=0, device="cuda")
    chosen = torch.empty((1,), dtype=torch.int32, device="cuda")
    got = omni.omni_expert_backward_auto(inp["x"], inp["W"], inp["V"], br.idx, br.gate, dy,
                                         chosen=chosen)
    torch.cuda.synchronize()
    want = _bwd_choice(br.idx, w.dtype, w.d, w.L)
    assert int(chosen.item()) == want == int(br.chosen.item())
    assert want == (1 if name.startswith("skewed") else 0)
    if want:
        order = omni.omni_schedule(br.idx, w.N, 1, token_order=True, tasks=False)[2]
        ref = omni.omni_expert_backward_blocked(inp["x"], inp["W"], inp["V"], br.idx, br.gate,
                                                dy, order)
    else:
        ref = omni.omni_expert_backward(inp["x"], inp["W"], inp["V"], br.idx, br.gate, dy)
    torch.cuda.synchronize()
    _assert_same_backward(got, ref, int(ref[3].item()))
    del inp, br, got, ref
    torch.cuda.empty_cache()


def test_auto_backward_graph_replays_switch_form_with_the_inputs():
    """A captured automatic backward replays correctly on routing of either
    kind: every replay equals the eager call on the same inputs bit for bit,
    with the flag of the form it took."""
    L, d, Nr, Nc, K, B = 512, 256, 128, 128, 16, 16
    N = Nr * Nc
    cases = {}
    for name, dist, seed in (("a", "clustered", 71), ("b", "normal", 72)):
        w, inp_cpu = synth.make_case(L, d, Nr, Nc, K, B, "bf16", x_dist=dist, seed=seed)
        inp = {k: v.cuda() for k, v in inp_cpu.items()}
        br = omni.RoutedBranch(L, d, Nr, Nc, K, B, torch.bfloat16)
        br.forward(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"])
        dy = synth.upstream_grad(w, seed=seed).cuda()
        chosen = torch.empty((1,), dtype=torch.int32, device="cuda")
        ref = omni.omni_expert_backward_auto(inp["x"], inp["W"], inp["V"], br.idx, br.gate, dy,
                                             chosen=chosen)
        torch.cuda.synchronize()
        cases[name] = (inp, br.idx.clone(), br.gate.clone(), dy, ref, int(chosen.item()))
    assert cases["a"][5] == 1 and cases["b"][5] == 0
    # static buffers the graph reads and writes
    inp_a = cases["a"][0]
    x, W, V = (inp_a[k].clone() for k in ("x", "W", "V"))
    idx, gate, dy = cases["a"][1].clone(), cases["a"][2].clone(), cases["a"][3].clone()
    cap = min(N, L * K)
    f32, i32 = torch.float32, torch.int32
    dx = torch.empty((L, d), dtype=f32, device="cuda")
    dgate = torch.empty((L, K), dtype=f32, device="cuda")
    uniq = torch.empty((cap,), dtype=i32, device="cuda")
    n_uniq = torch.empty((1,), dtype=i32, device="cuda")
    dW = torch.empty((cap, d), dtype=f32, device="cuda")
    dV = torch.empty((cap, d), dtype=f32, device="cuda")
    chosen = torch.empty((1,), dtype=i32, device="cuda")
    ws = torch.empty((omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_BACKWARD_AUTO, L=L, d=d,
                                                K=K, N=N),), dtype=torch.uint8, device="cuda")

    def call():
        omni.omni_expert_backward_auto(x, W, V, idx, gate, dy, dx, dgate, uniq, n_uniq, dW, dV,
                                       ws, chosen=chosen)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(4):
        name = "a" if rep % 2 == 0 else "b"
        inp, idx_c, gate_c, dy_c, ref, want = cases[name]
        for dst, src in ((x, inp["x"]), (W, inp["W"]), (V, inp["V"]), (idx, idx_c),
                         (gate, gate_c), (dy, dy_c)):
            dst.copy_(src)
        torch.cuda.synchronize()
        say(f"backward graph replay {rep} ({name})")
        graph.replay()
        torch.cuda.synchronize()
        assert int(chosen.item()) == want, rep
        _assert_same_backward((dx, dgate, uniq, n_uniq, dW, dV), ref, int(ref[3].item()))


def test_auto_backward_above_the_blocked_token_limit_takes_per_task():
    """Past the blocked backward's token limit the automatic backward takes the
    per-task form even where the routing repeats its experts (here the
    forward takes the blocked form), and equals omni_expert_backward bit for
    bit."""
    L, d, Nr, Nc, K, B = BLK_BWD_MAX_L + 64, 256, 8, 8, 4, 8
    w, inp = synth.make_case(L, d, Nr, Nc, K, B, "bf16", seed=81, device="cuda")
    say(f"auto backward past the token limit: {w.name}")
    br = omni.RoutedBranch(L, d, Nr, Nc, K, B, torch.bfloat16)
    br.forward(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"])
    dy = synth.upstream_grad(w, seed=81, device="cuda")
    chosen = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    got = omni.omni_expert_backward_auto(inp["x"], inp["W"], inp["V"], br.idx, br.gate, dy,
                                         chosen=chosen)
    ref = omni.omni_expert_backward(inp["x"], inp["W"], inp["V"], br.idx, br.gate, dy)
    torch.cuda.synchronize()
    assert int(br.chosen.item()) == 1  # the forward's rule alone picks the blocked form
    assert int(chosen.item()) == 0 == _bwd_choice(br.idx, "bf16", d, L)
    _assert_same_backward(got, ref, int(ref[3].item()))
    del inp, br, got, ref, dy
    torch.cuda.empty_cache()
