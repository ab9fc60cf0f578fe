"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small and ragged cases are compared in full; the large workloads run in the
launch configuration the benchmark times (RoutedBranch: one workspace, three
calls on one stream) and are compared on sampled tokens (router, assembly)
and in full (schedule).
"""

import zlib

import numpy as np
import pytest
import torch

from atomic_expert_routing_amd import omni, synth
from oracle import omni_oracle as O
from parity import (DeviceRows, RTOL, RTOL_FP32_ARITH, check_schedule, check_topk, check_y,
                    to_np)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    omni.library()  # fails loudly if the HIP library is missing


def run_branch(inp, w, assembly="expert_centric"):
    """Router, schedule and assembly through RoutedBranch; the per-task passes
    unless another assembly is named (the full-size tests run the default,
    device-chosen one, as the benchmark does)."""
    br = omni.RoutedBranch(w.L, w.d, w.Nr, w.Nc, w.K, w.B, w.torch_dtype, assembly=assembly)
    br.forward(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"])
    torch.cuda.synchronize()
    return br


def full_check(w, inp_cpu):
    """Whole-tensor comparison for a workload small enough for the oracle."""
    inp = {k: v.cuda() for k, v in inp_cpu.items()}
    say(f"case {w.name}")
    br = run_branch(inp, w)
    idx_o, score_o, gate_o, p_r, p_c = O.route(inp_cpu["x"], inp_cpu["Wr"], inp_cpu["Wc"], w.K)
    swaps = check_topk(br.idx, br.score, br.gate, p_r, p_c, w.K)
    check_schedule(br.idx, br.perm, br.group_off, w.N, w.B)
    perm_o, off_o = O.schedule(to_np(br.idx).astype(np.int64), w.N, w.B)
    y_o = O.assemble_expert_centric(inp_cpu["x"], inp_cpu["W"], inp_cpu["V"], to_np(br.idx),
                                    to_np(br.gate), perm_o, off_o)
    nrm, mx = check_y(br.y, y_o, min(RTOL[w.dtype], RTOL_FP32_ARITH))
    say(f"  swaps={swaps} y_err norm={nrm:.2e} max={mx:.2e}")
    return br, swaps


def test_tiny_workload_matches_oracle_and_bruteforce():
    w = synth.WORKLOADS[synth.TINY]
    inp = synth.make_inputs(w, seed=0)
    br, swaps = full_check(w, inp)
    # on this small grid the explicit brute force is affordable too: the same
    # rule must hold against it
    _, _, _, p_r, p_c = O.route(inp["x"], inp["Wr"], inp["Wc"], w.K, method="explicit")
    idx_e, _ = O.topk_explicit(p_r, p_c, w.K)
    same = (np.sort(to_np(br.idx), 1) == np.sort(idx_e, 1)).all(1).mean()
    say(f"  tokens whose id set equals the brute-force set: {same:.3f} (swaps {swaps})")


RAGGED = [
    # L, d, Nr, Nc, K, B, dtype
    (1, 8, 1, 1, 1, 1, "f32"),            # one token, one expert
    (3, 24, 5, 7, 35, 4, "f32"),          # K = N: every grid cell
    (5, 16, 1, 40, 9, 6, "f32"),          # single grid row
    (130, 72, 37, 29, 50, 7, "bf16"),     # K > N_r and K > N_c; ragged tiles
    (257, 136, 130, 200, 64, 100, "bf16"),
    (200, 520, 300, 301, 128, 128, "bf16"),  # d crosses a 512-column chunk
    (300, 64, 50, 50, 37, 3, "f32"),      # several schedule tiles, ragged tail
    (64, 64, 32, 32, 16, 1, "bf16"),      # B = 1: one group per expert
    (64, 64, 32, 32, 16, 5000, "bf16"),   # B >= N: one group
    (40, 64, 600, 700, 512, 512, "bf16"),  # K at its limit
    (20, 64, 4096, 3, 100, 33, "f32"),    # grid side at its limit
    (33, 64, 2900, 70, 256, 64, "bf16"),  # 46 row values per lane
    (17, 48, 700, 1100, 200, 77, "bf16"),  # 11 and 18 values per lane
    (16, 4096, 64, 64, 32, 64, "bf16"),   # d at its bf16 limit
    (24, 2048, 40, 40, 20, 16, "f32"),    # d at its fp32 limit
]


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: "L{}_d{}_{}x{}_K{}_B{}_{}".format(*c))
def test_ragged_and_edge_cases(case):
    L, d, Nr, Nc, K, B, dt = case
    w, inp = synth.make_case(L, d, Nr, Nc, K, B, dt, seed=zlib.crc32(repr(case).encode()) % 1000)
    full_check(w, inp)


def test_schedule_on_oracle_routing_is_bit_exact():
    # the schedule fed with the oracle's own ids (not the GPU router's)
    w = synth.WORKLOADS[synth.TINY]
    inp = synth.make_inputs(w, seed=3)
    idx_o, _, _, _, _ = O.route(inp["x"], inp["Wr"], inp["Wc"], w.K)
    for B in (1, 3, 16, 64, 1000, 2000):
        say(f"schedule oracle ids B={B}")
        idx = torch.as_tensor(idx_o, dtype=torch.int32, device="cuda")
        perm, off = omni.omni_schedule(idx, w.N, B)
        torch.cuda.synchronize()
        check_schedule(idx_o, perm, off, w.N, B)


SCHED_SIZES = [
    (3000, 100, 50000, 7, None),          # 300,000 tasks, 2 x 256 per tile, ragged tail
    (8192, 128, 1700416, 128, None),      # 2^20 tasks: 4 x 256 per tile
    (16384, 128, 280900, 64, None),       # 2^21 tasks: 8 x 256 per tile
    (16384, 200, 1048576, 128, None),     # 3,276,800 tasks: 16 x 256 per tile, ragged
    (16384, 128, 1700416, 128, 3000),     # 2^21 tasks on 3000 experts: few, crowded groups
    (4096, 64, 1700416, 16, None),        # 106,276 groups: three radix passes
    (16384, 520, 1048576, 128, None),     # 8,519,680 tasks: 2080 tiles of 16 x 256
]


@pytest.mark.parametrize("case", SCHED_SIZES, ids=lambda c: "L{}_K{}_N{}_B{}_ids{}".format(*c))
def test_schedule_tile_sizes_are_bit_exact(case):
    """The radix passes size their tiles by the task count (2 to 16 rounds of
    256 tasks, past 1024 tiles at the most); perm and group_off must match the
    oracle bit for bit at each, with one to three radix passes."""
    L, K, N, B, span = case
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    idx_np = rng.integers(0, span or N, size=(L, K), dtype=np.int64)
    say(f"schedule sizes {case}")
    idx = torch.as_tensor(idx_np, dtype=torch.int32, device="cuda")
    perm, off = omni.omni_schedule(idx, N, B)
    torch.cuda.synchronize()
    check_schedule(idx_np, perm, off, N, B)


def test_expert_forward_on_oracle_routing():
    w = synth.WORKLOADS[synth.TINY]
    inp = synth.make_inputs(w, seed=4)
    out = O.routed_forward(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"], w.K, w.B)
    g = {k: v.cuda() for k, v in inp.items()}
    idx = torch.as_tensor(out["idx"], dtype=torch.int32, device="cuda")
    gate = torch.as_tensor(out["gate"], dtype=torch.float32, device="cuda")
    perm = torch.as_tensor(out["perm"], dtype=torch.int32, device="cuda")
    off = torch.as_tensor(out["group_off"], dtype=torch.int32, device="cuda")
    say("expert forward on oracle routing")
    y = omni.omni_expert_forward(g["x"], g["W"], g["V"], idx, gate, perm, off, w.B)
    torch.cuda.synchronize()
    # the gate went through fp32 on its way in: compare with the oracle's y
    # for the same fp32 gate values
    y_o = O.assemble_token_centric(inp["x"], inp["W"], inp["V"], out["idx"], to_np(gate))
    check_y(y, y_o, RTOL["f32"])


@pytest.mark.parametrize("case", [(64, 64, 32, 32, 16, 16, "f32"), (130, 72, 37, 29, 50, 7, "bf16"),
                                  (200, 520, 300, 301, 128, 128, "bf16"),
                                  (16, 4096, 64, 64, 32, 64, "bf16"), (24, 2048, 40, 40, 20, 16, "f32"),
                                  (40, 64, 600, 700, 512, 512, "bf16")],
                         ids=lambda c: "L{}_d{}_{}x{}_K{}_B{}_{}".format(*c))
def test_token_centric_baseline_matches_oracle(case):
    L, d, Nr, Nc, K, B, dt = case
    w, inp_cpu = synth.make_case(L, d, Nr, Nc, K, B, dt, seed=zlib.crc32(repr(case).encode()) % 1000)
    inp = {k: v.cuda() for k, v in inp_cpu.items()}
    say(f"token-centric {w.name}")
    br = run_branch(inp, w)
    y_tc = omni.omni_expert_forward_token_centric(inp["x"], inp["W"], inp["V"], br.idx, br.gate)
    torch.cuda.synchronize()
    y_o = O.assemble_token_centric(inp_cpu["x"], inp_cpu["W"], inp_cpu["V"], to_np(br.idx),
                                   to_np(br.gate))
    check_y(y_tc, y_o, RTOL_FP32_ARITH)
    # same k-order sum of the V pass: equal to the expert-centric path up to
    # the rounding of the activations' dot products
    check_y(y_tc, to_np(br.y), RTOL_FP32_ARITH)


def check_token_order(inp, br, w):
    """The schedule's token order equals the oracle's (bit-exact), and the
    output pass that follows it reproduces br.y bit for bit: each token's
    sum is taken in k order whatever order the tokens run in."""
    perm, off, order = omni.omni_schedule(br.idx, w.N, w.B, token_order=True)
    y = omni.omni_expert_forward(inp["x"], inp["W"], inp["V"], br.idx, br.gate, perm, off, w.B,
                                 token_order=order)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(order), O.token_order(to_np(br.idx), w.B))
    assert torch.equal(perm, br.perm) and torch.equal(off, br.group_off)
    assert torch.equal(y, br.y)


@pytest.mark.parametrize("case", [RAGGED[0], RAGGED[1], RAGGED[3], RAGGED[6], RAGGED[7],
                                  RAGGED[9], (1001, 64, 40, 40, 8, 2, "bf16")],
                         ids=lambda c: "L{}_d{}_{}x{}_K{}_B{}_{}".format(*c))
def test_token_ordered_output_pass(case):
    # L from 1 to 1001 (not a multiple of 8: slots past L in the last XCD's
    # eighth), B = 1 and B > N
    L, d, Nr, Nc, K, B, dt = case
    w, inp_cpu = synth.make_case(L, d, Nr, Nc, K, B, dt, seed=zlib.crc32(repr(case).encode()) % 1000)
    inp = {k: v.cuda() for k, v in inp_cpu.items()}
    say(f"token order {w.name}")
    br = run_branch(inp, w)
    check_token_order(inp, br, w)
    # through RoutedBranch, run twice (the second over a stale y)
    bo = omni.RoutedBranch(w.L, w.d, w.Nr, w.Nc, w.K, w.B, w.torch_dtype, token_order=True,
                           assembly="expert_centric")
    for _ in range(2):
        bo.forward(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"])
        torch.cuda.synchronize()
        assert torch.equal(bo.y, br.y)
        bo.y.fill_(7.0)


TIE_CASES = [
    (40, 50, 16, "bf16"),     # candidates in one register per lane
    (8, 8, 20, "f32"),        # K > N_c: the top K spans three rows
    (1304, 1304, 256, "bf16"),  # 24 candidate registers per lane
    (600, 700, 512, "bf16"),  # more than 24*64 candidates: LDS select
    (2900, 70, 256, "bf16"),  # grid side above 24*64: LDS select
]


@pytest.mark.parametrize("case", TIE_CASES, ids=lambda c: "{}x{}_K{}_{}".format(*c))
def test_exact_ties_take_the_smallest_ids(case):
    """x = 0 makes every logit 0, so every cell scores -log N_r - log N_c:
    under (S desc, n asc) the top K is n = 0 .. K-1 in that order, with
    gates 1/K (a closed form, independent of the oracle)."""
    Nr, Nc, K, dtype = case
    L, d = 5, 64
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(3)
    x = torch.zeros((L, d), dtype=tdt, device="cuda")
    Wr = (torch.randn((Nr, d), generator=g) / d ** 0.5).to(tdt).cuda()
    Wc = (torch.randn((Nc, d), generator=g) / d ** 0.5).to(tdt).cuda()
    say(f"ties {case}")
    idx, score, gate = omni.omni_router(x, Wr, Wc, K)
    torch.cuda.synchronize()
    want = torch.arange(K, dtype=torch.int32).expand(L, K)
    assert torch.equal(idx.cpu(), want)
    s_star = -float(np.log(Nr)) - float(np.log(Nc))
    assert torch.allclose(score.cpu(), torch.full((L, K), s_star), atol=1e-5, rtol=0)
    assert torch.allclose(gate.cpu(), torch.full((L, K), 1.0 / K), atol=1e-7, rtol=1e-5)


def test_repeat_runs_are_bitwise_identical():
    w = synth.WORKLOADS[synth.TINY]
    inp = {k: v.cuda() for k, v in synth.make_inputs(w, seed=5).items()}
    say("determinism")
    ref = run_branch(inp, w)
    snap = [t.clone() for t in (ref.idx, ref.score, ref.gate, ref.perm, ref.group_off, ref.y)]
    for _ in range(10):
        ref.forward(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"])
    torch.cuda.synchronize()
    for a, b in zip(snap, (ref.idx, ref.score, ref.gate, ref.perm, ref.group_off, ref.y)):
        assert torch.equal(a, b)


def test_y_is_overwritten_not_accumulated():
    w = synth.WORKLOADS[synth.TINY]
    inp = {k: v.cuda() for k, v in synth.make_inputs(w, seed=6).items()}
    say("y overwrite")
    br = run_branch(inp, w)
    y1 = br.y.clone()
    br.y.fill_(123.0)
    br.expert_forward(inp["x"], inp["W"], inp["V"])
    torch.cuda.synchronize()
    assert torch.equal(br.y, y1)


# ------------------------------------------------------------ full-size workloads

LARGE = ["L4096_N280900_d768", "L4096_N1048576_d1024", synth.HEADLINE,
         "skewed_L16384_N1700416_d2048"]


def class_sample(L, per_class=8, seed=7):
    """Tokens 0 and L-1 plus per_class random tokens of each class t % 8 (the
    activation pass splits its work by that class across the XCDs)."""
    rs = np.random.Generator(np.random.PCG64(seed))
    picks = [0, L - 1]
    for c in range(8):
        members = np.arange(c, L, 8)
        picks.extend(rs.choice(members, min(per_class, len(members)), replace=False))
    return np.unique(np.asarray(picks, np.int64))


def check_rows(y, y_ref, rtol):
    """Row by row: max |y - y_ref| <= rtol * max |y_ref| within each row."""
    diff = (y - y_ref).abs().amax(dim=1)
    scale = y_ref.abs().amax(dim=1).clamp_min(1e-30)
    worst = (diff / scale).max().item()
    assert worst <= rtol, worst
    return worst


@pytest.mark.parametrize("name", LARGE)
def test_full_size_workload_sampled(name):
    w = synth.WORKLOADS[name]
    say(f"full-size {name}: generating inputs")
    inp = synth.make_inputs(w, seed=0, device="cuda")
    say(f"full-size {name}: routed forward (default assembly, as the benchmark runs it)")
    br = run_branch(inp, w, assembly="auto")
    chosen = int(br.chosen.item())
    # the device picks the blocked form for the clustered workload only
    assert chosen == (1 if w.x_dist == "clustered" else 0), chosen
    # schedule of the same ids (omni_schedule): whole arrays, bit-exact
    br.perm, br.group_off = omni.omni_schedule(br.idx, w.N, w.B)
    torch.cuda.synchronize()
    check_schedule(br.idx, br.perm, br.group_off, w.N, w.B)
    # router and assembly: 8 sampled tokens of every class t % 8, plus the ends
    toks = class_sample(w.L)
    xs = to_np(inp["x"][torch.as_tensor(toks, device="cuda")])
    _, _, _, p_r, p_c = O.route(xs, inp["Wr"], inp["Wc"], w.K)
    idx = to_np(br.idx)[toks]
    swaps = check_topk(idx, to_np(br.score)[toks], to_np(br.gate)[toks], p_r, p_c, w.K)
    y_o = O.assemble_token_centric(xs, DeviceRows(inp["W"]), DeviceRows(inp["V"]),
                                   idx, to_np(br.gate)[toks])
    nrm, mx = check_y(to_np(br.y)[toks], y_o, min(RTOL[w.dtype], RTOL_FP32_ARITH))
    say(f"  chosen={chosen} swaps={swaps} over {len(toks)} tokens; y_err norm={nrm:.2e} "
        f"max={mx:.2e}")
    # the per-task passes on the same routing: the sampled tokens against the
    # oracle, and the whole y against the token-centric kernel row by row
    y_pt = omni.omni_expert_forward(inp["x"], inp["W"], inp["V"], br.idx, br.gate, br.perm,
                                    br.group_off, w.B)
    torch.cuda.synchronize()
    check_y(to_np(y_pt)[toks], y_o, min(RTOL[w.dtype], RTOL_FP32_ARITH))
    y_tc = omni.omni_expert_forward_token_centric(inp["x"], inp["W"], inp["V"], br.idx, br.gate)
    torch.cuda.synchronize()
    dy = (y_tc - y_pt).norm() / y_pt.norm()
    assert dy.item() <= RTOL_FP32_ARITH, dy.item()
    worst = check_rows(y_tc, y_pt, RTOL_FP32_ARITH)
    if chosen:
        check_rows(br.y, y_pt, RTOL_FP32_ARITH)
    else:
        assert torch.equal(br.y, y_pt)  # the same kernels ran
    say(f"  token-centric vs per-task: norm {dy.item():.2e}, worst row {worst:.2e}")
    # token-ordered output pass: the order bit-exact, y bitwise unchanged
    say(f"full-size {name}: token order")
    br.y.copy_(y_pt)
    check_token_order(inp, br, w)
    del inp, br
    torch.cuda.empty_cache()
