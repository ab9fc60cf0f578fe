"""GPU parity of the blocked assembly (omni_expert_forward_blocked) through
the C ABI: against the oracle's assembly of the same routing, against the
per-task assembly, and at the full sizes of both large-K workloads.

The W-side product is exact bf16 x bf16 in fp32; the activations enter the
V-side product as hi + lo bf16 terms (relative error below 2^-16 per term);
all sums are fp32.  So y is held to the same fp32-arithmetic bound as the
per-task path.
"""

import zlib

import numpy as np
import pytest
import torch

from atomic_expert_routing_amd import omni, synth
from oracle import omni_oracle as O
from parity import DeviceRows, RTOL_FP32_ARITH, check_y, to_np

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    omni.library()


def routed(inp, w):
    """Router + schedule with the token order, then the per-task assembly."""
    br = omni.RoutedBranch(w.L, w.d, w.Nr, w.Nc, w.K, w.B, w.torch_dtype, token_order=True,
                           assembly="expert_centric")
    br.forward(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"])
    torch.cuda.synchronize()
    return br


CASES = [
    # L, d, Nr, Nc, K, B
    (64, 256, 32, 32, 16, 16),      # one block
    (130, 256, 37, 29, 50, 7),      # ragged last block, unions over several column tiles
    (1, 256, 4, 4, 3, 2),           # one token
    (200, 512, 20, 20, 1, 4),       # K = 1
    (65, 256, 30, 30, 512, 64),     # K at its limit: 32768 ids sorted per block
    (96, 2048, 40, 40, 128, 128),   # d of the large workloads
    (70, 256, 3, 4, 12, 5),         # K = N: every block uses all 12 experts
    (300, 768, 64, 64, 64, 64),     # several blocks, unions of a few thousand
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "L{}_d{}_{}x{}_K{}_B{}".format(*c))
def test_blocked_matches_oracle(case):
    L, d, Nr, Nc, K, B = case
    w, inp_cpu = synth.make_case(L, d, Nr, Nc, K, B, "bf16",
                                 seed=zlib.crc32(repr(case).encode()) % 1000)
    inp = {k: v.cuda() for k, v in inp_cpu.items()}
    say(f"blocked {w.name}")
    br = routed(inp, w)
    for order in (br.token_order, torch.arange(L, dtype=torch.int32, device="cuda")):
        y = omni.omni_expert_forward_blocked(inp["x"], inp["W"], inp["V"], br.idx, br.gate, order)
        torch.cuda.synchronize()
        y_o = O.assemble_token_centric(inp_cpu["x"], inp_cpu["W"], inp_cpu["V"], to_np(br.idx),
                                       to_np(br.gate))
        nrm, mx = check_y(y, y_o, RTOL_FP32_ARITH)
        say(f"  y_err norm={nrm:.2e} max={mx:.2e}")
        # the per-task assembly on the same routing
        d_rel = ((y - br.y).norm() / br.y.norm()).item()
        assert d_rel <= RTOL_FP32_ARITH, d_rel


def test_blocked_is_deterministic_and_overwrites_y():
    w, inp_cpu = synth.make_case(300, 512, 48, 48, 64, 8, "bf16", seed=5)
    inp = {k: v.cuda() for k, v in inp_cpu.items()}
    say("blocked determinism")
    br = routed(inp, w)
    bb = omni.RoutedBranch(w.L, w.d, w.Nr, w.Nc, w.K, w.B, w.torch_dtype, assembly="blocked")
    bb.forward(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"])
    torch.cuda.synchronize()
    first = bb.y.clone()
    assert torch.equal(bb.idx, br.idx) and torch.equal(bb.token_order, br.token_order)
    for _ in range(3):
        bb.y.fill_(7.0)
        bb.forward(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"])
        torch.cuda.synchronize()
        assert torch.equal(bb.y, first)


def test_blocked_skips_order_entries_outside_range():
    # entries outside [0, L) are skipped by the kernels: only the rows of the
    # tokens that do appear are written
    w, inp_cpu = synth.make_case(100, 256, 16, 16, 8, 4, "bf16", seed=9)
    inp = {k: v.cuda() for k, v in inp_cpu.items()}
    say("blocked with a partial order")
    br = routed(inp, w)
    order = br.token_order.clone()
    dropped = order[[3, 70]].clone()
    order[3] = -1
    order[70] = 1000
    y = torch.full((w.L, w.d), 5.0, device="cuda")
    omni.omni_expert_forward_blocked(inp["x"], inp["W"], inp["V"], br.idx, br.gate, order, y)
    torch.cuda.synchronize()
    keep = torch.ones(w.L, dtype=torch.bool, device="cuda")
    keep[dropped.long()] = False
    assert torch.all(y[~keep] == 5.0)
    d_rel = ((y[keep] - br.y[keep]).norm() / br.y[keep].norm()).item()
    assert d_rel <= RTOL_FP32_ARITH


@pytest.mark.parametrize("name", ["skewed_L16384_N1700416_d2048", synth.HEADLINE])
def test_blocked_full_size(name):
    """Full size, in the configuration RoutedBranch(assembly="blocked") runs:
    whole y against the per-task assembly, sampled tokens against the oracle."""
    w = synth.WORKLOADS[name]
    say(f"blocked full-size {name}")
    inp = synth.make_inputs(w, seed=0, device="cuda")
    br = routed(inp, w)
    bb = omni.RoutedBranch(w.L, w.d, w.Nr, w.Nc, w.K, w.B, w.torch_dtype, assembly="blocked")
    bb.forward(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"])
    torch.cuda.synchronize()
    assert torch.equal(bb.idx, br.idx)
    d_rel = ((bb.y - br.y).norm() / br.y.norm()).item()
    say(f"  ||y_blocked - y_per_task|| / ||y|| = {d_rel:.2e}")
    assert d_rel <= RTOL_FP32_ARITH
    rs = np.random.Generator(np.random.PCG64(3))
    toks = np.unique(np.concatenate([[0, w.L - 1], rs.choice(w.L, 24, replace=False)]))
    xs = to_np(inp["x"][torch.as_tensor(toks, device="cuda")])
    y_o = O.assemble_token_centric(xs, DeviceRows(inp["W"]), DeviceRows(inp["V"]),
                                   to_np(br.idx)[toks], to_np(br.gate)[toks])
    nrm, mx = check_y(to_np(bb.y)[toks], y_o, RTOL_FP32_ARITH)
    say(f"  sampled y_err norm={nrm:.2e} max={mx:.2e}")
    del inp, br, bb
    torch.cuda.empty_cache()
