"""GPU parity of the backward pass (omni_expert_backward, omni_router_backward)
against the backward oracle, through the C ABI.

The routing (idx, gate) comes from the forward oracle, so the backward is
judged on identical routing.  Every product and sum runs in fp32 on the GPU
(bf16 inputs are widened exactly; the router's logit gradients are split
into two bf16 terms carrying about 16 significant bits), so all gradients are
held to the fp32-arithmetic bound, norm-wise as y is in the forward tests.
The list of used experts is compared exactly.
"""

import numpy as np
import pytest
import torch

from atomic_expert_routing_amd import omni, synth
from oracle import omni_backward_oracle as BO
from oracle import omni_oracle as O
from parity import DeviceRows, RTOL_FP32_ARITH, check_y, to_np

pytestmark = pytest.mark.gpu

# The router's logit gradients enter the MFMA products as ds = hi + lo, two
# bf16 roundings that leave a relative error of at most 2^-17 per element;
# with fp32 accumulation on top, 4 * 2^-17 bounds the products' error.
RTOL_ROUTER = 3e-5


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    omni.library()


def gpu_backward(inp, idx, gate, dy, grad_dtype=torch.float32):
    out = omni.omni_expert_backward(inp["x"], inp["W"], inp["V"], idx, gate, dy,
                                    grad_dtype=grad_dtype)
    dx, dgate, uniq, n_uniq, dW, dV = out
    dx_total = dx.clone()
    _, dWr, dWc = omni.omni_router_backward(inp["x"], inp["Wr"], inp["Wc"], idx, gate, dgate,
                                            dx_total)
    torch.cuda.synchronize()
    return dict(dx=dx, dgate=dgate, uniq=uniq, n=int(n_uniq.item()), dW=dW, dV=dV,
                dx_total=dx_total, dWr=dWr, dWc=dWc)


CASES = [
    (64, 64, 32, 32, 16, "f32"),
    (130, 72, 37, 29, 50, "bf16"),   # ragged L, d, N_r + N_c not a multiple of 64
    (33, 8, 5, 7, 3, "f32"),         # smallest d
    (64, 2048, 40, 40, 128, "bf16"),
    (200, 256, 64, 64, 32, "bf16"),
    (96, 4096, 16, 16, 8, "bf16"),   # largest bf16 d
    (50, 2048, 16, 16, 100, "f32"),  # largest fp32 d
    (40, 64, 8, 8, 64, "bf16"),      # K = N: every expert used by every token
    (70, 128, 20, 20, 1, "bf16"),    # K = 1: gate 1, no router gradient
    # fewer tokens than XCD classes (the row pass deals the used experts out
    # by t % 8 of their first token: empty classes, then uneven ones)
    (1, 128, 8, 8, 32, "f32"),
    (3, 64, 8, 8, 16, "bf16"),
    (9, 256, 12, 12, 48, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "L{}_d{}_{}x{}_K{}_{}".format(*c))
def test_backward_matches_oracle(case):
    L, d, Nr, Nc, K, dtype = case
    say(f"backward case {case}")
    w, inp_cpu = synth.make_case(L, d, Nr, Nc, K, 8, dtype, seed=3)
    idx_o, _, gate_o, _, _ = O.route(inp_cpu["x"], inp_cpu["Wr"], inp_cpu["Wc"], K)
    inp = {k: v.cuda() for k, v in inp_cpu.items()}
    idx = torch.as_tensor(idx_o, dtype=torch.int32).cuda()
    gate = torch.as_tensor(gate_o, dtype=torch.float32).cuda()
    dy = synth.upstream_grad(w, seed=3).cuda()
    g = gpu_backward(inp, idx, gate, dy)

    gate_f = to_np(gate).astype(np.float64)  # the fp32 gates the GPU used
    dy_c = to_np(dy).astype(np.float64)
    terms = BO.task_terms(inp_cpu["x"], inp_cpu["W"], inp_cpu["V"], idx_o, gate_f, dy_c)
    uniq_o = np.unique(idx_o)
    assert g["n"] == uniq_o.size
    np.testing.assert_array_equal(to_np(g["uniq"])[: g["n"]], uniq_o)
    dW_o, dV_o = BO.expert_grads(inp_cpu["x"], dy_c, idx_o, terms, uniq_o)
    dx_o = BO.input_grad_expert(inp_cpu["W"], idx_o, terms["dh"])
    errs = {}
    errs["dgate"] = check_y(g["dgate"], terms["dgate"].reshape(L, K), RTOL_FP32_ARITH)
    errs["dx_expert"] = check_y(g["dx"], dx_o, RTOL_FP32_ARITH)
    errs["dW"] = check_y(to_np(g["dW"])[: g["n"]], dW_o, RTOL_FP32_ARITH)
    errs["dV"] = check_y(to_np(g["dV"])[: g["n"]], dV_o, RTOL_FP32_ARITH)
    # router on the GPU's own dgate
    dgate_g = to_np(g["dgate"]).astype(np.float64)
    dWr_o, dWc_o, dxr_o, _ = BO.router_backward(inp_cpu["x"], inp_cpu["Wr"], inp_cpu["Wc"], idx_o,
                                                gate_f, dgate_g)
    if K == 1:
        assert torch.count_nonzero(g["dWr"]).item() == 0
        assert torch.count_nonzero(g["dWc"]).item() == 0
        assert torch.equal(g["dx_total"], g["dx"])
    else:
        errs["dWr"] = check_y(g["dWr"], dWr_o, RTOL_ROUTER)
        errs["dWc"] = check_y(g["dWc"], dWc_o, RTOL_ROUTER)
        errs["dx"] = check_y(g["dx_total"], to_np(g["dx"]).astype(np.float64) + dxr_o, RTOL_ROUTER)
    say("  " + " ".join(f"{k}={v[0]:.1e}" for k, v in errs.items()))
    # bf16 gradient rows: the same fp32 sums rounded to nearest even
    b = gpu_backward(inp, idx, gate, dy, grad_dtype=torch.bfloat16)
    n = g["n"]
    assert b["n"] == n and b["dW"].dtype == torch.bfloat16
    assert torch.equal(b["dW"][:n], g["dW"][:n].to(torch.bfloat16))
    assert torch.equal(b["dV"][:n], g["dV"][:n].to(torch.bfloat16))
    assert torch.equal(b["dx"], g["dx"]) and torch.equal(b["dgate"], g["dgate"])


def test_backward_is_deterministic():
    w, inp_cpu = synth.make_case(300, 512, 48, 48, 64, 8, "bf16", seed=5)
    idx_o, _, gate_o, _, _ = O.route(inp_cpu["x"], inp_cpu["Wr"], inp_cpu["Wc"], w.K)
    inp = {k: v.cuda() for k, v in inp_cpu.items()}
    idx = torch.as_tensor(idx_o, dtype=torch.int32).cuda()
    gate = torch.as_tensor(gate_o, dtype=torch.float32).cuda()
    dy = synth.upstream_grad(w, seed=5).cuda()
    a = gpu_backward(inp, idx, gate, dy)
    b = gpu_backward(inp, idx, gate, dy)
    n = a["n"]
    assert n == b["n"]
    for k in ("dx", "dgate", "dx_total", "dWr", "dWc"):
        assert torch.equal(a[k], b[k]), k
    for k in ("uniq", "dW", "dV"):
        assert torch.equal(a[k][:n], b[k][:n]), k


@pytest.mark.parametrize("name", [synth.HEADLINE, "skewed_L16384_N1700416_d2048",
                                  "L4096_N1048576_d1024", "L4096_N280900_d768"])
def test_full_size_backward_sampled(name):
    """The 4096-token shapes at 1.7M, 1M and 280,900 experts and the skewed
    16384-token one (K = 256, tasks piled onto few experts): used-expert
    list in full, dx and
    dgate on sampled tokens, dW and dV on sampled experts (every task of
    each; fewer experts on the skewed routing, whose experts carry hundreds
    of tasks), dW_r and dW_c in full (the oracle's dense products over all
    tokens)."""
    w = synth.WORKLOADS[name]
    n_exp = 16 if w.x_dist == "normal" else 6
    say(f"full-size backward {name}: inputs and forward routing")
    inp = synth.make_inputs(w, seed=0, device="cuda")
    br = omni.RoutedBranch(w.L, w.d, w.Nr, w.Nc, w.K, w.B, w.torch_dtype)
    br.forward(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"])
    dy = synth.upstream_grad(w, seed=0, device="cuda")
    say("  backward")
    g = gpu_backward(inp, br.idx, br.gate, dy)
    idx = to_np(br.idx).astype(np.int64)
    gate_f = to_np(br.gate).astype(np.float64)
    uniq_o = np.unique(idx)
    assert g["n"] == uniq_o.size
    np.testing.assert_array_equal(to_np(g["uniq"][: g["n"]]), uniq_o)
    rs = np.random.Generator(np.random.PCG64(11))
    Wd, Vd = DeviceRows(inp["W"]), DeviceRows(inp["V"])
    # sampled tokens: dgate and the expert part of dx
    toks = np.unique(np.concatenate([[0, w.L - 1], rs.choice(w.L, 24, replace=False)]))
    xs = to_np(inp["x"][torch.as_tensor(toks, device="cuda")]).astype(np.float64)
    dys = to_np(dy[torch.as_tensor(toks, device="cuda")]).astype(np.float64)
    sub_idx = idx[toks]
    terms = BO.task_terms(xs, Wd, Vd, sub_idx, gate_f[toks], dys)
    check_y(to_np(g["dgate"])[toks], terms["dgate"].reshape(len(toks), w.K), RTOL_FP32_ARITH)
    dx_o = BO.input_grad_expert(Wd, sub_idx, terms["dh"])
    check_y(to_np(g["dx"])[toks], dx_o, RTOL_FP32_ARITH)
    # sampled experts (first, last and spread): every task of each
    pick = np.unique(np.concatenate([[0, g["n"] - 1], rs.choice(g["n"], n_exp, replace=False)]))
    ex = uniq_o[pick]
    m_all = np.nonzero(np.isin(idx.reshape(-1), ex))[0]
    say(f"  {len(ex)} sampled experts, {m_all.size} tasks")
    t_all = np.unique(m_all // w.K)
    x_rows = to_np(inp["x"][torch.as_tensor(t_all, device="cuda")]).astype(np.float64)
    dy_rows = to_np(dy[torch.as_tensor(t_all, device="cuda")]).astype(np.float64)
    # re-index the tasks onto the gathered token rows
    tpos = {int(t): i for i, t in enumerate(t_all)}
    local_idx = np.zeros((len(t_all), w.K), np.int64)
    local_gate = np.zeros((len(t_all), w.K))
    for t in t_all:
        local_idx[tpos[int(t)]] = idx[t]
        local_gate[tpos[int(t)]] = gate_f[t]
    lm = np.array([tpos[int(m // w.K)] * w.K + m % w.K for m in m_all])
    terms_e = BO.task_terms(x_rows, Wd, Vd, local_idx, local_gate, dy_rows, m=lm)
    dW_o, dV_o = BO.expert_grads(x_rows, dy_rows, local_idx, terms_e, ex)
    check_y(to_np(g["dW"][torch.as_tensor(pick, device="cuda")]), dW_o, RTOL_FP32_ARITH)
    check_y(to_np(g["dV"][torch.as_tensor(pick, device="cuda")]), dV_o, RTOL_FP32_ARITH)
    # router gradients in full, on the GPU's dgate
    say("  router gradients (oracle over all tokens)")
    x_all = to_np(inp["x"]).astype(np.float64)
    dWr_o, dWc_o, _, dS = BO.router_backward(x_all, inp["Wr"], inp["Wc"], idx, gate_f,
                                             to_np(g["dgate"]).astype(np.float64))
    nr = check_y(g["dWr"], dWr_o, RTOL_ROUTER)
    nc = check_y(g["dWc"], dWc_o, RTOL_ROUTER)
    say(f"  dWr err {nr[0]:.1e} dWc err {nc[0]:.1e}")
    del inp, br, g
    torch.cuda.empty_cache()


BLOCKED_CASES = [
    (64, 256, 32, 32, 16),
    (130, 256, 37, 29, 50),   # ragged last block, unions over several column tiles
    (1, 256, 4, 4, 3),        # one token
    (200, 512, 20, 20, 1),    # K = 1
    (65, 256, 30, 30, 512),   # K at its limit
    (96, 2048, 40, 40, 128),
]


@pytest.mark.parametrize("case", BLOCKED_CASES, ids=lambda c: "L{}_d{}_{}x{}_K{}".format(*c))
def test_blocked_backward_matches_oracle(case):
    """omni_expert_backward_blocked on the oracle's routing: against the
    backward oracle (fp32-arithmetic bound) and, bit for bit where the two
    share the summation (uniq, n_uniq), against omni_expert_backward."""
    L, d, Nr, Nc, K = case
    say(f"blocked backward case {case}")
    w, inp_cpu = synth.make_case(L, d, Nr, Nc, K, 8, "bf16", seed=4)
    idx_o, _, gate_o, _, _ = O.route(inp_cpu["x"], inp_cpu["Wr"], inp_cpu["Wc"], K)
    inp = {k: v.cuda() for k, v in inp_cpu.items()}
    idx = torch.as_tensor(idx_o, dtype=torch.int32).cuda()
    gate = torch.as_tensor(gate_o, dtype=torch.float32).cuda()
    dy = synth.upstream_grad(w, seed=4).cuda()
    _, _, order = omni.omni_schedule(idx, w.N, w.B, token_order=True)
    dx, dgate, uniq, n_uniq, dW, dV = omni.omni_expert_backward_blocked(
        inp["x"], inp["W"], inp["V"], idx, gate, dy, order)
    ref = omni.omni_expert_backward(inp["x"], inp["W"], inp["V"], idx, gate, dy)
    torch.cuda.synchronize()
    n = int(n_uniq.item())
    assert n == int(ref[3].item())
    assert torch.equal(uniq[:n], ref[2][:n])
    gate_f = to_np(gate).astype(np.float64)
    dy_c = to_np(dy).astype(np.float64)
    terms = BO.task_terms(inp_cpu["x"], inp_cpu["W"], inp_cpu["V"], idx_o, gate_f, dy_c)
    uniq_o = np.unique(idx_o)
    dW_o, dV_o = BO.expert_grads(inp_cpu["x"], dy_c, idx_o, terms, uniq_o)
    dx_o = BO.input_grad_expert(inp_cpu["W"], idx_o, terms["dh"])
    errs = {"dgate": check_y(dgate, terms["dgate"].reshape(L, K), RTOL_FP32_ARITH),
            "dx": check_y(dx, dx_o, RTOL_FP32_ARITH),
            "dW": check_y(to_np(dW)[:n], dW_o, RTOL_FP32_ARITH),
            "dV": check_y(to_np(dV)[:n], dV_o, RTOL_FP32_ARITH)}
    say("  " + " ".join(f"{k}={v[0]:.1e}" for k, v in errs.items()))
    # deterministic: a second call reproduces every output bit for bit
    again = omni.omni_expert_backward_blocked(inp["x"], inp["W"], inp["V"], idx, gate, dy, order)
    torch.cuda.synchronize()
    for a, b in zip((dx, dgate, dW[:n], dV[:n]), (again[0], again[1], again[4][:n], again[5][:n])):
        assert torch.equal(a, b)
    # bf16 gradient rows: the same fp32 sums rounded to nearest even
    b16 = omni.omni_expert_backward_blocked(inp["x"], inp["W"], inp["V"], idx, gate, dy, order,
                                            grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert b16[4].dtype == torch.bfloat16 and int(b16[3].item()) == n
    assert torch.equal(b16[4][:n], dW[:n].to(torch.bfloat16))
    assert torch.equal(b16[5][:n], dV[:n].to(torch.bfloat16))
    assert torch.equal(b16[0], dx) and torch.equal(b16[1], dgate)


@pytest.mark.parametrize("name", ["skewed_L16384_N1700416_d2048", synth.HEADLINE])
def test_blocked_backward_full_size(name):
    """Both full-size workloads: every output of the blocked backward against
    the per-task backward on the same routing (norm-wise, fp32 bound)."""
    w = synth.WORKLOADS[name]
    say(f"blocked backward full-size {name}")
    inp = synth.make_inputs(w, seed=0, device="cuda")
    br = omni.RoutedBranch(w.L, w.d, w.Nr, w.Nc, w.K, w.B, w.torch_dtype, token_order=True,
                           assembly="expert_centric")
    br.forward(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"])
    dy = synth.upstream_grad(w, seed=0, device="cuda")
    ref = omni.omni_expert_backward(inp["x"], inp["W"], inp["V"], br.idx, br.gate, dy)
    got = omni.omni_expert_backward_blocked(inp["x"], inp["W"], inp["V"], br.idx, br.gate, dy,
                                            br.token_order)
    torch.cuda.synchronize()
    n = int(ref[3].item())
    assert int(got[3].item()) == n and torch.equal(got[2][:n], ref[2][:n])
    for name_, a, b in (("dx", got[0], ref[0]), ("dgate", got[1], ref[1]),
                        ("dW", got[4][:n], ref[4][:n]), ("dV", got[5][:n], ref[5][:n])):
        rel = ((a - b).norm() / b.norm()).item()
        say(f"  {name_}: rel diff {rel:.2e}")
        assert rel <= RTOL_FP32_ARITH, name_
    del inp, br, ref, got
    torch.cuda.empty_cache()
