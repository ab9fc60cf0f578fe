#!/usr/bin/env python3
"""Routed-branch forward benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole routed branch (omni_router, omni_schedule,
omni_expert_forward) over one batch of seeded synthetic inputs that are
already resident in HBM.  The default workload is 4096 tokens over 1.7M
atomic experts (d = 2048, N_r = N_c = 1304, K = B = 128, bf16 inputs, fp32
arithmetic).  Prints ONE JSON line.

Timing: W untimed steps, then exactly K timed steps between two device
synchronisations, each step after a cache flush (a 1 GiB read, which leaves
every L2 and the 256 MB Infinity Cache holding clean, unrelated lines), with
HIP events (torch.cuda.Event on the stream the library launches on) around
each call.  The value is the mean of those K cold steps.  The same step run
K times back to back (warm caches) is reported beside it, as are two
batches in flight on two streams (one step's router and schedule overlap
the other's assembly; a throughput figure, not the value) and replays of the
step captured as a HIP graph.
The assembly is the one RoutedBranch runs by default (--assembly auto): the
device picks the per-task passes or the blocked form from the routing's
reuse; config.assembly_chosen says which ran.  The roofline entry covers the
assembly call: for the per-task passes its algorithmic bytes are the unique
W and V rows gathered, x read once, y written once and 12 bytes of task
metadata per task (the unique expert count is taken from the step's own
ids); for the blocked form it is the executed MFMA work.  The line also
carries the measured ceilings of this GPU for the assembly's access pattern
(a random gather of the step's own V rows) and for a device copy.

cpu_baseline: the float64 CPU oracle timed on this host on a bounded sample
of the same workload's tokens, scaled to the full token count.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms per 4096-token routed-branch forward (router+sched+experts); % HBM peak"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096,
                    help="tokens the CPU oracle routes and assembles (capped at L)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense-router", action="store_true",
                    help="skip timing the fully connected router of the ablation")
    ap.add_argument("--token-order", action="store_true",
                    help="time the step with the token-ordered output pass as the headline")
    ap.add_argument("--assembly", choices=("auto", "expert_centric", "blocked"), default="auto",
                    help="assembly of the headline step: auto (the device picks per call, "
                         "RoutedBranch's default), expert_centric (the per-task passes) or "
                         "blocked (dense products per token block)")
    ap.add_argument("--no-two-stream", action="store_true",
                    help="skip the two-batch, two-stream throughput measurement (profiling runs "
                         "use it so that kernel durations are not measured while two steps "
                         "share the GPU)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing the backward calls")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before timing, run one plain device copy of this many MiB "
                         "(reference kernel for scaling hardware byte counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


CSRC = os.path.join(ROOT, "atomic_expert_routing_amd", "csrc")
# the sources of every kernel an automatic-assembly call launches
TRAFFIC_SRCS = ("assembly.hip", "schedule.hip", "blocked.hip", "omni_internal.h")


def profile_path(workload_name):
    return os.path.join(ROOT, "profiles", f"routed_forward_{workload_name}.md")


def sources_sha256():
    import hashlib

    h = hashlib.sha256()
    for name in TRAFFIC_SRCS:
        h.update(name.encode())
        h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()


def measured_traffic(workload_name, assembly):
    """Counter-measured bytes per assembly call from the committed rocprofv3
    summary of this workload, or None when there is none for this assembly
    or it was taken on other kernel source."""
    import re

    path = profile_path(workload_name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel sources sha256 \([^)]*\): ([0-9a-f]{64})", text)
    m_bytes = re.search(r"assembly call traffic bytes \(%s\): (\d+)" % assembly, text)
    if not (m_hash and m_bytes) or m_hash.group(1) != sources_sha256():
        return None
    return int(m_bytes.group(1))


def cpu_baseline(inp, w, n_tok, seed):
    """Time the oracle (as it stands) on n_tok sampled tokens; scale to L."""
    import numpy as np
    import threadpoolctl
    import torch

    from oracle import omni_oracle as O

    rs = np.random.Generator(np.random.PCG64(seed + 1))
    toks = np.sort(rs.choice(w.L, size=min(n_tok, w.L), replace=False))
    # setup (untimed): bring the sampled inputs and the router weights to host
    x = inp["x"][torch.as_tensor(toks, device=inp["x"].device)].to("cpu", torch.float64).numpy()
    Wr = inp["Wr"].to("cpu", torch.float64).numpy()
    Wc = inp["Wc"].to("cpu", torch.float64).numpy()
    t0 = time.perf_counter()
    idx, score, gate, _, _ = O.route(x, Wr, Wc, w.K)
    t_route = time.perf_counter() - t0
    # setup (untimed): the W and V rows those routes need
    uids = np.unique(idx)
    ids_dev = torch.as_tensor(uids, device=inp["W"].device)
    rows_W = inp["W"].index_select(0, ids_dev).to("cpu", torch.float64).numpy()
    rows_V = inp["V"].index_select(0, ids_dev).to("cpu", torch.float64).numpy()

    class Rows:
        def __init__(self, rows):
            self.rows = rows

        def __getitem__(self, ids):
            return self.rows[np.searchsorted(uids, ids)]

    t0 = time.perf_counter()
    perm, off = O.schedule(idx, w.N, w.B)
    O.assemble_expert_centric(x, Rows(rows_W), Rows(rows_V), idx, gate, perm, off)
    t_rest = time.perf_counter() - t0
    secs = t_route + t_rest
    blas = [p for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
    cores = max([p.get("num_threads", 1) for p in blas] + [1])
    return {
        "value": round(secs * 1e3 * w.L / len(toks), 3),
        "unit": "ms",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{len(toks)} of {w.L} tokens (seeded), router+schedule+expert-centric "
                   f"assembly in float64, {secs:.2f} s measured, scaled x{w.L / len(toks):g}; "
                   f"host affinity {len(os.sched_getaffinity(0))} cpus; W/V rows and router "
                   f"weights copied to host before timing"),
        "stages_s": {"route": round(t_route, 3), "schedule+assembly": round(t_rest, 3)},
    }


def time_mlp(inp, w, steps, seed, step_ms):
    """The layer's shared dense MLP (SwiGLU, d_ff = 8d/3 rounded to 128),
    accumulated into a routed output; the layer is the routed step plus it."""
    import torch

    from atomic_expert_routing_amd import omni, synth

    F = synth.mlp_hidden(w.d)
    mw = synth.mlp_weights(w.L, w.d, F, w.dtype, seed=seed, device="cuda")
    y = torch.zeros((w.L, w.d), dtype=torch.float32, device="cuda")
    dt = omni.OMNI_BF16 if w.dtype == "bf16" else omni.OMNI_F32
    ws = torch.empty(omni.omni_workspace_bytes(omni.OMNI_OP_SHARED_MLP, w.L, w.d, 1, 1, 1, F, 1, dt),
                     dtype=torch.uint8, device="cuda")
    run = lambda: omni.omni_shared_mlp(inp["x"], mw["Wg"], mw["Wu"], mw["Wd"], y, True, ws)
    for _ in range(2):
        run()
    torch.cuda.synchronize()
    ts = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = statistics.median(ts)
    flops = 3 * 2.0 * w.L * w.d * F
    return {"d_ff": F, "ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "layer_ms": round(step_ms + ms, 4),
            "note": "SwiGLU MLP; layer = routed branch step (events) + this MLP"}


def time_dense_router(inp, w, router_ms, seed, reps=3):
    """The ablation's fully connected router over all N experts (seeded
    Wn [N, d] ~ N(0, 1/d)), against the Cartesian router stage."""
    import torch

    from atomic_expert_routing_amd import omni, synth

    Wn = synth.normal_rows("W", w.N, w.d, 1.0 / math.sqrt(w.d), seed + 1, "cuda",
                           w.torch_dtype)
    dt = omni.OMNI_BF16 if w.dtype == "bf16" else omni.OMNI_F32
    ws = torch.empty(omni.omni_workspace_bytes(omni.OMNI_OP_DENSE_ROUTER, w.L, w.d, 1, 1, w.K,
                                               w.N, 1, dt), dtype=torch.uint8, device="cuda")
    idx = torch.empty((w.L, w.K), dtype=torch.int32, device="cuda")
    sc = torch.empty((w.L, w.K), dtype=torch.float32, device="cuda")
    g = torch.empty((w.L, w.K), dtype=torch.float32, device="cuda")
    run = lambda: omni.omni_dense_router(inp["x"], Wn, w.K, idx, sc, g, ws)
    run()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = statistics.median(ts)
    flops = 2.0 * w.L * w.d * w.N
    del Wn, ws
    torch.cuda.empty_cache()
    return {"ms": round(ms, 3), "logit_tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "vs_cartesian_router": round(ms / router_ms, 1),
            "note": "s = x Wn^T over all N experts in 65536-expert chunks, exact top-K, "
                    "LogSoftmax over N; the pages report 30.6x latency for this substitution"}


def blocked_roofline(br, w, mean_ms, order):
    """The blocked assembly's MFMA work: per block of 64 tokens, 64 x npad x d
    products on the W side and twice that on the V side (hi and lo terms),
    npad = the block's union size rounded up to whole 128-column tiles."""
    import torch

    order = order.long()
    npad = 0
    for b0 in range(0, w.L, 64):
        u = int(torch.unique(br.idx[order[b0:b0 + 64]]).numel())
        npad += max(1, -(-u // 128)) * 128
    flops = 64 * npad * w.d * 2 * 3
    achieved = flops / (mean_ms * 1e-3) / 1e12
    return {"kernel": "omni_expert_forward_blocked (blk_union, blk_plan, blk_gates, blk_act, "
                      "blk_out)",
            "bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None, "mfma_flops": flops, "definition_flops": 4 * w.M * w.d,
            "mean_ms": round(mean_ms, 4)}


def time_variant(inp, w, br, steps, token_order, assembly, flush):
    """Another configuration of the step timed on the same inputs, cold as
    the value: per-stage medians, and how its y compares with the headline
    step's (bitwise where the same sums are taken in the same order; to fp32
    rounding otherwise)."""
    import torch

    from atomic_expert_routing_amd import omni

    bo = omni.RoutedBranch(w.L, w.d, w.Nr, w.Nc, w.K, w.B, w.torch_dtype,
                           token_order=token_order, assembly=assembly)
    for _ in range(2):
        bo.forward(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"])
    torch.cuda.synchronize()
    evs = []
    for _ in range(steps):
        flush()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record()
        bo.router(inp["x"], inp["Wr"], inp["Wc"])
        ev[1].record()
        bo.schedule()
        ev[2].record()
        bo.expert_forward(inp["x"], inp["W"], inp["V"])
        ev[3].record()
        evs.append(ev)
    torch.cuda.synchronize()

    def med(a, b):
        return round(statistics.median(e[a].elapsed_time(e[b]) for e in evs), 4)

    same = bool(torch.equal(bo.y, br.y))
    rel = ((bo.y - br.y).norm() / br.y.norm()).item()
    del bo
    return {"token_order": bool(token_order or assembly == "blocked"), "assembly": assembly,
            "step_events_ms": med(0, 3), "schedule_ms": med(1, 2), "expert_forward_ms": med(2, 3),
            "y_bitwise_equal": same, "y_rel_diff": rel}


def _median_ms(fn, steps):
    """Median over `steps` calls of fn, each bracketed by events on the
    current stream, after one untimed call."""
    import torch

    fn()
    torch.cuda.synchronize()
    ev = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        ev.append((e0, e1))
    torch.cuda.synchronize()
    return statistics.median(a.elapsed_time(b) for a, b in ev)


def time_backward(inp, w, br, steps, seed):
    """omni_expert_backward + omni_router_backward on the step's routing, for a
    seeded upstream gradient; preallocated outputs and workspaces.  The expert
    backward is timed with fp32 and with bf16 gradient rows."""
    import torch

    from atomic_expert_routing_amd import omni, synth

    dy = synth.upstream_grad(w, seed=seed, device="cuda")
    L, d, K, N = w.L, w.d, w.K, w.N
    cap = min(N, L * K)
    f32, i32 = torch.float32, torch.int32
    dx = torch.empty((L, d), dtype=f32, device="cuda")
    dgate = torch.empty((L, K), dtype=f32, device="cuda")
    uniq = torch.empty((cap,), dtype=i32, device="cuda")
    n_uniq = torch.empty((1,), dtype=i32, device="cuda")
    dW = torch.empty((cap, d), dtype=f32, device="cuda")
    dV = torch.empty((cap, d), dtype=f32, device="cuda")
    dW16 = torch.empty((cap, d), dtype=torch.bfloat16, device="cuda")
    dV16 = torch.empty((cap, d), dtype=torch.bfloat16, device="cuda")
    dWr = torch.empty((w.Nr, d), dtype=f32, device="cuda")
    dWc = torch.empty((w.Nc, d), dtype=f32, device="cuda")
    dt = omni.OMNI_BF16 if w.dtype == "bf16" else omni.OMNI_F32
    ws_e = torch.empty(omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_BACKWARD, L, d, 1, 1, K, N,
                                                 1, dt), dtype=torch.uint8, device="cuda")
    ws_r = torch.empty(omni.omni_workspace_bytes(omni.OMNI_OP_ROUTER_BACKWARD, L, d, w.Nr, w.Nc,
                                                 K, N, 1, dt), dtype=torch.uint8, device="cuda")

    def run(ev=None, rows=(dW, dV)):
        if ev is not None:
            ev[0].record()
        omni.omni_expert_backward(inp["x"], inp["W"], inp["V"], br.idx, br.gate, dy, dx, dgate,
                                  uniq, n_uniq, rows[0], rows[1], ws_e)
        if ev is not None:
            ev[1].record()
        omni.omni_router_backward(inp["x"], inp["Wr"], inp["Wc"], br.idx, br.gate, dgate, dx,
                                  dWr, dWc, ws_r)
        if ev is not None:
            ev[2].record()

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in evs:
        run(e)
    torch.cuda.synchronize()
    exp_ms = statistics.median(e[0].elapsed_time(e[1]) for e in evs)
    rt_ms = statistics.median(e[1].elapsed_time(e[2]) for e in evs)
    evs16 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    run(rows=(dW16, dV16))
    for e in evs16:
        run(e, rows=(dW16, dV16))
    torch.cuda.synchronize()
    exp16_ms = statistics.median(e[0].elapsed_time(e[1]) for e in evs16)
    blocked_ms = None
    if w.dtype == "bf16" and d % 256 == 0:
        # the blocked form, over the schedule's token order (fp32 rows)
        _, _, order = omni.omni_schedule(br.idx, w.N, w.B, token_order=True)
        ws_b = torch.empty(omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_BACKWARD_BLOCKED, L, d,
                                                     1, 1, K, N, 1, dt),
                           dtype=torch.uint8, device="cuda")

        def run_blocked():
            omni.omni_expert_backward_blocked(inp["x"], inp["W"], inp["V"], br.idx, br.gate, dy,
                                              order, dx, dgate, uniq, n_uniq, dW, dV, ws_b)

        blocked_ms = _median_ms(run_blocked, steps)
        del ws_b
    # the automatic backward: the device picks the form by the forward's rule
    ws_a = torch.empty(omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_BACKWARD_AUTO, L, d, 1, 1, K,
                                                 N, 1, dt), dtype=torch.uint8, device="cuda")
    chosen = torch.empty((1,), dtype=i32, device="cuda")

    def run_auto():
        omni.omni_expert_backward_auto(inp["x"], inp["W"], inp["V"], br.idx, br.gate, dy, dx,
                                       dgate, uniq, n_uniq, dW, dV, ws_a, chosen=chosen)

    auto_ms = _median_ms(run_auto, steps)
    auto_chosen = int(chosen.item())
    del ws_a
    U = int(n_uniq.item())
    es = 2 if w.dtype == "bf16" else 4
    # unique W and V rows read, their fp32 dW and dV rows written; x and dy
    # read, dx written; dgate written and 12 B of task metadata per task
    exp_bytes = 2 * U * d * es + 2 * U * d * 4 + L * d * es + 2 * L * d * 4 + w.M * (4 + 12)
    router_flops = 2 * 2.0 * L * d * (w.Nr + w.Nc)  # ds^T x and ds W_rc
    exp16_bytes = exp_bytes - 2 * U * d * 2
    return {
        "expert_backward_ms": round(exp_ms, 4),
        "expert_backward_bf16_rows_ms": round(exp16_ms, 4),
        "expert_backward_blocked_ms": None if blocked_ms is None else round(blocked_ms, 4),
        "expert_backward_auto_ms": round(auto_ms, 4),
        "expert_backward_auto_chosen": "blocked" if auto_chosen else "per_task",
        "expert_backward_bf16_rows_hbm_frac": round(
            exp16_bytes / (exp16_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "router_backward_ms": round(rt_ms, 4),
        "unique_experts": U,
        "expert_backward_algorithmic_bytes": exp_bytes,
        "expert_backward_hbm_frac": round(exp_bytes / (exp_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "router_backward_tflops": round(router_flops / (rt_ms * 1e-3) / 1e12, 1),
        "note": "router products run twice (bf16 high and low parts of the logit gradients)",
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {max(args.gpus, world)}): the routed "
              "branch here is a single-GPU kernel path (it would shard by token or by ranges of "
              "expert groups, with an all-gather of ids and x and a reduce-scatter of y)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from atomic_expert_routing_amd import omni, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    pipe_streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    w = synth.WORKLOADS[args.workload or synth.HEADLINE]
    log(f"[bench] workload {w.name}: generating inputs on the GPU")
    inp = synth.make_inputs(w, seed=args.seed, device="cuda")
    br = omni.RoutedBranch(w.L, w.d, w.Nr, w.Nc, w.K, w.B, w.torch_dtype,
                           token_order=args.token_order, assembly=args.assembly)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        br.router(inp["x"], inp["Wr"], inp["Wc"])
        if ev is not None:
            ev[1].record()
        br.schedule()
        if ev is not None:
            ev[2].record()
        br.expert_forward(inp["x"], inp["W"], inp["V"])
        if ev is not None:
            ev[3].record()

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] copy probe: {args.copy_probe_mib} MiB read + written")

    # cache flush between cold steps: a 1 GiB read evicts every L2 and the
    # 256 MB Infinity Cache with clean lines (no write-back left for the step)
    flush_src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")

    def flush():
        flush_src.sum()

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the value: exactly K steps, each after a flush; the events bracket the
    # step alone, the flushes between them are not counted
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} cold-cache steps")
    torch.cuda.synchronize()
    for i in range(args.steps):
        flush()
        step(evs[i])
    torch.cuda.synchronize()
    cold_ms = statistics.fmean(e[0].elapsed_time(e[3]) for e in evs)
    # warm: K steps back to back between two synchronisations (wall clock)
    log(f"[bench] timing {args.steps} warm steps")
    evs_w = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs_w[i])
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_step = cold_ms
    chosen = (int(br.chosen.item()) if args.assembly == "auto"
              else int(args.assembly == "blocked"))
    # two batches in flight: a second branch (own outputs and workspace) on a
    # second stream, steps alternating between the two; each step does the
    # whole path, and the two streams overlap one step's router and schedule
    # with the other's assembly.  Timed before any graph capture: after one,
    # launches on the two streams were measured to no longer overlap.
    br2 = omni.RoutedBranch(w.L, w.d, w.Nr, w.Nc, w.K, w.B, w.torch_dtype,
                            token_order=args.token_order, assembly=args.assembly)
    pair = [(br, pipe_streams[0]), (br2, pipe_streams[1])]

    def two_stream(n):
        start = torch.cuda.Event()
        start.record(torch.cuda.current_stream())
        for _, st in pair:
            st.wait_event(start)
        for i in range(n):
            b, st = pair[i % 2]
            with torch.cuda.stream(st):
                b.forward(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"])
        for _, st in pair:
            done = torch.cuda.Event()
            done.record(st)
            torch.cuda.current_stream().wait_event(done)

    two_stream_ms, two_stream_same_y = None, None
    if not args.no_two_stream:
        two_stream(args.warmup + 1)
        torch.cuda.synchronize()
        log(f"[bench] timing {args.steps} steps on two streams")
        t0 = time.perf_counter()
        two_stream(args.steps)
        torch.cuda.synchronize()
        two_stream_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        two_stream_same_y = bool(torch.equal(br.y, br2.y))
    del br2, pair
    # the same step captured once as a HIP graph and replayed (warm)
    br.capture(inp["x"], inp["Wr"], inp["Wc"], inp["W"], inp["V"])
    for _ in range(args.warmup):
        br.replay()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} graph replays")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        br.replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    def med(ev, a, b):
        return statistics.median(e[a].elapsed_time(e[b]) for e in ev)

    router_ms, sched_ms, expert_ms = med(evs, 0, 1), med(evs, 1, 2), med(evs, 2, 3)
    step_min_ms = min(e[0].elapsed_time(e[3]) for e in evs)
    expert_mean_ms = statistics.fmean(e[2].elapsed_time(e[3]) for e in evs)
    step_ev_ms = med(evs, 0, 3)

    # algorithmic bytes of one expert-assembly call (the per-task passes)
    uniq = torch.unique(br.idx)
    U = int(uniq.numel())
    es = 2 if w.dtype == "bf16" else 4
    expert_bytes = U * 2 * w.d * es + w.L * w.d * es + w.L * w.d * 4 + w.M * 12
    achieved = expert_bytes / (expert_mean_ms * 1e-3) / 1e9
    router_bytes = (w.L + w.Nr + w.Nc) * w.d * es + w.M * 12
    sched_bytes = w.M * 4 + w.M * 4 + (w.G + 1) * 4
    branch_bytes = expert_bytes + router_bytes + sched_bytes
    router_flops = 2.0 * w.L * w.d * (w.Nr + w.Nc)

    # measured ceilings: the step's own V rows gathered in random order (the
    # assembly's access pattern), cold; and a 1 GiB device copy
    log("[bench] ceilings: row gather and copy")
    g = torch.Generator(device="cuda").manual_seed(args.seed + 11)
    rows = uniq[torch.randperm(U, generator=g, device="cuda")].to(torch.int32).contiguous()
    sink = omni.omni_gather_probe(inp["V"], rows)
    gather_t = []
    for _ in range(5):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        omni.omni_gather_probe(inp["V"], rows, sink)
        e1.record()
        torch.cuda.synchronize()
        gather_t.append(e0.elapsed_time(e1))
    gather_gbs = U * w.d * es / (statistics.median(gather_t) * 1e-3) / 1e9
    cdst = torch.empty_like(flush_src)
    copy_t = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        cdst.copy_(flush_src)
        e1.record()
        torch.cuda.synchronize()
        copy_t.append(e0.elapsed_time(e1))
    copy_gbs = 2 * flush_src.numel() / (statistics.median(copy_t) * 1e-3) / 1e9
    del cdst, sink

    if chosen:
        order = omni.omni_schedule(br.idx, w.N, w.B, token_order=True, tasks=False)[2]
        roofline = blocked_roofline(br, w, expert_mean_ms, order)
        roofline["traffic"] = measured_traffic(w.name, args.assembly)
        roofline["kernel"] = ("omni_expert_forward_auto, blocked form chosen (auto_clear, "
                              "auto_mark, the token order sort, blk_union, blk_plan, blk_act, "
                              "blk_out; the per-task launches return at once)"
                              if args.assembly == "auto" else roofline["kernel"])
    else:
        roofline = {
            "kernel": ("omni_expert_forward_auto, schedule and per-task passes chosen "
                       "(auto_clear, auto_mark, the schedule's radix sort and sched_offsets, "
                       "act_plan, expert_act, expert_out_w; the blocked launches return at "
                       "once)"
                       if args.assembly == "auto"
                       else "omni_expert_forward (act_plan, expert_act, expert_out_w)"),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(w.name, args.assembly),
            "algorithmic_bytes": expert_bytes,
            "mean_ms": round(expert_mean_ms, 4),
            "ceiling_row_gather_GBs": round(gather_gbs, 1),
            "frac_of_row_gather_ceiling": round(achieved / gather_gbs, 4),
        }

    out = {
        "metric": METRIC,
        "value": round(ms_step, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype if w.dtype == "bf16" else "f32",
        "data": "synthetic: seeded Gaussian x and random-init W, V, W_r, W_c (no trained weights)",
        "config": {**w.describe(), "parallelism": "single GPU",
                   "token_ordered_output": bool(args.token_order or args.assembly == "blocked"),
                   "assembly": args.assembly,
                   "assembly_chosen": "blocked" if chosen else "per_task"},
        "tokens_per_s": round(w.L / (ms_step * 1e-3), 1),
        "timing": "mean of the K timed steps, each after a cache flush (cold); events around "
                  "the step",
        "warm_ms_per_step": round(eager_ms, 4),
        "graph_ms_per_step": round(graph_ms, 4),
        "two_stream_ms_per_step": None if two_stream_ms is None else round(two_stream_ms, 4),
        "two_stream_note": "throughput with two independent batches in flight on two streams "
                           "(each step the whole path on its own buffers, warm); not the value",
        "two_stream_y_bitwise_equal": two_stream_same_y,
        "branch_hbm_frac": round(branch_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "stages_ms_median": {"router": round(router_ms, 4), "schedule": round(sched_ms, 4),
                             "expert_forward": round(expert_ms, 4),
                             "step_events": round(step_ev_ms, 4)},
        "warm_stages_ms_median": {"router": round(med(evs_w, 0, 1), 4),
                                  "schedule": round(med(evs_w, 1, 2), 4),
                                  "expert_forward": round(med(evs_w, 2, 3), 4),
                                  "step_events": round(med(evs_w, 0, 3), 4)},
        "unique_experts": U,
        "roofline": roofline,
        "ceilings": {"row_gather_GBs": round(gather_gbs, 1), "copy_GBs": round(copy_gbs, 1),
                     "note": "row gather: the step's unique V rows read once in random order, "
                             "one wave per row, after a flush (omni_gather_probe); copy: a "
                             "1 GiB device copy, bytes read plus written"},
        "router_gemm_flops": router_flops,
    }
    out["step_events_ms_min"] = round(step_min_ms, 4)

    # the token-centric order the expert-centric schedule replaces, timed on
    # the same routing (same y up to rounding), cold as the value
    tc_times = []
    y_tc = torch.empty_like(br.y)
    omni.omni_expert_forward_token_centric(inp["x"], inp["W"], inp["V"], br.idx, br.gate, y_tc)
    for i in range(args.steps):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        omni.omni_expert_forward_token_centric(inp["x"], inp["W"], inp["V"], br.idx, br.gate, y_tc)
        e1.record()
        torch.cuda.synchronize()
        tc_times.append(e0.elapsed_time(e1))
    tc_ms = statistics.median(tc_times)
    out["token_centric_assembly_ms"] = round(tc_ms, 4)
    out["expert_centric_speedup_vs_token_centric"] = round(tc_ms / expert_ms, 3)

    variants = []
    if args.assembly != "expert_centric":
        variants.append(time_variant(inp, w, br, args.steps, False, "expert_centric", flush))
    variants.append(time_variant(inp, w, br, args.steps, True, "expert_centric", flush))
    if w.dtype == "bf16" and w.d % 256 == 0 and args.assembly != "blocked":
        variants.append(time_variant(inp, w, br, args.steps, True, "blocked", flush))
    out["variants"] = variants

    out["shared_mlp"] = time_mlp(inp, w, args.steps, args.seed, step_ev_ms)
    if not args.no_dense_router:
        out["dense_router"] = time_dense_router(inp, w, router_ms, args.seed)

    if not args.no_backward:
        out["backward"] = time_backward(inp, w, br, args.steps, args.seed)

    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {args.cpu_sample_tokens} tokens")
        out["cpu_baseline"] = cpu_baseline(inp, w, args.cpu_sample_tokens, args.seed)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
