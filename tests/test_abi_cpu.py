"""Host-side checks of libomni.so that need no GPU.

The library must load, export every function include/omni.h declares, size
workspaces, and reject invalid arguments before it touches the GPU (the
validation runs on the host, so these calls never reach the HIP runtime).
"""

import ctypes
import os
import re

import pytest

from atomic_expert_routing_amd import omni

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "omni.h")

pytestmark = pytest.mark.skipif(not os.path.exists(omni._LIB_PATH),
                                reason="libomni.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"OMNI_API\s+[\w\s\*]+?\b(omni_\w+)\s*\(", text)


def test_header_declares_the_abi():
    names = declared_functions()
    assert set(names) == set(omni.EXPORTED), names


def test_library_loads_and_exports_every_declared_symbol():
    lib = omni.library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.omni_abi_version() == 10


def test_status_strings():
    lib = omni.library()
    for s in range(5):
        assert lib.omni_status_string(s).decode()
    assert lib.omni_status_string(99).decode() == "unknown status"


def test_workspace_sizes():
    # router: fp32 logits [L, N_r + N_c], 256-byte aligned
    assert omni.omni_workspace_bytes(omni.OMNI_OP_ROUTER, L=4096, d=2048, Nr=1304, Nc=1304,
                                     K=128) == 4096 * 2608 * 4
    # expert forward: fp32 activations [L*K], then the activation pass's chunk
    # starts (one per 32 scheduled tasks, plus the end), each part 256-byte aligned
    M = 4096 * 128
    assert omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_FORWARD, L=4096, d=2048, K=128,
                                     N=1700416, B=128) == M * 4 + -(-(M // 32 + 1) * 4 // 256) * 256
    for B in (0, 2**31):
        with pytest.raises(omni.OmniError):
            omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_FORWARD, L=4, d=64, K=2, N=100, B=B)
    # schedule: four O(M) int32 sort buffers plus the digit table
    ws = omni.omni_workspace_bytes(omni.OMNI_OP_SCHEDULE, L=4096, K=128, N=1700416, B=128)
    assert 4 * 4096 * 128 * 4 <= ws < 5 * 4096 * 128 * 4


@pytest.mark.parametrize("kw,status", [
    (dict(L=0), omni.OMNI_ERR_INVALID_ARG),
    (dict(K=0), omni.OMNI_ERR_INVALID_ARG),
    (dict(d=12), omni.OMNI_ERR_UNSUPPORTED),
    (dict(d=-8), omni.OMNI_ERR_INVALID_ARG),
    (dict(d=8192), omni.OMNI_ERR_UNSUPPORTED),
    (dict(Nr=0), omni.OMNI_ERR_INVALID_ARG),
    (dict(Nr=5000), omni.OMNI_ERR_UNSUPPORTED),
    (dict(K=17, Nr=4, Nc=4), omni.OMNI_ERR_INVALID_ARG),  # K > N_r*N_c
    (dict(K=600, Nr=100, Nc=100), omni.OMNI_ERR_UNSUPPORTED),
    (dict(L=2**30, K=4), omni.OMNI_ERR_UNSUPPORTED),  # L*K >= 2^31
    (dict(dtype=7), omni.OMNI_ERR_INVALID_ARG),
])
def test_router_size_validation(kw, status):
    args = dict(L=64, d=64, Nr=32, Nc=32, K=16, N=1024, B=16, dtype=omni.OMNI_BF16)
    args.update(kw)
    with pytest.raises(omni.OmniError) as e:
        omni.omni_workspace_bytes(omni.OMNI_OP_ROUTER, **args)
    assert e.value.status == status


def test_fp32_d_limit_is_lower():
    assert omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_FORWARD, L=4, d=4096, K=2, N=8,
                                     dtype=omni.OMNI_BF16) > 0
    with pytest.raises(omni.OmniError) as e:
        omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_FORWARD, L=4, d=4096, K=2, N=8,
                                  dtype=omni.OMNI_F32)
    assert e.value.status == omni.OMNI_ERR_UNSUPPORTED


def test_expert_forward_k_limit():
    with pytest.raises(omni.OmniError) as e:
        omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_FORWARD, L=4, d=64, K=513, N=10000)
    assert e.value.status == omni.OMNI_ERR_UNSUPPORTED


def test_schedule_validation():
    for kw in (dict(N=0), dict(B=0), dict(N=2**31)):
        args = dict(L=4, K=2, N=100, B=8)
        args.update(kw)
        with pytest.raises(omni.OmniError):
            omni.omni_workspace_bytes(omni.OMNI_OP_SCHEDULE, **args)
    with pytest.raises(omni.OmniError):
        omni.omni_workspace_bytes(11)


@pytest.mark.parametrize("B", [2**31, 2**32, 2**32 + 5, 2**62])
def test_schedule_rejects_group_sizes_beyond_int32(B):
    """B is taken as an int by the kernels: B >= 2^31 is refused on the host
    (such a B would otherwise wrap to 0, INT_MIN or a small divisor)."""
    with pytest.raises(omni.OmniError) as e:
        omni.omni_workspace_bytes(omni.OMNI_OP_SCHEDULE, L=4, K=2, N=100, B=B)
    assert e.value.status == omni.OMNI_ERR_UNSUPPORTED and b"B =" in omni.library().omni_last_error()
    lib = omni.library()
    fake = ctypes.c_void_p(4096)  # never dereferenced: the call fails before any launch
    s = lib.omni_schedule(fake, 4, 2, 100, B, fake, fake, fake, fake, 1 << 30, None)
    assert s == omni.OMNI_ERR_UNSUPPORTED and b"B =" in lib.omni_last_error()


def test_schedule_group_size_at_or_above_n_is_one_group():
    """Every B >= N (up to 2^31-1) gives G = 1; the workspace equals B = N's."""
    one = omni.omni_workspace_bytes(omni.OMNI_OP_SCHEDULE, L=4096, K=128, N=1000, B=1000)
    for B in (1001, 2**20, 2**31 - 1):
        assert omni.omni_workspace_bytes(omni.OMNI_OP_SCHEDULE, L=4096, K=128, N=1000, B=B) == one


def test_calls_reject_before_launch():
    """Invalid calls return an error and a message without touching the GPU."""
    lib = omni.library()
    fake = ctypes.c_void_p(4096)  # never dereferenced: validation fails first
    # NULL output pointer
    s = lib.omni_router(fake, fake, fake, 4, 8, 2, 2, 2, omni.OMNI_F32, None, fake, fake,
                        fake, 1 << 20, None)
    assert s == omni.OMNI_ERR_INVALID_ARG and b"NULL" in lib.omni_last_error()
    # workspace too small
    s = lib.omni_router(fake, fake, fake, 4, 8, 2, 2, 2, omni.OMNI_F32, fake, fake, fake,
                        fake, 16, None)
    assert s == omni.OMNI_ERR_WORKSPACE and b"workspace" in lib.omni_last_error()
    # misaligned workspace
    s = lib.omni_schedule(fake, 4, 2, 10, 2, fake, fake, None, ctypes.c_void_p(4100), 1 << 20,
                          None)
    assert s == omni.OMNI_ERR_INVALID_ARG
    # perm without group_off, and no output at all
    s = lib.omni_schedule(fake, 4, 2, 10, 2, fake, None, None, fake, 1 << 20, None)
    assert s == omni.OMNI_ERR_INVALID_ARG and b"together" in lib.omni_last_error()
    s = lib.omni_schedule(fake, 4, 2, 10, 2, None, None, None, fake, 1 << 20, None)
    assert s == omni.OMNI_ERR_INVALID_ARG and b"no output" in lib.omni_last_error()
    # misaligned x
    s = lib.omni_expert_forward(ctypes.c_void_p(4098), fake, fake, fake, fake, fake, fake, None,
                                4, 8, 10, 2, 3, omni.OMNI_BF16, fake, fake, 1 << 20, None)
    assert s == omni.OMNI_ERR_INVALID_ARG
    # K larger than the grid
    s = lib.omni_router(fake, fake, fake, 4, 8, 2, 2, 5, omni.OMNI_F32, fake, fake, fake,
                        fake, 1 << 20, None)
    assert s == omni.OMNI_ERR_INVALID_ARG and b"K" in lib.omni_last_error()


def test_backward_workspace_sizes_and_validation():
    # expert backward: per-task terms, expert-sorted tasks, per-expert segments,
    # and the row order (a key, a sorted position and a 16-byte record per
    # possible used expert, U_cap = min(N, L*K), plus the sort's key offsets)
    ws = omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_BACKWARD, L=4096, d=2048, K=128,
                                   N=1700416)
    M = 4096 * 128
    assert ws >= (4 * M + 1700416 + 6 * M) * 4 and ws < (18 * M + 1700416 + 4096 + 4096) * 4
    # router backward (bf16): hi/lo logit gradients, their transposes, x^T, W_rc^T
    ws = omni.omni_workspace_bytes(omni.OMNI_OP_ROUTER_BACKWARD, L=4096, d=2048, Nr=1304,
                                   Nc=1304, K=128)
    assert ws == (2 * 4096 * 2624 * 2 + 2 * 2608 * 4096 * 2 + 2048 * 4096 * 2
                  + 2048 * 2624 * 2)
    # fp32: one fp32 logit-gradient matrix
    assert omni.omni_workspace_bytes(omni.OMNI_OP_ROUTER_BACKWARD, L=64, d=64, Nr=32, Nc=32,
                                     K=16, dtype=omni.OMNI_F32) == 64 * 64 * 4
    for op in (omni.OMNI_OP_EXPERT_BACKWARD, omni.OMNI_OP_ROUTER_BACKWARD):
        with pytest.raises(omni.OmniError) as e:
            omni.omni_workspace_bytes(op, L=4, d=12, Nr=4, Nc=4, K=2, N=16)
        assert e.value.status == omni.OMNI_ERR_UNSUPPORTED
    # the row pass keys tokens by 8 * ceil(L / 8) + 1 values, which must fit an int32
    with pytest.raises(omni.OmniError) as e:
        omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_BACKWARD, L=2**31 - 8, d=8, K=1, N=16)
    assert e.value.status == omni.OMNI_ERR_UNSUPPORTED and b"2^31-9" in omni.library().omni_last_error()
    lib = omni.library()
    fake = ctypes.c_void_p(4096)
    s = lib.omni_expert_backward(fake, fake, fake, fake, fake, fake, 4, 8, 16, 2, omni.OMNI_BF16,
                                 fake, fake, fake, None, omni.OMNI_F32, fake, fake, fake, 1 << 20,
                                 None)
    assert s == omni.OMNI_ERR_INVALID_ARG and b"NULL" in lib.omni_last_error()
    s = lib.omni_router_backward(fake, fake, fake, fake, fake, fake, 4, 8, 2, 2, 2, omni.OMNI_BF16,
                                 fake, fake, fake, fake, 16, None)
    assert s == omni.OMNI_ERR_WORKSPACE


def test_shared_mlp_workspace_and_validation():
    # bf16: the bf16 intermediate [L, d_ff]; fp32: two fp32 [L, d_ff] buffers
    assert omni.omni_workspace_bytes(omni.OMNI_OP_SHARED_MLP, L=4096, d=2048, N=5504) == 4096 * 5504 * 2
    assert omni.omni_workspace_bytes(omni.OMNI_OP_SHARED_MLP, L=64, d=64, N=128,
                                     dtype=omni.OMNI_F32) == 2 * 64 * 128 * 4
    for kw, st in ((dict(d=72, N=128), omni.OMNI_ERR_UNSUPPORTED),
                   (dict(d=64, N=100), omni.OMNI_ERR_UNSUPPORTED),
                   (dict(d=64, N=0), omni.OMNI_ERR_INVALID_ARG)):
        with pytest.raises(omni.OmniError) as e:
            omni.omni_workspace_bytes(omni.OMNI_OP_SHARED_MLP, L=8, **kw)
        assert e.value.status == st
    # fp32 takes any d % 8 == 0 and any d_ff
    assert omni.omni_workspace_bytes(omni.OMNI_OP_SHARED_MLP, L=8, d=72, N=100, dtype=omni.OMNI_F32) > 0


def test_dense_router_workspace_and_validation():
    # chunk logits [L, 65536] fp32 + running top-K keys [L, K] u64 + partials
    L, N, K = 4096, 1700416, 128
    chunks = -(-N // 65536)
    ws = omni.omni_workspace_bytes(omni.OMNI_OP_DENSE_ROUTER, L=L, d=2048, K=K, N=N)
    assert ws == L * 65536 * 4 + L * K * 8 + L * chunks * 8
    small = omni.omni_workspace_bytes(omni.OMNI_OP_DENSE_ROUTER, L=8, d=64, K=4, N=100)
    assert small >= 8 * 100 * 4
    for kw, st in ((dict(K=101, N=100), omni.OMNI_ERR_INVALID_ARG),
                   (dict(K=600, N=1000), omni.OMNI_ERR_UNSUPPORTED),
                   (dict(d=72, K=4, N=100), omni.OMNI_ERR_UNSUPPORTED),
                   (dict(N=0, K=1), omni.OMNI_ERR_INVALID_ARG)):
        args = dict(L=8, d=64)
        args.update(kw)
        with pytest.raises(omni.OmniError) as e:
            omni.omni_workspace_bytes(omni.OMNI_OP_DENSE_ROUTER, **args)
        assert e.value.status == st
    assert omni.omni_workspace_bytes(omni.OMNI_OP_DENSE_ROUTER, L=8, d=72, K=4, N=100,
                                     dtype=omni.OMNI_F32) > 0


def test_blocked_workspace_and_validation():
    """Blocks of 64 tokens; each block's union holds at most min(64 K, N) ids,
    padded to 128-column tiles; gate (fp32) and activation (2 x bf16) tiles
    are sized for every block at its largest union."""
    def a256(n):
        return (n + 255) // 256 * 256

    for L, K, N in ((16384, 256, 1700416), (4096, 128, 1700416), (100, 16, 1024), (65, 8, 50)):
        nb = -(-L // 64)
        ucap = -(-min(64 * K, N) // 128) * 128
        elems = nb * 64 * ucap
        want = (a256(nb * ucap * 4) + a256(nb * 4) + a256((nb + 1) * 4)
                + a256(elems * 4) + 2 * a256(elems * 2))
        got = omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_FORWARD_BLOCKED, L=L, d=2048, K=K, N=N)
        assert got == want, (L, K, N)
    for kw, st in ((dict(dtype=omni.OMNI_F32), omni.OMNI_ERR_UNSUPPORTED),
                   (dict(d=320), omni.OMNI_ERR_UNSUPPORTED),
                   (dict(K=513), omni.OMNI_ERR_UNSUPPORTED),
                   (dict(N=0), omni.OMNI_ERR_INVALID_ARG)):
        args = dict(L=128, d=256, K=16, N=1000)
        args.update(kw)
        with pytest.raises(omni.OmniError) as e:
            omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_FORWARD_BLOCKED, **args)
        assert e.value.status == st
    # the blocked backward: the forward's workspace, the task-slot map (as G),
    # dy split into two bf16 terms, then the per-task backward's workspace
    # then the expert sets: positions, keys and the sorted order of the used
    # experts (capacity min(N, L K)), the sort's buffers, per-set counts and
    # tile prefix, the token unions and the dense hi/lo tiles of dh and g SiLU
    for L, K, N, d in ((16384, 256, 1700416, 2048), (100, 16, 1024, 256)):
        nb = -(-L // 64)
        ucap = -(-min(64 * K, N) // 128) * 128
        fwd = omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_FORWARD_BLOCKED, L=L, d=d, K=K, N=N)
        rows = omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_BACKWARD, L=L, d=d, K=K, N=N)
        ue = min(N, L * K)
        smax = -(-ue // 64)
        tcap = L * K + 128 * smax
        got = omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_BACKWARD_BLOCKED, L=L, d=d, K=K, N=N)
        head = a256(fwd) + a256(nb * 64 * ucap * 4) + 2 * a256(L * d * 2) + a256(rows)
        tail = (a256(L * 4) + 2 * a256(ue * 4) + a256(smax * 4) + a256((smax + 1) * 4)
                + a256(tcap * 4) + 4 * a256(64 * tcap * 2))
        sort = got - head - tail  # the key sort's buffers: two key and value arrays and more
        assert 4 * ue * 4 <= sort <= 4 * a256(ue * 4) + 1 << 20, (L, K, N, sort)
    for kw in (dict(d=320), dict(L=524289)):
        args = dict(L=64, d=256, K=8, N=100)
        args.update(kw)
        with pytest.raises(omni.OmniError):
            omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_BACKWARD_BLOCKED, **args)
    lib = omni.library()
    fake = ctypes.c_void_p(4096)
    s = lib.omni_expert_backward_blocked(fake, fake, fake, fake, fake, fake, None, 64, 256, 1000,
                                         8, omni.OMNI_BF16, fake, fake, fake, fake, omni.OMNI_F32,
                                         fake, fake, fake, 1 << 30, None)
    assert s == omni.OMNI_ERR_INVALID_ARG and b"NULL" in lib.omni_last_error()
    # the token order is required
    s = lib.omni_expert_forward_blocked(fake, fake, fake, fake, fake, None, 64, 256, 1000, 8,
                                        omni.OMNI_BF16, fake, fake, 1 << 30, None)
    assert s == omni.OMNI_ERR_INVALID_ARG and b"NULL" in lib.omni_last_error()


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(4, 8)
    with pytest.raises(ValueError):
        omni.omni_router(x, torch.zeros(2, 8), torch.zeros(2, 8), 2)


def test_noalloc_schedule_rejects_before_touching_the_gpu():
    """omni_schedule_noalloc runs omni_schedule's checks, then refuses sizes
    whose sort buffers exceed its fixed scratch; all before any HIP call."""
    lib = omni.library()
    fake = ctypes.c_void_p(4096)  # never dereferenced
    s = lib.omni_schedule_noalloc(None, 4, 2, 100, 8, fake, fake, None, None)
    assert s == omni.OMNI_ERR_INVALID_ARG and b"NULL idx" in lib.omni_last_error()
    s = lib.omni_schedule_noalloc(fake, 4, 2, 100, 2**32 + 5, fake, fake, None, None)
    assert s == omni.OMNI_ERR_UNSUPPORTED and b"B =" in lib.omni_last_error()
    s = lib.omni_schedule_noalloc(fake, 4, 2, 100, 8, fake, None, None, None)
    assert s == omni.OMNI_ERR_INVALID_ARG and b"together" in lib.omni_last_error()
    # 16384 x 512 tasks need about 129 MiB of sort buffers: above the 80 MiB
    need = omni.omni_workspace_bytes(omni.OMNI_OP_SCHEDULE, L=16384, K=512, N=1700416, B=256)
    assert need > 80 << 20
    s = lib.omni_schedule_noalloc(fake, 16384, 512, 1700416, 256, fake, fake, None, None)
    assert s == omni.OMNI_ERR_UNSUPPORTED and b"scratch" in lib.omni_last_error()
    # the largest configured workload (16384 x 256 tasks) fits
    assert omni.omni_workspace_bytes(omni.OMNI_OP_SCHEDULE, L=16384, K=256, N=1700416,
                                     B=256) <= 80 << 20


def test_auto_assembly_workspace_and_validation():
    """omni_expert_forward_auto: the schedule's and the assembly's size rules,
    a workspace that holds either form, and rejections before any launch."""
    L, d, K, N, B = 4096, 2048, 128, 1700416, 128
    auto = omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_FORWARD_AUTO, L=L, d=d, K=K, N=N, B=B)
    blocked = omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_FORWARD_BLOCKED, L=L, d=d, K=K, N=N)
    per_task = omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_FORWARD, L=L, d=d, K=K, N=N, B=B)
    assert auto >= blocked and auto >= per_task + L * K * 4
    # fp32 inputs never take the blocked form: a smaller workspace
    f32 = omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_FORWARD_AUTO, L=L, d=d, K=K, N=N, B=B,
                                    dtype=omni.OMNI_F32)
    assert f32 < blocked
    for kw, st in ((dict(B=0), omni.OMNI_ERR_INVALID_ARG), (dict(B=2**31), omni.OMNI_ERR_UNSUPPORTED),
                   (dict(K=513), omni.OMNI_ERR_UNSUPPORTED), (dict(d=12), omni.OMNI_ERR_UNSUPPORTED)):
        args = dict(L=64, d=256, K=16, N=1024, B=16)
        args.update(kw)
        with pytest.raises(omni.OmniError) as e:
            omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_FORWARD_AUTO, **args)
        assert e.value.status == st
    lib = omni.library()
    fake = ctypes.c_void_p(4096)
    s = lib.omni_expert_forward_auto(fake, fake, fake, None, fake, 64, 256, 1024, 16, 16,
                                     omni.OMNI_BF16, fake, None, fake, 1 << 30, None)
    assert s == omni.OMNI_ERR_INVALID_ARG and b"NULL" in lib.omni_last_error()
    s = lib.omni_expert_forward_auto(fake, fake, fake, fake, fake, 64, 256, 1024, 16, 16,
                                     omni.OMNI_BF16, fake, None, fake, 16, None)
    assert s == omni.OMNI_ERR_WORKSPACE


def test_auto_backward_workspace_and_validation():
    """omni_expert_backward_auto: the per-task backward's size rules, a
    workspace that holds either form (the blocked one holds the per-task
    one's buffers), and rejections before any launch."""
    L, d, K, N = 4096, 2048, 128, 1700416
    auto = omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_BACKWARD_AUTO, L=L, d=d, K=K, N=N)
    blocked = omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_BACKWARD_BLOCKED, L=L, d=d, K=K, N=N)
    per_task = omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_BACKWARD, L=L, d=d, K=K, N=N)
    assert auto >= blocked + L * 4 and auto >= per_task
    # fp32 inputs, d % 256 != 0 or L above the blocked form's limit: the
    # per-task backward alone
    for kw in (dict(dtype=omni.OMNI_F32), dict(d=2112), dict(L=524288 + 64, K=2)):
        args = dict(L=L, d=d, K=K, N=N)
        args.update(kw)
        alone = omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_BACKWARD, **args)
        got = omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_BACKWARD_AUTO, **args)
        assert got == (alone + 255) // 256 * 256, kw
    for kw, st in ((dict(K=513), omni.OMNI_ERR_UNSUPPORTED), (dict(d=12), omni.OMNI_ERR_UNSUPPORTED),
                   (dict(N=0), omni.OMNI_ERR_INVALID_ARG)):
        args = dict(L=64, d=256, K=16, N=1024)
        args.update(kw)
        with pytest.raises(omni.OmniError) as e:
            omni.omni_workspace_bytes(omni.OMNI_OP_EXPERT_BACKWARD_AUTO, **args)
        assert e.value.status == st
    lib = omni.library()
    fake = ctypes.c_void_p(4096)
    s = lib.omni_expert_backward_auto(fake, fake, fake, fake, fake, None, 64, 256, 1024, 16,
                                      omni.OMNI_BF16, fake, fake, fake, fake, omni.OMNI_F32, fake,
                                      fake, None, fake, 1 << 30, None)
    assert s == omni.OMNI_ERR_INVALID_ARG and b"NULL" in lib.omni_last_error()
    s = lib.omni_expert_backward_auto(fake, fake, fake, fake, fake, fake, 64, 256, 1024, 16,
                                      omni.OMNI_BF16, fake, fake, fake, fake, 7, fake, fake, None,
                                      fake, 1 << 30, None)
    assert s == omni.OMNI_ERR_INVALID_ARG and b"grad_dt" in lib.omni_last_error()
    s = lib.omni_expert_backward_auto(fake, fake, fake, fake, fake, fake, 64, 256, 1024, 16,
                                      omni.OMNI_BF16, fake, fake, fake, fake, omni.OMNI_F32, fake,
                                      fake, None, fake, 16, None)
    assert s == omni.OMNI_ERR_WORKSPACE


def test_gather_probe_validation():
    lib = omni.library()
    fake = ctypes.c_void_p(4096)
    s = lib.omni_gather_probe(fake, 10, 24, fake, 5, fake, 1 << 20, None)
    assert s == omni.OMNI_ERR_UNSUPPORTED  # row bytes not a multiple of 16
    s = lib.omni_gather_probe(fake, 10, 64, fake, 5, fake, 16, None)
    assert s == omni.OMNI_ERR_WORKSPACE  # sink too small
    s = lib.omni_gather_probe(None, 10, 64, fake, 5, fake, 1 << 20, None)
    assert s == omni.OMNI_ERR_INVALID_ARG
