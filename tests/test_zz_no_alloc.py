"""omni_schedule_noalloc (the schedule with its sort buffers in the
library's fixed per-GPU scratch array) against omni_schedule with a caller
workspace: the same perm, group_off and token order, bit for bit, on two
calls in a row, the second with a smaller input, and the second on a side
stream."""

import numpy as np
import pytest
import torch

from atomic_expert_routing_amd import omni
from oracle import omni_oracle as O

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    omni.library()  # fails loudly if the HIP library is missing


def random_ids(L, K, N, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randint(0, N, (L, K), generator=g, device="cuda", dtype=torch.int64).to(torch.int32)


def both(idx, N, B, stream=None):
    ref = omni.omni_schedule(idx, N, B, token_order=True, stream=stream)
    got = omni.omni_schedule_noalloc(idx, N, B, token_order=True, stream=stream)
    torch.cuda.synchronize()
    for name, a, b in zip(("perm", "group_off", "token_order"), ref, got):
        assert torch.equal(a, b), f"{name} differs"
    return got


def test_noalloc_schedule_matches_the_workspace_schedule_on_two_calls():
    # first call: 4096 tokens x K = 128 over 1.7M experts, groups of 128
    L, K, N, B = 4096, 128, 1304 * 1304, 128
    say(f"case noalloc first call L={L} K={K} N={N} B={B}")
    both(random_ids(L, K, N, 1), N, B)
    # second call, smaller, on a side stream: the scratch keeps the first
    # call's contents, which must not leak into this result
    L, K, N, B = 300, 37, 2500, 3
    say(f"case noalloc second call L={L} K={K} N={N} B={B} (side stream)")
    idx = random_ids(L, K, N, 2)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        perm, off, order = both(idx, N, B, stream=side)
    torch.cuda.synchronize()
    ids = idx.cpu().numpy().astype(np.int64)
    perm_o, off_o = O.schedule(ids, N, B)
    assert (perm.cpu().numpy() == perm_o).all() and (off.cpu().numpy() == off_o).all()
    assert (order.cpu().numpy() == O.token_order(ids, B)).all()


def test_noalloc_schedule_at_the_largest_configured_task_count():
    L, K, N, B = 16384, 256, 1304 * 1304, 256
    say(f"case noalloc L={L} K={K} N={N} B={B}")
    both(random_ids(L, K, N, 3), N, B)


def test_noalloc_schedule_refuses_sizes_beyond_its_scratch():
    L, K, N, B = 16384, 512, 1304 * 1304, 256  # 8.4M tasks: above the fixed scratch
    idx = torch.zeros((L, K), dtype=torch.int32, device="cuda")
    perm = torch.full((L * K,), -7, dtype=torch.int32, device="cuda")
    off = torch.full((-(-N // B) + 1,), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(omni.OmniError) as e:
        omni.omni_schedule_noalloc(idx, N, B, perm, off)
    assert e.value.status == omni.OMNI_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (perm == -7).all() and (off == -7).all()  # nothing was launched
