"""ctypes binding of libomni.so (include/omni.h), same names as the C ABI.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their device pointers and sizes go to the C entry points, and
the call is enqueued on torch's current HIP stream.  Outputs and workspaces
that the caller does not pass are allocated with torch (device memory is the
only thing PyTorch provides here).  Every step of the routed branch runs in
the library's HIP kernels; if the library is missing this module raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libomni.so")
_ABI_VERSION = 10

OMNI_OK, OMNI_ERR_INVALID_ARG, OMNI_ERR_UNSUPPORTED, OMNI_ERR_WORKSPACE, OMNI_ERR_HIP = range(5)
OMNI_F32, OMNI_BF16 = 0, 1
OMNI_OP_ROUTER, OMNI_OP_SCHEDULE, OMNI_OP_EXPERT_FORWARD = 0, 1, 2
OMNI_OP_EXPERT_BACKWARD, OMNI_OP_ROUTER_BACKWARD, OMNI_OP_SHARED_MLP = 3, 4, 5
OMNI_OP_DENSE_ROUTER, OMNI_OP_EXPERT_FORWARD_BLOCKED, OMNI_OP_EXPERT_BACKWARD_BLOCKED = 6, 7, 8
OMNI_OP_EXPERT_FORWARD_AUTO, OMNI_OP_EXPERT_BACKWARD_AUTO = 9, 10
EXPORTED = ("omni_router", "omni_schedule", "omni_schedule_noalloc", "omni_expert_forward", "omni_expert_forward_auto",
            "omni_expert_forward_blocked",
            "omni_expert_backward_blocked", "omni_expert_backward_auto",
            "omni_expert_forward_token_centric", "omni_expert_backward", "omni_router_backward",
            "omni_shared_mlp", "omni_dense_router", "omni_gather_probe", "omni_workspace_bytes",
            "omni_status_string",
            "omni_last_error", "omni_abi_version")


class OmniError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {detail} (status {status})")


_lib = None


def library() -> ctypes.CDLL:
    """Open libomni.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python -m atomic_expert_routing_amd.build` "
            "(there is no fallback path)")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    lib.omni_router.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int,
                                vp, vp, vp, vp, sz, vp]
    lib.omni_schedule.argtypes = [vp, i64, i64, i64, i64, vp, vp, vp, vp, sz, vp]
    lib.omni_schedule_noalloc.argtypes = [vp, i64, i64, i64, i64, vp, vp, vp, vp]
    lib.omni_expert_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                        i64, ctypes.c_int, vp, vp, sz, vp]
    lib.omni_expert_forward_auto.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                             ctypes.c_int, vp, vp, vp, sz, vp]
    lib.omni_expert_forward_blocked.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                                ctypes.c_int, vp, vp, sz, vp]
    lib.omni_expert_forward_token_centric.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                                      ctypes.c_int, vp, vp]
    lib.omni_expert_backward.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                         ctypes.c_int, vp, vp, vp, vp, ctypes.c_int, vp, vp,
                                         vp, sz, vp]
    lib.omni_expert_backward_auto.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                              ctypes.c_int, vp, vp, vp, vp, ctypes.c_int, vp, vp,
                                              vp, vp, sz, vp]
    lib.omni_expert_backward_blocked.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                                 ctypes.c_int, vp, vp, vp, vp, ctypes.c_int, vp,
                                                 vp, vp, sz, vp]
    lib.omni_router_backward.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                         ctypes.c_int, vp, vp, vp, vp, sz, vp]
    lib.omni_shared_mlp.argtypes = [vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, vp,
                                    ctypes.c_int, vp, sz, vp]
    lib.omni_dense_router.argtypes = [vp, vp, i64, i64, i64, i64, ctypes.c_int, vp, vp, vp, vp,
                                      sz, vp]
    lib.omni_gather_probe.argtypes = [vp, i64, i64, vp, i64, vp, sz, vp]
    lib.omni_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, i64, i64,
                                         ctypes.c_int, ctypes.POINTER(sz)]
    for f in ("omni_router", "omni_schedule", "omni_schedule_noalloc", "omni_expert_forward",
              "omni_expert_forward_auto", "omni_expert_forward_blocked",
              "omni_expert_backward_blocked", "omni_expert_backward_auto",
              "omni_expert_forward_token_centric", "omni_expert_backward",
              "omni_router_backward", "omni_shared_mlp", "omni_dense_router",
              "omni_gather_probe", "omni_workspace_bytes"):
        getattr(lib, f).restype = ctypes.c_int
    lib.omni_status_string.argtypes = [ctypes.c_int]
    lib.omni_status_string.restype = ctypes.c_char_p
    lib.omni_last_error.argtypes = []
    lib.omni_last_error.restype = ctypes.c_char_p
    lib.omni_abi_version.argtypes = []
    lib.omni_abi_version.restype = ctypes.c_int
    if lib.omni_abi_version() != _ABI_VERSION:
        raise RuntimeError(f"{_LIB_PATH}: ABI version {lib.omni_abi_version()} != {_ABI_VERSION}; rebuild")
    _lib = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != OMNI_OK:
        lib = library()
        raise OmniError(status, where, lib.omni_last_error().decode() or
                        lib.omni_status_string(status).decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return OMNI_BF16
    if t.dtype == torch.float32:
        return OMNI_F32
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def omni_workspace_bytes(op: int, L=1, d=8, Nr=1, Nc=1, K=1, N=1, B=1, dtype=OMNI_BF16) -> int:
    out = ctypes.c_size_t(0)
    _check(library().omni_workspace_bytes(op, L, d, Nr, Nc, K, N, B, dtype, ctypes.byref(out)),
           "omni_workspace_bytes")
    return out.value


def _workspace(ws, need: int, device) -> tuple[int, int]:
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    _dev(ws, "ws")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def omni_router(x, Wr, Wc, K: int, idx=None, score=None, gate=None, ws=None, stream=None):
    """Cartesian Product Router -> (idx [L,K] int32, score [L,K] f32, gate [L,K] f32)."""
    L, d = x.shape
    Nr, Nc = Wr.shape[0], Wc.shape[0]
    dt = _dtype_code(x)
    px = _dev(x, "x")
    pr = _dev(Wr, "Wr", x.dtype, (Nr, d))
    pc = _dev(Wc, "Wc", x.dtype, (Nc, d))
    kw = dict(device=x.device)
    idx = torch.empty((L, K), dtype=torch.int32, **kw) if idx is None else idx
    score = torch.empty((L, K), dtype=torch.float32, **kw) if score is None else score
    gate = torch.empty((L, K), dtype=torch.float32, **kw) if gate is None else gate
    pi = _dev(idx, "idx", torch.int32, (L, K))
    ps = _dev(score, "score", torch.float32, (L, K))
    pg = _dev(gate, "gate", torch.float32, (L, K))
    if ws is None:
        need = omni_workspace_bytes(OMNI_OP_ROUTER, L, d, Nr, Nc, K, Nr * Nc, 1, dt)
    else:
        need = 0
    pw, nw = _workspace(ws, need, x.device)
    _check(library().omni_router(px, pr, pc, L, d, Nr, Nc, K, dt, pi, ps, pg, pw, nw,
                                 _stream(stream)), "omni_router")
    return idx, score, gate


def omni_schedule(idx, N: int, B: int, perm=None, group_off=None, ws=None, stream=None,
                  token_order=None, tasks=True):
    """Expert-centric schedule -> (perm [L*K] int32, group_off [G+1] int32).

    token_order: None (not computed), True (allocate) or an [L] int32 tensor;
    when given, the tokens sorted by the group of their first expert are
    written there and returned as a third element.  tasks=False computes the
    token order alone (perm and group_off are returned as None).
    """
    L, K = idx.shape
    G = -(-N // B)
    pi = _dev(idx, "idx", torch.int32)
    kw = dict(device=idx.device, dtype=torch.int32)
    if tasks:
        perm = torch.empty((L * K,), **kw) if perm is None else perm
        group_off = torch.empty((G + 1,), **kw) if group_off is None else group_off
        pp = _dev(perm, "perm", torch.int32, (L * K,))
        po = _dev(group_off, "group_off", torch.int32, (G + 1,))
    else:
        perm = group_off = pp = po = None
    need = omni_workspace_bytes(OMNI_OP_SCHEDULE, L, 8, 1, 1, K, N, B) if ws is None else 0
    if token_order is True:
        token_order = torch.empty((L,), **kw)
    pt = None if token_order is None else _dev(token_order, "token_order", torch.int32, (L,))
    pw, nw = _workspace(ws, need, idx.device)
    _check(library().omni_schedule(pi, L, K, N, B, pp, po, pt, pw, nw, _stream(stream)),
           "omni_schedule")
    return (perm, group_off) if token_order is None else (perm, group_off, token_order)


def omni_schedule_noalloc(idx, N: int, B: int, perm=None, group_off=None, stream=None,
                          token_order=None, tasks=True):
    """omni_schedule with its sort buffers in the library's fixed per-GPU
    scratch array (no workspace argument; the C call allocates nothing).
    Same arguments and returns as omni_schedule without ws."""
    L, K = idx.shape
    G = -(-N // B)
    pi = _dev(idx, "idx", torch.int32)
    kw = dict(device=idx.device, dtype=torch.int32)
    if tasks:
        perm = torch.empty((L * K,), **kw) if perm is None else perm
        group_off = torch.empty((G + 1,), **kw) if group_off is None else group_off
        pp = _dev(perm, "perm", torch.int32, (L * K,))
        po = _dev(group_off, "group_off", torch.int32, (G + 1,))
    else:
        perm = group_off = pp = po = None
    if token_order is True:
        token_order = torch.empty((L,), **kw)
    pt = None if token_order is None else _dev(token_order, "token_order", torch.int32, (L,))
    _check(library().omni_schedule_noalloc(pi, L, K, N, B, pp, po, pt, _stream(stream)),
           "omni_schedule_noalloc")
    return (perm, group_off) if token_order is None else (perm, group_off, token_order)


def omni_expert_forward(x, W, V, idx, gate, perm, group_off, B: int, y=None, ws=None,
                        stream=None, token_order=None):
    """Dynamic Expert Assembly over the schedule (perm, group_off of group
    size B, from omni_schedule) -> y [L, d] float32.

    token_order (optional [L] int32, from omni_schedule) sets the order in
    which the output pass visits tokens; y does not depend on it."""
    L, d = x.shape
    N = W.shape[0]
    K = idx.shape[1]
    G = -(-N // B)
    dt = _dtype_code(x)
    px = _dev(x, "x")
    pW = _dev(W, "W", x.dtype, (N, d))
    pV = _dev(V, "V", x.dtype, (N, d))
    pi = _dev(idx, "idx", torch.int32, (L, K))
    pg = _dev(gate, "gate", torch.float32, (L, K))
    pp = _dev(perm, "perm", torch.int32, (L * K,))
    po = _dev(group_off, "group_off", torch.int32, (G + 1,))
    pt = None if token_order is None else _dev(token_order, "token_order", torch.int32, (L,))
    y = torch.empty((L, d), dtype=torch.float32, device=x.device) if y is None else y
    py = _dev(y, "y", torch.float32, (L, d))
    need = omni_workspace_bytes(OMNI_OP_EXPERT_FORWARD, L, d, 1, 1, K, N, B, dt) if ws is None else 0
    pw, nw = _workspace(ws, need, x.device)
    _check(library().omni_expert_forward(px, pW, pV, pi, pg, pp, po, pt, L, d, N, K, B, dt, py,
                                         pw, nw, _stream(stream)), "omni_expert_forward")
    return y


def omni_expert_forward_auto(x, W, V, idx, gate, B: int, y=None, ws=None, stream=None,
                             chosen=None):
    """Schedule and assembly in the form the device picks from a sample of the
    routing (the pages' schedule and the per-task passes, or the token order
    and the blocked form when the sampled tasks repeat their experts twice or
    more) -> y [L, d] float32.  chosen (optional [1] int32) receives 1 when
    the blocked form ran, else 0."""
    L, d = x.shape
    N = W.shape[0]
    K = idx.shape[1]
    dt = _dtype_code(x)
    args = (_dev(x, "x"), _dev(W, "W", x.dtype, (N, d)), _dev(V, "V", x.dtype, (N, d)),
            _dev(idx, "idx", torch.int32, (L, K)), _dev(gate, "gate", torch.float32, (L, K)))
    y = torch.empty((L, d), dtype=torch.float32, device=x.device) if y is None else y
    py = _dev(y, "y", torch.float32, (L, d))
    pc = None if chosen is None else _dev(chosen, "chosen", torch.int32, (1,))
    need = (omni_workspace_bytes(OMNI_OP_EXPERT_FORWARD_AUTO, L, d, 1, 1, K, N, B, dt)
            if ws is None else 0)
    pw, nw = _workspace(ws, need, x.device)
    _check(library().omni_expert_forward_auto(*args, L, d, N, K, B, dt, py, pc, pw, nw,
                                              _stream(stream)), "omni_expert_forward_auto")
    return y


def omni_expert_forward_blocked(x, W, V, idx, gate, token_order, y=None, ws=None, stream=None):
    """The assembly as dense products over blocks of 64 tokens of token_order
    and the union of their experts -> y [L, d] float32 (bf16 inputs)."""
    L, d = x.shape
    N = W.shape[0]
    K = idx.shape[1]
    dt = _dtype_code(x)
    px = _dev(x, "x")
    pW = _dev(W, "W", x.dtype, (N, d))
    pV = _dev(V, "V", x.dtype, (N, d))
    pi = _dev(idx, "idx", torch.int32, (L, K))
    pg = _dev(gate, "gate", torch.float32, (L, K))
    pt = _dev(token_order, "token_order", torch.int32, (L,))
    y = torch.empty((L, d), dtype=torch.float32, device=x.device) if y is None else y
    py = _dev(y, "y", torch.float32, (L, d))
    need = (omni_workspace_bytes(OMNI_OP_EXPERT_FORWARD_BLOCKED, L, d, 1, 1, K, N, 1, dt)
            if ws is None else 0)
    pw, nw = _workspace(ws, need, x.device)
    _check(library().omni_expert_forward_blocked(px, pW, pV, pi, pg, pt, L, d, N, K, dt, py, pw,
                                                 nw, _stream(stream)),
           "omni_expert_forward_blocked")
    return y


def omni_expert_forward_token_centric(x, W, V, idx, gate, y=None, stream=None):
    """Token-centric baseline of the assembly (no schedule) -> y [L, d] float32."""
    L, d = x.shape
    N = W.shape[0]
    K = idx.shape[1]
    dt = _dtype_code(x)
    px = _dev(x, "x")
    pW = _dev(W, "W", x.dtype, (N, d))
    pV = _dev(V, "V", x.dtype, (N, d))
    pi = _dev(idx, "idx", torch.int32, (L, K))
    pg = _dev(gate, "gate", torch.float32, (L, K))
    y = torch.empty((L, d), dtype=torch.float32, device=x.device) if y is None else y
    py = _dev(y, "y", torch.float32, (L, d))
    _check(library().omni_expert_forward_token_centric(px, pW, pV, pi, pg, L, d, N, K, dt, py,
                                                       _stream(stream)),
           "omni_expert_forward_token_centric")
    return y


def omni_expert_backward(x, W, V, idx, gate, dy, dx=None, dgate=None, uniq=None, n_uniq=None,
                         dW_rows=None, dV_rows=None, ws=None, stream=None,
                         grad_dtype=torch.float32):
    """Gradients of the expert assembly.

    Returns (dx [L,d] f32 (expert part), dgate [L,K] f32, uniq [U_cap] int32,
    n_uniq [1] int32, dW_rows [U_cap,d], dV_rows [U_cap,d]) with
    U_cap = min(N, L*K); only the first n_uniq entries / rows are defined.
    The gradient rows are float32 or bfloat16 (grad_dtype).
    """
    return _expert_backward(None, x, W, V, idx, gate, dy, dx, dgate, uniq, n_uniq, dW_rows,
                            dV_rows, ws, stream, grad_dtype)


def omni_expert_backward_auto(x, W, V, idx, gate, dy, dx=None, dgate=None, uniq=None,
                              n_uniq=None, dW_rows=None, dV_rows=None, ws=None, stream=None,
                              grad_dtype=torch.float32, chosen=None):
    """omni_expert_backward in the form the device picks by the forward's
    rule (per-task, or blocked over the tokens sorted by their first expert);
    same returns.  chosen (optional [1] int32) receives 1 when the blocked
    form ran, else 0."""
    return _expert_backward("auto", x, W, V, idx, gate, dy, dx, dgate, uniq, n_uniq, dW_rows,
                            dV_rows, ws, stream, grad_dtype, chosen)


def omni_expert_backward_blocked(x, W, V, idx, gate, dy, token_order, dx=None, dgate=None,
                                 uniq=None, n_uniq=None, dW_rows=None, dV_rows=None, ws=None,
                                 stream=None, grad_dtype=torch.float32):
    """omni_expert_backward with the per-token part over the blocked
    assembly's token blocks (token_order: [L] int32); same returns."""
    return _expert_backward(token_order, x, W, V, idx, gate, dy, dx, dgate, uniq, n_uniq,
                            dW_rows, dV_rows, ws, stream, grad_dtype)


def _expert_backward(token_order, x, W, V, idx, gate, dy, dx, dgate, uniq, n_uniq, dW_rows,
                     dV_rows, ws, stream, grad_dtype, chosen=None):
    L, d = x.shape
    N = W.shape[0]
    K = idx.shape[1]
    dt = _dtype_code(x)
    cap = min(N, L * K)
    f32, i32 = torch.float32, torch.int32
    kw = dict(device=x.device)
    dx = torch.empty((L, d), dtype=f32, **kw) if dx is None else dx
    dgate = torch.empty((L, K), dtype=f32, **kw) if dgate is None else dgate
    uniq = torch.empty((cap,), dtype=i32, **kw) if uniq is None else uniq
    n_uniq = torch.empty((1,), dtype=i32, **kw) if n_uniq is None else n_uniq
    gdt = dW_rows.dtype if dW_rows is not None else grad_dtype
    dW_rows = torch.empty((cap, d), dtype=gdt, **kw) if dW_rows is None else dW_rows
    dV_rows = torch.empty((cap, d), dtype=gdt, **kw) if dV_rows is None else dV_rows
    args = (_dev(x, "x"), _dev(W, "W", x.dtype, (N, d)), _dev(V, "V", x.dtype, (N, d)),
            _dev(idx, "idx", i32, (L, K)), _dev(gate, "gate", f32, (L, K)),
            _dev(dy, "dy", f32, (L, d)), L, d, N, K, dt, _dev(dx, "dx", f32, (L, d)),
            _dev(dgate, "dgate", f32, (L, K)), _dev(uniq, "uniq", i32, (cap,)),
            _dev(n_uniq, "n_uniq", i32, (1,)), _dtype_code(dW_rows),
            _dev(dW_rows, "dW_rows", gdt, (cap, d)), _dev(dV_rows, "dV_rows", gdt, (cap, d)))
    auto = isinstance(token_order, str)
    op = (OMNI_OP_EXPERT_BACKWARD_AUTO if auto else
          OMNI_OP_EXPERT_BACKWARD if token_order is None else OMNI_OP_EXPERT_BACKWARD_BLOCKED)
    need = omni_workspace_bytes(op, L, d, 1, 1, K, N, 1, dt) if ws is None else 0
    pw, nw = _workspace(ws, need, x.device)
    if auto:
        pc = None if chosen is None else _dev(chosen, "chosen", i32, (1,))
        _check(library().omni_expert_backward_auto(*args, pc, pw, nw, _stream(stream)),
               "omni_expert_backward_auto")
    elif token_order is None:
        _check(library().omni_expert_backward(*args, pw, nw, _stream(stream)),
               "omni_expert_backward")
    else:
        po = _dev(token_order, "token_order", i32, (L,))
        _check(library().omni_expert_backward_blocked(*args[:6], po, *args[6:], pw, nw,
                                                      _stream(stream)),
               "omni_expert_backward_blocked")
    return dx, dgate, uniq, n_uniq, dW_rows, dV_rows


def omni_router_backward(x, Wr, Wc, idx, gate, dgate, dx, dWr=None, dWc=None, ws=None,
                         stream=None):
    """Router gradients: adds the router part into dx (in place) and returns
    (dx, dWr [N_r,d] f32, dWc [N_c,d] f32)."""
    L, d = x.shape
    Nr, Nc = Wr.shape[0], Wc.shape[0]
    K = idx.shape[1]
    dt = _dtype_code(x)
    f32 = torch.float32
    dWr = torch.empty((Nr, d), dtype=f32, device=x.device) if dWr is None else dWr
    dWc = torch.empty((Nc, d), dtype=f32, device=x.device) if dWc is None else dWc
    args = (_dev(x, "x"), _dev(Wr, "Wr", x.dtype, (Nr, d)), _dev(Wc, "Wc", x.dtype, (Nc, d)),
            _dev(idx, "idx", torch.int32, (L, K)), _dev(gate, "gate", f32, (L, K)),
            _dev(dgate, "dgate", f32, (L, K)), L, d, Nr, Nc, K, dt, _dev(dx, "dx", f32, (L, d)),
            _dev(dWr, "dWr", f32, (Nr, d)), _dev(dWc, "dWc", f32, (Nc, d)))
    need = omni_workspace_bytes(OMNI_OP_ROUTER_BACKWARD, L, d, Nr, Nc, K, Nr * Nc, 1, dt) \
        if ws is None else 0
    pw, nw = _workspace(ws, need, x.device)
    _check(library().omni_router_backward(*args, pw, nw, _stream(stream)), "omni_router_backward")
    return dx, dWr, dWc


def omni_shared_mlp(x, Wg, Wu, Wd, y=None, accumulate=False, ws=None, stream=None):
    """Shared dense MLP: y = MLP(x), or y += MLP(x) with accumulate -> y [L, d] f32."""
    L, d = x.shape
    F = Wg.shape[0]
    dt = _dtype_code(x)
    y = torch.empty((L, d), dtype=torch.float32, device=x.device) if y is None else y
    args = (_dev(x, "x"), _dev(Wg, "Wg", x.dtype, (F, d)), _dev(Wu, "Wu", x.dtype, (F, d)),
            _dev(Wd, "Wd", x.dtype, (d, F)), L, d, F, dt, _dev(y, "y", torch.float32, (L, d)),
            1 if accumulate else 0)
    need = omni_workspace_bytes(OMNI_OP_SHARED_MLP, L, d, 1, 1, 1, F, 1, dt) if ws is None else 0
    pw, nw = _workspace(ws, need, x.device)
    _check(library().omni_shared_mlp(*args, pw, nw, _stream(stream)), "omni_shared_mlp")
    return y


def omni_dense_router(x, Wn, K: int, idx=None, score=None, gate=None, ws=None, stream=None):
    """Fully connected router over all N experts -> (idx, score, gate), each [L, K]."""
    L, d = x.shape
    N = Wn.shape[0]
    dt = _dtype_code(x)
    kw = dict(device=x.device)
    idx = torch.empty((L, K), dtype=torch.int32, **kw) if idx is None else idx
    score = torch.empty((L, K), dtype=torch.float32, **kw) if score is None else score
    gate = torch.empty((L, K), dtype=torch.float32, **kw) if gate is None else gate
    args = (_dev(x, "x"), _dev(Wn, "Wn", x.dtype, (N, d)), L, d, N, K, dt,
            _dev(idx, "idx", torch.int32, (L, K)), _dev(score, "score", torch.float32, (L, K)),
            _dev(gate, "gate", torch.float32, (L, K)))
    need = omni_workspace_bytes(OMNI_OP_DENSE_ROUTER, L, d, 1, 1, K, N, 1, dt) if ws is None else 0
    pw, nw = _workspace(ws, need, x.device)
    _check(library().omni_dense_router(*args, pw, nw, _stream(stream)), "omni_dense_router")
    return idx, score, gate


def omni_gather_probe(A, rows, sink=None, stream=None):
    """Measurement aid: read the listed rows of A (2-D, contiguous) in the
    assembly's access pattern; returns the checksum sink."""
    n = rows.numel()
    row_bytes = A.shape[1] * A.element_size()
    need = 256 * min(8192, max(1, -(-n // 32)))
    sink = torch.empty(need, dtype=torch.float32, device=A.device) if sink is None else sink
    _check(library().omni_gather_probe(_dev(A, "A"), A.shape[0], row_bytes,
                                       _dev(rows, "rows", torch.int32), n,
                                       _dev(sink, "sink", torch.float32), sink.numel(),
                                       _stream(stream)), "omni_gather_probe")
    return sink


class RoutedBranch:
    """Preallocated outputs and workspaces for repeated routed-branch forwards.

    One instance per (shape, dtype): `forward(x, Wr, Wc, W, V)` enqueues the
    three C calls on the current stream and allocates nothing.

    assembly="auto" (the default) runs omni_router then
    omni_expert_forward_auto: the device picks, per call, the pages' schedule
    and the per-task passes (spread-out routing) or the token order and the
    blocked form (routing whose tasks pile onto few experts), and writes its
    choice to `self.chosen` (1 = blocked); `perm` and `group_off` are not
    filled in this mode (the schedule stays in the workspace).  assembly="expert_centric" always runs the
    per-task passes (omni_expert_forward); with token_order=True the schedule
    also sorts the tokens by their first expert's group and the output pass
    follows that order.  assembly="blocked" always runs
    omni_expert_forward_blocked over that order.
    """

    def __init__(self, L, d, Nr, Nc, K, B, dtype=torch.bfloat16, device="cuda",
                 token_order=False, assembly="auto"):
        self.L, self.d, self.Nr, self.Nc, self.K, self.B = L, d, Nr, Nc, K, B
        self.N = Nr * Nc
        self.G = -(-self.N // B)
        dt = OMNI_BF16 if dtype == torch.bfloat16 else OMNI_F32
        i32, f32 = torch.int32, torch.float32
        kw = dict(device=device)
        self.idx = torch.empty((L, K), dtype=i32, **kw)
        self.score = torch.empty((L, K), dtype=f32, **kw)
        self.gate = torch.empty((L, K), dtype=f32, **kw)
        self.perm = torch.empty((L * K,), dtype=i32, **kw)
        self.group_off = torch.empty((self.G + 1,), dtype=i32, **kw)
        self.y = torch.empty((L, d), dtype=f32, **kw)
        self.chosen = torch.zeros((1,), dtype=i32, **kw)
        if assembly not in ("auto", "expert_centric", "blocked"):
            raise ValueError(f"unknown assembly {assembly!r}")
        self.assembly = assembly
        token_order = (token_order and assembly == "expert_centric") or assembly == "blocked"
        self.token_order = torch.empty((L,), dtype=i32, **kw) if token_order else None
        op = {"auto": OMNI_OP_EXPERT_FORWARD_AUTO, "blocked": OMNI_OP_EXPERT_FORWARD_BLOCKED,
              "expert_centric": OMNI_OP_EXPERT_FORWARD}[assembly]
        sizes = [omni_workspace_bytes(OMNI_OP_ROUTER, L, d, Nr, Nc, K, self.N, B, dt),
                 omni_workspace_bytes(OMNI_OP_SCHEDULE, L, d, Nr, Nc, K, self.N, B, dt),
                 omni_workspace_bytes(op, L, d, Nr, Nc, K, self.N, B, dt)]
        # the three calls run in order on one stream, so they share one workspace
        self.ws = torch.empty(max(sizes), dtype=torch.uint8, **kw)

    def router(self, x, Wr, Wc, stream=None):
        return omni_router(x, Wr, Wc, self.K, self.idx, self.score, self.gate, self.ws, stream)

    def schedule(self, stream=None):
        # the automatic assembly schedules inside its own call (in the form it
        # picks); the blocked assembly reads only the token order
        if self.assembly == "auto":
            return None
        return omni_schedule(self.idx, self.N, self.B, self.perm, self.group_off, self.ws, stream,
                             self.token_order, tasks=self.assembly != "blocked")

    def expert_forward(self, x, W, V, stream=None):
        if self.assembly == "auto":
            return omni_expert_forward_auto(x, W, V, self.idx, self.gate, self.B, self.y,
                                            self.ws, stream, self.chosen)
        if self.assembly == "blocked":
            return omni_expert_forward_blocked(x, W, V, self.idx, self.gate, self.token_order,
                                               self.y, self.ws, stream)
        return omni_expert_forward(x, W, V, self.idx, self.gate, self.perm, self.group_off, self.B,
                                   self.y, self.ws, stream, self.token_order)

    def forward(self, x, Wr, Wc, W, V, stream=None):
        self.router(x, Wr, Wc, stream)
        self.schedule(stream)
        return self.expert_forward(x, W, V, stream)

    def capture(self, x, Wr, Wc, W, V):
        """Record one forward (router, schedule, assembly) as a HIP graph over
        these input tensors and this instance's buffers; replay() reruns it.
        The library allocates nothing and issues no memset, so the three
        calls capture as plain kernel nodes."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # warm-up outside the capture
            self.forward(x, Wr, Wc, W, V)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.forward(x, Wr, Wc, W, V)
        torch.cuda.synchronize()
        return self.graph

    def replay(self):
        self.graph.replay()
        return self.y
