"""ctypes binding of libss (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libss.so")
_lib = None

F32, BF16 = 0, 1
DISC_DT, DISC_ZOH = 0, 1
ABI_VERSION = 12
EXPORTS = ("ss_abi_version", "ss_status_string", "ss_fwd", "ss_fwd_ex", "ss_fwd_noalloc", "ss_fwd_conv",
           "ss_fwd_workspace_size", "ss_workspace_status", "ss_step", "ss_step_ex",
           "ss_bwd_workspace_size", "ss_bwd", "ss_proj", "ss_proj_conv")
SS_ERR_SPLIT_WAIT = 9


class FwdOptions(ctypes.Structure):
    """ss_fwd_options: kernel 0 automatic / 1 sequential / 2 time-chunked / 3 state-parallel;
    chunk_len 0, 4, 8; discretization 0 (input term dt*B) / 1 (exact zero-order hold);
    chunk_rows 0 (automatic), 16, 12 or 32 time chunks per workgroup tile; split_parts 0
    (automatic), 1 (never) or 2..16 sequence parts for the time-chunked kernel; workspace and
    workspace_bytes: the caller's device memory for the split (or NULL); split_wait_limit:
    0 default, n > 0 polls, < 0 every hand-off wait gives up (testing)."""
    _fields_ = [("kernel", ctypes.c_int), ("chunk_len", ctypes.c_int),
                ("discretization", ctypes.c_int), ("chunk_rows", ctypes.c_int),
                ("split_parts", ctypes.c_int), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("split_wait_limit", ctypes.c_int)]


class SSError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {status_string(status)}")


def lib_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libss.so (built in-tree by __graft_entry__.build()); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.ss_abi_version.restype = i32
    lib.ss_abi_version.argtypes = []
    lib.ss_status_string.restype = ctypes.c_char_p
    lib.ss_status_string.argtypes = [i32]
    lib.ss_fwd.restype = i32
    lib.ss_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, i64, i64, i64, i64, i32, vp]
    lib.ss_fwd_ex.restype = i32
    lib.ss_fwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, i64, i64, i64, i64, i32,
                              ctypes.POINTER(FwdOptions), vp]
    lib.ss_fwd_noalloc.restype = i32
    lib.ss_fwd_noalloc.argtypes = lib.ss_fwd_ex.argtypes
    lib.ss_fwd_conv.restype = i32
    lib.ss_fwd_conv.argtypes = [vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp,
                                i64, i64, i64, i64, i32, ctypes.POINTER(FwdOptions), vp]
    lib.ss_fwd_workspace_size.restype = i32
    lib.ss_fwd_workspace_size.argtypes = [i64, i64, i64, i64, i32, ctypes.POINTER(FwdOptions),
                                          ctypes.POINTER(ctypes.c_size_t)]
    lib.ss_workspace_status.restype = i32
    lib.ss_workspace_status.argtypes = [vp, ctypes.c_size_t, vp, vp]
    lib.ss_step.restype = i32
    lib.ss_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i64, i64, i64, i32, vp]
    lib.ss_step_ex.restype = i32
    lib.ss_step_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i64, i64, i64, i32, i32, vp]
    lib.ss_bwd_workspace_size.restype = ctypes.c_size_t
    lib.ss_bwd_workspace_size.argtypes = [i64, i64, i64, i64]
    lib.ss_bwd.restype = i32
    lib.ss_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp,
                           vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                           i64, i64, i64, i64, i32, vp]
    lib.ss_proj.restype = i32
    lib.ss_proj.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp]
    lib.ss_proj_conv.restype = i32
    lib.ss_proj_conv.argtypes = [vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp]
    if lib.ss_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{_LIB_PATH} has ABI version {lib.ss_abi_version()}, this binding "
                           f"needs {ABI_VERSION}: rebuild it")
    _lib = lib
    return lib


def status_string(s: int) -> str:
    return load_library().ss_status_string(int(s)).decode()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _in_dtype(*ts) -> int:
    kinds = {t.dtype for t in ts if t is not None}
    if kinds == {torch.float32}:
        return F32
    if kinds == {torch.bfloat16}:
        return BF16
    raise TypeError(f"u, delta, z, B, C must all be float32 or all bfloat16, got {kinds}")


def _check(t, name, device, dtype=None, shape=None):
    if t is None:
        return
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a device tensor on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _options(kernel=0, chunk_len=0, zoh=False, chunk_rows=0, split_parts=0, workspace=None,
             split_wait_limit=0):
    ws = None if workspace is None else workspace
    return FwdOptions(int(kernel), int(chunk_len), DISC_ZOH if zoh else DISC_DT, int(chunk_rows),
                      int(split_parts), None if ws is None else ws.data_ptr(),
                      0 if ws is None else ws.numel() * ws.element_size(), int(split_wait_limit))


def fwd_workspace_size(batch, seqlen, dim, dstate, dtype=torch.float32, kernel=0, chunk_len=0,
                       zoh=False, chunk_rows=0, split_parts=0) -> int:
    """Bytes of workspace (``ss_fwd_workspace_size``) a forward call with these sizes and
    options uses on the current device (0: its plan does not split the sequences)."""
    opt = _options(kernel, chunk_len, zoh, chunk_rows, split_parts)
    out = ctypes.c_size_t(0)
    dt = BF16 if dtype == torch.bfloat16 else F32
    rc = load_library().ss_fwd_workspace_size(batch, seqlen, dim, dstate, dt, ctypes.byref(opt),
                                              ctypes.byref(out))
    if rc != 0:
        raise SSError(rc, "ss_fwd_workspace_size")
    return int(out.value)


def workspace_status(workspace, stream=None):
    """``ss_workspace_status``: (status, give-ups) of the most recent split call that used
    this workspace. The library enqueues the count into a device word; reading it here waits
    for the stream. status is SS_ERR_SPLIT_WAIT (9) when a wait gave up, else 0."""
    n = torch.empty(1, dtype=torch.int32, device=workspace.device)  # (overwritten by the copy)
    rc = load_library().ss_workspace_status(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                            _ptr(n), _stream(workspace.device, stream))
    if rc != 0:
        raise SSError(rc, "ss_workspace_status")
    torch.cuda.synchronize(workspace.device)  # (the copy runs on `stream`, not torch's current one)
    count = int(n.item())
    return (SS_ERR_SPLIT_WAIT if count else 0), count


def _fwd_workspace(workspace, dev, batch, L, dim, N, dtype, **opt):
    """The workspace tensor of a forward call: the given one, none (False), or, for None, a
    new uint8 device tensor of the size the library asks for (None when it needs none)."""
    if workspace is False:
        return None
    if workspace is not None:
        _check(workspace, "workspace", dev, torch.uint8)
        return workspace
    need = fwd_workspace_size(batch, L, dim, N, dtype, **opt)
    return torch.empty(need, dtype=torch.uint8, device=dev) if need > 0 else None


def fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, y=None,
        last_state=None, return_last_state=True, stream=None, kernel=0, chunk_len=0, h0=None,
        zoh=False, chunk_rows=0, split_parts=0, workspace=None, split_wait_limit=0):
    """Selective-scan forward (``ss_fwd_ex``). u, delta, z: (batch, L, dim); B, C: (batch, L,
    N); A: (dim, N) fp32; D, delta_bias: (dim,) fp32; h0: (batch, dim, N) fp32 initial state
    or None; zoh: exact zero-order-hold input term. workspace: a uint8 device tensor for the
    sequence split, False for none (no split), or None to allocate one of the size
    ``fwd_workspace_size`` gives for this call. Returns y (fp32) and, unless
    return_last_state is False, the final state (batch, dim, N) fp32."""
    dev = u.device
    batch, L, dim = u.shape
    N = A.shape[1]
    dt = _in_dtype(u, delta, B, C, z)
    _check(u, "u", dev)
    _check(delta, "delta", dev, shape=u.shape)
    _check(z, "z", dev, shape=u.shape)
    _check(B, "B", dev, shape=(batch, L, N))
    _check(C, "C", dev, shape=(batch, L, N))
    _check(A, "A", dev, torch.float32, (dim, N))
    _check(D, "D", dev, torch.float32, (dim,))
    _check(delta_bias, "delta_bias", dev, torch.float32, (dim,))
    _check(h0, "h0", dev, torch.float32, (batch, dim, N))
    if y is None:
        y = torch.empty((batch, L, dim), dtype=torch.float32, device=dev)
    _check(y, "y", dev, torch.float32, (batch, L, dim))
    if last_state is None and return_last_state:
        last_state = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    _check(last_state, "last_state", dev, torch.float32, (batch, dim, N))
    lib = load_library()
    plan = dict(kernel=kernel, chunk_len=chunk_len, zoh=zoh, chunk_rows=chunk_rows, split_parts=split_parts)
    ws = _fwd_workspace(workspace, dev, batch, L, dim, N, u.dtype, **plan)
    opt = _options(workspace=ws, split_wait_limit=split_wait_limit, **plan)
    rc = lib.ss_fwd_ex(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                       int(bool(softplus)), _ptr(y), _ptr(last_state), _ptr(h0), batch, L, dim, N, dt,
                       ctypes.byref(opt), _stream(dev, stream))
    if rc != 0:
        raise SSError(rc, "ss_fwd")
    return (y, last_state) if return_last_state else y


def fwd_noalloc(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, y=None,
                last_state=None, stream=None, kernel=0, chunk_len=0, h0=None, zoh=False, chunk_rows=0,
                split_parts=0):
    """``ss_fwd_noalloc``: ``fwd`` with the sequence split's scratch in the library's fixed
    per-device array instead of a workspace (y and last_state must be given to allocate
    nothing here either). Returns (y, last_state)."""
    dev = u.device
    batch, L, dim = u.shape
    N = A.shape[1]
    dt = _in_dtype(u, delta, B, C, z)
    for t, name in ((u, "u"), (delta, "delta"), (z, "z"), (B, "B"), (C, "C"), (h0, "h0")):
        _check(t, name, dev)
    _check(A, "A", dev, torch.float32, (dim, N))
    if y is None:
        y = torch.empty((batch, L, dim), dtype=torch.float32, device=dev)
    if last_state is None:
        last_state = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    _check(y, "y", dev, torch.float32, (batch, L, dim))
    _check(last_state, "last_state", dev, torch.float32, (batch, dim, N))
    opt = _options(kernel, chunk_len, zoh, chunk_rows, split_parts)
    rc = load_library().ss_fwd_noalloc(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                       _ptr(delta_bias), int(bool(softplus)), _ptr(y), _ptr(last_state),
                                       _ptr(h0), batch, L, dim, N, dt, ctypes.byref(opt), _stream(dev, stream))
    if rc != 0:
        raise SSError(rc, "ss_fwd_noalloc")
    return y, last_state


def fwd_plain(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, y=None,
              last_state=None, stream=None):
    """``ss_fwd`` itself (no options, no workspace, never split). Returns (y, last_state)."""
    dev = u.device
    batch, L, dim = u.shape
    N = A.shape[1]
    dt = _in_dtype(u, delta, B, C, z)
    for t, name in ((u, "u"), (delta, "delta"), (z, "z"), (B, "B"), (C, "C")):
        _check(t, name, dev)
    _check(A, "A", dev, torch.float32, (dim, N))
    if y is None:
        y = torch.empty((batch, L, dim), dtype=torch.float32, device=dev)
    if last_state is None:
        last_state = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    _check(y, "y", dev, torch.float32, (batch, L, dim))
    _check(last_state, "last_state", dev, torch.float32, (batch, dim, N))
    rc = load_library().ss_fwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                               _ptr(delta_bias), int(bool(softplus)), _ptr(y), _ptr(last_state), batch, L,
                               dim, N, dt, _stream(dev, stream))
    if rc != 0:
        raise SSError(rc, "ss_fwd")
    return y, last_state


def fwd_conv(x, conv_w, delta, A, B, C, conv_b=None, conv_state=None, D=None, z=None,
             delta_bias=None, softplus=True, y=None, last_state=None, h0=None, u_out=None,
             stream=None, kernel=0, chunk_len=0, zoh=False, chunk_rows=0, split_parts=0,
             workspace=None):
    """Forward with the fused prologue (``ss_fwd_conv``): u = silu(causal depthwise
    conv1d(x) + conv_b), then the scan of ``fwd`` on it. x: (batch, L, dim); conv_w
    (dim, K) fp32, K <= 4; conv_b (dim,) fp32 or None; conv_state (batch, dim, K-1) fp32 or
    None (the K-1 inputs before the sequence, oldest first). u_out: None, True (allocate),
    or an fp32 (batch, L, dim) tensor that receives u. Returns (y, last_state) or, with
    u_out, (y, last_state, u)."""
    dev = x.device
    batch, L, dim = x.shape
    N = A.shape[1]
    K = conv_w.shape[1] if conv_w.dim() == 2 else 0
    dt = _in_dtype(x, delta, B, C, z)
    _check(x, "x", dev)
    _check(conv_w, "conv_w", dev, torch.float32, (dim, K))
    _check(conv_b, "conv_b", dev, torch.float32, (dim,))
    _check(conv_state, "conv_state", dev, torch.float32, (batch, dim, K - 1))
    _check(delta, "delta", dev, shape=x.shape)
    _check(z, "z", dev, shape=x.shape)
    _check(B, "B", dev, shape=(batch, L, N))
    _check(C, "C", dev, shape=(batch, L, N))
    _check(A, "A", dev, torch.float32, (dim, N))
    _check(D, "D", dev, torch.float32, (dim,))
    _check(delta_bias, "delta_bias", dev, torch.float32, (dim,))
    _check(h0, "h0", dev, torch.float32, (batch, dim, N))
    f = dict(dtype=torch.float32, device=dev)
    if y is None:
        y = torch.empty((batch, L, dim), **f)
    _check(y, "y", dev, torch.float32, (batch, L, dim))
    if last_state is None:
        last_state = torch.empty((batch, dim, N), **f)
    _check(last_state, "last_state", dev, torch.float32, (batch, dim, N))
    want_u = u_out is not None and u_out is not False
    if u_out is True:
        u_out = torch.empty((batch, L, dim), **f)
    if not want_u:
        u_out = None
    _check(u_out, "u_out", dev, torch.float32, (batch, L, dim))
    plan = dict(kernel=kernel, chunk_len=chunk_len, zoh=zoh, chunk_rows=chunk_rows, split_parts=split_parts)
    ws = _fwd_workspace(workspace, dev, batch, L, dim, N, x.dtype, **plan)
    opt = _options(workspace=ws, **plan)
    rc = load_library().ss_fwd_conv(_ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), K, _ptr(delta),
                                    _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                                    int(bool(softplus)), _ptr(y), _ptr(last_state), _ptr(h0), _ptr(u_out),
                                    batch, L, dim, N, dt, ctypes.byref(opt), _stream(dev, stream))
    if rc != 0:
        raise SSError(rc, "ss_fwd_conv")
    return (y, last_state, u_out) if want_u else (y, last_state)


def step(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, y=None,
         stream=None, zoh=False):
    """One decode step (``ss_step``; ``ss_step_ex`` with zoh); state (batch, dim, N) fp32 is
    updated in place. u, delta, z: (batch, dim); B, C: (batch, N). Returns y (batch, dim)."""
    dev = state.device
    batch, dim, N = state.shape
    dt = _in_dtype(u, delta, B, C, z)
    _check(state, "state", dev, torch.float32)
    _check(u, "u", dev, shape=(batch, dim))
    _check(delta, "delta", dev, shape=(batch, dim))
    _check(z, "z", dev, shape=(batch, dim))
    _check(B, "B", dev, shape=(batch, N))
    _check(C, "C", dev, shape=(batch, N))
    _check(A, "A", dev, torch.float32, (dim, N))
    _check(D, "D", dev, torch.float32, (dim,))
    _check(delta_bias, "delta_bias", dev, torch.float32, (dim,))
    if y is None:
        y = torch.empty((batch, dim), dtype=torch.float32, device=dev)
    _check(y, "y", dev, torch.float32, (batch, dim))
    args = (_ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
            _ptr(delta_bias), int(bool(softplus)), _ptr(y), batch, dim, N, dt)
    lib = load_library()
    if zoh:
        rc = lib.ss_step_ex(*args, DISC_ZOH, _stream(dev, stream))
    else:
        rc = lib.ss_step(*args, _stream(dev, stream))
    if rc != 0:
        raise SSError(rc, "ss_step")
    return y


def bwd_workspace_size(batch, seqlen, dim, dstate) -> int:
    return int(load_library().ss_bwd_workspace_size(batch, seqlen, dim, dstate))


def bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, softplus=True, h0=None,
        dlast=None, stream=None, workspace=None, out=None):
    """Backward of ``fwd`` (``ss_bwd``; input term dt*B) for dL/dy = dy (batch, L, dim)
    fp32 and dL/dlast_state = dlast (batch, dim, N) fp32 or None.

    Returns a dict of fp32 device tensors: du, ddelta, dz (batch, L, dim) [dz None without
    z]; dA (dim, N); dB, dC (batch, L, N); dD, ddelta_bias (dim,) [None when D / delta_bias
    is None]; dh0 (batch, dim, N). ``workspace``: a uint8 device tensor of at least
    bwd_workspace_size() bytes, allocated here when None. ``out``: a dict like the returned
    one whose tensors are written instead of new ones (reuse across calls)."""
    dev = u.device
    batch, L, dim = u.shape
    N = A.shape[1]
    dt = _in_dtype(u, delta, B, C, z)
    _check(u, "u", dev)
    _check(delta, "delta", dev, shape=u.shape)
    _check(z, "z", dev, shape=u.shape)
    _check(B, "B", dev, shape=(batch, L, N))
    _check(C, "C", dev, shape=(batch, L, N))
    _check(A, "A", dev, torch.float32, (dim, N))
    _check(D, "D", dev, torch.float32, (dim,))
    _check(delta_bias, "delta_bias", dev, torch.float32, (dim,))
    _check(h0, "h0", dev, torch.float32, (batch, dim, N))
    _check(dy, "dy", dev, torch.float32, (batch, L, dim))
    _check(dlast, "dlast", dev, torch.float32, (batch, dim, N))
    f = dict(dtype=torch.float32, device=dev)
    if out is not None:
        shapes = dict(du=(batch, L, dim), ddelta=(batch, L, dim), dz=(batch, L, dim), dA=(dim, N),
                      dB=(batch, L, N), dC=(batch, L, N), dD=(dim,), ddelta_bias=(dim,),
                      dh0=(batch, dim, N))
        for k, shape in shapes.items():
            _check(out.get(k), k, dev, torch.float32, shape)
        for k in ("du", "ddelta", "dA", "dB", "dC") + (("dz",) if z is not None else ()):
            if out.get(k) is None:
                raise ValueError(f"out[{k!r}] is required")
    else:
        out = dict(du=torch.empty((batch, L, dim), **f), ddelta=torch.empty((batch, L, dim), **f),
                   dz=torch.empty((batch, L, dim), **f) if z is not None else None,
                   dA=torch.empty((dim, N), **f), dB=torch.empty((batch, L, N), **f),
                   dC=torch.empty((batch, L, N), **f),
                   dD=torch.empty((dim,), **f) if D is not None else None,
                   ddelta_bias=torch.empty((dim,), **f) if delta_bias is not None else None,
                   dh0=torch.empty((batch, dim, N), **f))
    lib = load_library()
    need = int(lib.ss_bwd_workspace_size(batch, L, dim, N))
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    _check(workspace, "workspace", dev, torch.uint8)
    rc = lib.ss_bwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                    _ptr(delta_bias), int(bool(softplus)), _ptr(h0), _ptr(dy), _ptr(dlast),
                    _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dB"]),
                    _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dz"]), _ptr(out["ddelta_bias"]),
                    _ptr(out["dh0"]), _ptr(workspace), workspace.numel(), batch, L, dim, N, dt,
                    _stream(dev, stream))
    if rc != 0:
        raise SSError(rc, "ss_bwd")
    return out


def _proj_outputs(u, W_x, W_dt, rank, delta_raw, B, C):
    dev = u.device
    batch, L, dim = u.shape
    N = (W_x.shape[0] - rank) // 2
    tdt = u.dtype
    _check(u, "u", dev)
    _check(W_x, "W_x", dev, tdt, (rank + 2 * N, dim))
    _check(W_dt, "W_dt", dev, tdt, (dim, rank))
    if delta_raw is None:
        delta_raw = torch.empty((batch, L, dim), dtype=tdt, device=dev)
    if B is None:
        B = torch.empty((batch, L, N), dtype=tdt, device=dev)
    if C is None:
        C = torch.empty((batch, L, N), dtype=tdt, device=dev)
    _check(delta_raw, "delta_raw", dev, tdt, (batch, L, dim))
    _check(B, "B", dev, tdt, (batch, L, N))
    _check(C, "C", dev, tdt, (batch, L, N))
    return N, delta_raw, B, C


def proj(u, W_x, W_dt, rank, delta_raw=None, B=None, C=None, stream=None):
    """Input projections (``ss_proj``): for every token, xp = W_x u_t, delta_raw = W_dt
    xp[:rank], B = xp[rank:rank+N], C = xp[rank+N:]. u: (batch, L, dim); W_x: (rank + 2N,
    dim); W_dt: (dim, rank); all float32 or all bfloat16. Returns (delta_raw, B, C) in the
    same dtype, ready for ``fwd``."""
    dt = _in_dtype(u, W_x, W_dt)
    batch, L, dim = u.shape
    N, delta_raw, B, C = _proj_outputs(u, W_x, W_dt, rank, delta_raw, B, C)
    rc = load_library().ss_proj(_ptr(u), _ptr(W_x), _ptr(W_dt), _ptr(delta_raw), _ptr(B), _ptr(C),
                                batch, L, dim, N, int(rank), dt, _stream(u.device, stream))
    if rc != 0:
        raise SSError(rc, "ss_proj")
    return delta_raw, B, C


def proj_conv(x, conv_w, W_x, W_dt, rank, conv_b=None, conv_state=None, delta_raw=None, B=None, C=None,
              stream=None):
    """Input projections with the fused prologue (``ss_proj_conv``): ``proj`` of u =
    silu(causal depthwise conv1d(x) + conv_b), u formed on the fly and never stored. x:
    (batch, L, dim) like ``proj``'s u; conv_w (dim, K) fp32, K <= 4; conv_b (dim,) fp32 or
    None; conv_state (batch, dim, K-1) fp32 or None. Returns (delta_raw, B, C)."""
    dev = x.device
    dt = _in_dtype(x, W_x, W_dt)
    batch, L, dim = x.shape
    K = conv_w.shape[1] if conv_w.dim() == 2 else 0
    _check(conv_w, "conv_w", dev, torch.float32, (dim, K))
    _check(conv_b, "conv_b", dev, torch.float32, (dim,))
    _check(conv_state, "conv_state", dev, torch.float32, (batch, dim, K - 1))
    N, delta_raw, B, C = _proj_outputs(x, W_x, W_dt, rank, delta_raw, B, C)
    rc = load_library().ss_proj_conv(_ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), K, _ptr(W_x),
                                     _ptr(W_dt), _ptr(delta_raw), _ptr(B), _ptr(C), batch, L, dim, N, int(rank),
                                     dt, _stream(dev, stream))
    if rc != 0:
        raise SSError(rc, "ss_proj_conv")
    return delta_raw, B, C
