"""fp64 CPU oracle for the selective-scan (S6) forward, decode step, backward, conv prologue
and input projections.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package. It never imports or calls the GPU library,
and the GPU library never imports it.

The arithmetic lives in ``ss_oracle.c`` (plain sequential loops in IEEE double, one
independent recurrence per (batch, channel)); this module only compiles it with gcc and
marshals numpy arrays. Inputs are numpy arrays: ``float32`` for fp32 data, ``uint16``
holding bf16 bit patterns for bf16 data (u, delta, z, B, C share one of the two);
A, D and delta_bias are ``float32``. Results are ``float64``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ss_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libss_oracle.so")
_lib = None

F32 = 0
BF16 = 1
F64 = 2


CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-std=c11", "-Wall",
          "-Wextra", "-shared", "-fPIC"]


def compile_source(src: str, out: str) -> str:
    """gcc the given C file into a shared library at ``out``."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast math, no contraction, OpenMP over channels)."""
    if force or not os.path.exists(_LIB_PATH):
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


def _bind(path):
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.ss_oracle_fwd.restype = i32
    lib.ss_oracle_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp,
                                  i64, i64, i64, i64, i32, vp, vp, i64, i32]
    lib.ss_oracle_step.restype = i32
    lib.ss_oracle_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp,
                                   i64, i64, i64, i32, i32]
    lib.ss_oracle_bwd.restype = i32
    lib.ss_oracle_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp,
                                  vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                  i64, i64, i64, i64, i32, vp, vp, i64, i32]
    lib.ss_oracle_conv_silu.restype = i32
    lib.ss_oracle_conv_silu.argtypes = [vp, vp, vp, vp, i64, vp, i64, i64, i64, i32, i32]
    lib.ss_oracle_proj.restype = i32
    lib.ss_oracle_proj.argtypes = [vp, vp, vp, i32, i32, i64, i64, i64, i64, i64, vp, vp, vp, i32]
    lib.ss_oracle_max_threads.restype = i32
    lib.ss_oracle_max_threads.argtypes = []
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _bind(_LIB_PATH)
    return _lib


def max_threads() -> int:
    return int(_load().ss_oracle_max_threads())


def _dtype_of(*arrays) -> int:
    kinds = {a.dtype for a in arrays if a is not None}
    if kinds == {np.dtype(np.float32)}:
        return F32
    if kinds == {np.dtype(np.uint16)}:
        return BF16
    if kinds == {np.dtype(np.float64)}:
        return F64
    raise TypeError(f"u, delta, z, B, C must all be float32, all uint16 (bf16 bits) or all "
                    f"float64, got {kinds}")


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if dtype is not None and a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, h0=None,
        channels=None, nthreads=0, want_y=True, zoh=False, _lib=None):
    """Forward scan. Shapes: u, delta, z (batch, L, dim); B, C (batch, L, N); A (dim, N);
    D, delta_bias (dim,); h0 (batch, dim, N) float64 or None.
    zoh: input term (exp(dt A) - 1)/A * B instead of dt * B.

    channels: None for every channel, else an int array of shape (k, 2) of (b, d) pairs;
    then y is (k, L) and last_state is (k, N).
    Returns (y, last_state) as float64 arrays (y is None when want_y is False).
    """
    u, delta, B, C, z = _c(u), _c(delta), _c(B), _c(C), _c(z)
    A, D, delta_bias = _c(A, np.float32), _c(D, np.float32), _c(delta_bias, np.float32)
    dt = _dtype_of(u, delta, B, C, z)
    batch, L, dim = u.shape
    N = A.shape[1]
    if delta.shape != u.shape or (z is not None and z.shape != u.shape):
        raise ValueError("u, delta and z must share a shape")
    if B.shape != (batch, L, N) or C.shape != (batch, L, N) or A.shape != (dim, N):
        raise ValueError("bad B, C or A shape")
    if h0 is not None:
        h0 = _c(h0, np.float64)
        if h0.shape != (batch, dim, N):
            raise ValueError("bad h0 shape")
    if channels is None:
        nchan, cb, cd = 0, None, None
        y = np.empty((batch, L, dim), np.float64) if want_y else None
        st = np.empty((batch, dim, N), np.float64)
    else:
        ch = np.ascontiguousarray(np.asarray(channels, dtype=np.int64).reshape(-1, 2))
        nchan = ch.shape[0]
        cb, cd = np.ascontiguousarray(ch[:, 0]), np.ascontiguousarray(ch[:, 1])
        y = np.empty((nchan, L), np.float64) if want_y else None
        st = np.empty((nchan, N), np.float64)
        if nchan == 0:
            return y, st
    rc = (_lib or _load()).ss_oracle_fwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                               _ptr(delta_bias), int(bool(softplus)), int(bool(zoh)), _ptr(h0),
                               _ptr(y), _ptr(st),
                               batch, L, dim, N, dt, _ptr(cb), _ptr(cd), nchan, int(nthreads))
    if rc != 0:
        raise ValueError("ss_oracle_fwd rejected its arguments")
    return y, st


def step(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, nthreads=0,
         zoh=False, _lib=None):
    """One decode step, state (batch, dim, N) float64 updated in place. u, delta, z are
    (batch, dim); B, C are (batch, N). Returns y (batch, dim) float64."""
    if state.dtype != np.float64 or not state.flags.c_contiguous:
        raise TypeError("state must be a C-contiguous float64 array")
    u, delta, B, C, z = _c(u), _c(delta), _c(B), _c(C), _c(z)
    A, D, delta_bias = _c(A, np.float32), _c(D, np.float32), _c(delta_bias, np.float32)
    dt = _dtype_of(u, delta, B, C, z)
    batch, dim = u.shape
    N = A.shape[1]
    if state.shape != (batch, dim, N) or B.shape != (batch, N) or C.shape != (batch, N):
        raise ValueError("bad state, B or C shape")
    y = np.empty((batch, dim), np.float64)
    rc = (_lib or _load()).ss_oracle_step(_ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                _ptr(D), _ptr(z), _ptr(delta_bias), int(bool(softplus)),
                                int(bool(zoh)), _ptr(y),
                                batch, dim, N, dt, int(nthreads))
    if rc != 0:
        raise ValueError("ss_oracle_step rejected its arguments")
    return y


def bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, softplus=True, h0=None,
        dlast=None, channels=None, nthreads=0, _lib=None):
    """Backward of ``fwd`` (input term dt*B) for dL/dy = dy (batch, L, dim) float32 and
    dL/dlast_state = dlast (batch, dim, N) float32 or None.

    Returns a dict of float64 arrays: du, ddelta, dz (batch, L, dim) [dz only with z];
    dA (dim, N); dD, ddelta_bias (dim,); dh0 (batch, dim, N); dB, dC (batch, L, N).
    With channels ((k, 2) array of (b, d)): du, ddelta, dz are (k, L); dA, dh0 (k, N) and
    dD, ddelta_bias (k,) are each channel's own terms; dB, dC sum the listed channels.
    """
    u, delta, B, C, z = _c(u), _c(delta), _c(B), _c(C), _c(z)
    A, D, delta_bias = _c(A, np.float32), _c(D, np.float32), _c(delta_bias, np.float32)
    dy, dlast = _c(dy, np.float32), _c(dlast, np.float32)
    dt = _dtype_of(u, delta, B, C, z)
    batch, L, dim = u.shape
    N = A.shape[1]
    if delta.shape != u.shape or (z is not None and z.shape != u.shape) or dy.shape != u.shape:
        raise ValueError("u, delta, z and dy must share a shape")
    if B.shape != (batch, L, N) or C.shape != (batch, L, N) or A.shape != (dim, N):
        raise ValueError("bad B, C or A shape")
    if h0 is not None:
        h0 = _c(h0, np.float64)
        if h0.shape != (batch, dim, N):
            raise ValueError("bad h0 shape")
    if dlast is not None and dlast.shape != (batch, dim, N):
        raise ValueError("bad dlast shape")
    f = np.float64
    if channels is None:
        nchan, cb, cd = 0, None, None
        tok, per_ch, rows = (batch, L, dim), (dim,), (batch, dim)
    else:
        ch = np.ascontiguousarray(np.asarray(channels, dtype=np.int64).reshape(-1, 2))
        nchan = ch.shape[0]
        cb, cd = np.ascontiguousarray(ch[:, 0]), np.ascontiguousarray(ch[:, 1])
        tok, per_ch, rows = (nchan, L), (nchan,), (nchan,)
    out = dict(du=np.zeros(tok, f), ddelta=np.zeros(tok, f),
               dz=np.zeros(tok, f) if z is not None else None,
               dA=np.zeros(per_ch + (N,), f), dD=np.zeros(per_ch, f), ddelta_bias=np.zeros(per_ch, f),
               dh0=np.zeros(rows + (N,), f), dB=np.zeros((batch, L, N), f), dC=np.zeros((batch, L, N), f))
    if channels is not None and nchan == 0:
        return out
    rc = (_lib or _load()).ss_oracle_bwd(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
        int(bool(softplus)), _ptr(h0), _ptr(dy), _ptr(dlast), _ptr(out["du"]), _ptr(out["ddelta"]),
        _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dz"]),
        _ptr(out["ddelta_bias"]), _ptr(out["dh0"]), batch, L, dim, N, dt, _ptr(cb), _ptr(cd), nchan,
        int(nthreads))
    if rc != 0:
        raise ValueError("ss_oracle_bwd rejected its arguments")
    return out


def conv_silu(x, conv_w, conv_b=None, conv_state=None, nthreads=0, _lib=None):
    """The prologue u = silu(causal depthwise conv1d(x) + conv_b): x (batch, L, dim) float32,
    uint16 (bf16 bits) or float64; conv_w (dim, K) float32; conv_b (dim,) float32 or None;
    conv_state (batch, dim, K-1) float32 or None (the K-1 inputs before t = 0, oldest
    first; zeros when None). Returns u (batch, L, dim) float64."""
    x = _c(x)
    conv_w, conv_b, conv_state = _c(conv_w, np.float32), _c(conv_b, np.float32), _c(conv_state, np.float32)
    dt = _dtype_of(x)
    batch, L, dim = x.shape
    K = conv_w.shape[1]
    if conv_w.shape != (dim, K) or (conv_b is not None and conv_b.shape != (dim,)):
        raise ValueError("bad conv_w or conv_b shape")
    if conv_state is not None and conv_state.shape != (batch, dim, K - 1):
        raise ValueError("bad conv_state shape")
    u = np.empty((batch, L, dim), np.float64)
    rc = (_lib or _load()).ss_oracle_conv_silu(_ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), K,
                                              _ptr(u), batch, L, dim, dt, int(nthreads))
    if rc != 0:
        raise ValueError("ss_oracle_conv_silu rejected its arguments")
    return u


def _widen(a):
    """float32 / bf16-bit arrays to float64, exactly."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def fwd_conv(x, conv_w, delta, A, B, C, conv_b=None, conv_state=None, D=None, z=None,
             delta_bias=None, softplus=True, h0=None, channels=None, nthreads=0, zoh=False, _lib=None):
    """Forward with the conv prologue: u = conv_silu(x, ...) in fp64, then the scan of
    ``fwd`` on that u (delta, B, C, z widened exactly to fp64). Returns (y, last_state, u)."""
    u = conv_silu(x, conv_w, conv_b, conv_state, nthreads=nthreads, _lib=_lib)
    y, st = fwd(u, _widen(_c(delta)), A, _widen(_c(B)), _widen(_c(C)), D=D, z=_widen(_c(z)),
                delta_bias=delta_bias, softplus=softplus, h0=h0, channels=channels,
                nthreads=nthreads, zoh=zoh, _lib=_lib)
    return y, st, u


def proj(u, W_x, W_dt, rank, dstate, conv_w=None, conv_b=None, conv_state=None, nthreads=0, _lib=None):
    """Projections of the token inputs: xp = W_x u_t, delta_raw = W_dt xp[:rank],
    B = xp[rank:rank+N], C = xp[rank+N:rank+2N] (see ss_oracle_proj). u (batch, L, dim) is
    float32, uint16 (bf16 bits) or float64; with conv_w it is x, and u = conv_silu(x, ...)
    first (fp64). W_x (rank + 2N, dim) and W_dt (dim, rank): float32 or uint16 (bf16 bits).
    Returns (delta_raw, B, C) as float64."""
    lib = _lib or _load()
    if conv_w is not None:
        u = conv_silu(u, conv_w, conv_b, conv_state, nthreads=nthreads, _lib=lib)
    u, W_x, W_dt = _c(u), _c(W_x), _c(W_dt)
    batch, L, dim = u.shape
    if W_x.shape != (rank + 2 * dstate, dim) or W_dt.shape != (dim, rank):
        raise ValueError("bad W_x or W_dt shape")
    wdt = _dtype_of(W_x, W_dt)
    delta_raw = np.empty((batch, L, dim), np.float64)
    B = np.empty((batch, L, dstate), np.float64)
    C = np.empty((batch, L, dstate), np.float64)
    rc = lib.ss_oracle_proj(_ptr(u), _ptr(W_x), _ptr(W_dt), _dtype_of(u), wdt, batch, L, dim, dstate, rank,
                            _ptr(delta_raw), _ptr(B), _ptr(C), int(nthreads))
    if rc != 0:
        raise ValueError("ss_oracle_proj rejected its arguments")
    return delta_raw, B, C


class Library:
    """The oracle API bound to another build of the same C source (used by the tests that
    plant mistakes in a copy of the oracle and check that the pins catch them)."""

    def __init__(self, path):
        self._h = _bind(path)

    def fwd(self, *a, **k):
        return fwd(*a, _lib=self._h, **k)

    def step(self, *a, **k):
        return step(*a, _lib=self._h, **k)

    def bwd(self, *a, **k):
        return bwd(*a, _lib=self._h, **k)

    def conv_silu(self, *a, **k):
        return conv_silu(*a, _lib=self._h, **k)

    def fwd_conv(self, *a, **k):
        return fwd_conv(*a, _lib=self._h, **k)

    def proj(self, *a, **k):
        return proj(*a, _lib=self._h, **k)
