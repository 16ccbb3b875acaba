"""GPU parity of the exact zero-order-hold input term (ss_fwd_ex / ss_step_ex with
SS_DISC_ZOH) against the fp64 oracle run with zoh=True, element by element.

The input coefficient (exp(dt A) - 1)/A is evaluated in fp32 by a short series for
|dt A| < 1/16 and by the difference of the decay otherwise; the tests cover both sides of
that switch, A = 0 (the limit dt) and growing modes (A > 0). Tolerance as for the default
input term: |gpu - ref| <= tol * (1 + |ref|), tol = 1e-4 (fp32 inputs), 2e-3 (bf16).
"""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_86_amd as ss
from selective_state_space_86_amd import inputs
from tests import parity_util as pu

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
KERNELS = [(1, 0, 0), (2, 4, 16), (2, 8, 16), (2, 4, 12), (2, 8, 32), (2, 4, 32)]  # (kernel, chunk_len, chunk_rows)


def _announce(msg):
    print(f"\n[zoh] {msg}", flush=True)


def _check(x, y, st, gated=True, h0=None, softplus=True, what=""):
    y_ref, st_ref = pu.oracle_full(x, gated, softplus=softplus, zoh=True, h0=h0)
    tol = pu.tol_of(x)
    ey = pu.scaled_err(y.double().cpu().numpy(), y_ref)
    es = pu.scaled_err(st.double().cpu().numpy(), st_ref)
    assert ey <= tol, f"{what}: y max scaled error {ey:.3e} > {tol}"
    assert es <= tol, f"{what}: state max scaled error {es:.3e} > {tol}"


@pytest.mark.parametrize("kernel,chunk,rows", KERNELS)
@pytest.mark.parametrize("batch,L,dim,N,dt", [(3, 37, 100, 16, "f32"), (2, 129, 70, 16, "bf16"),
                                              (2, 1000, 130, 16, "f32"), (1, 300, 17, 16, "f32"),
                                              (2, 64, 40, 7, "f32")])
def test_zoh_every_kernel_choice(kernel, chunk, rows, batch, L, dim, N, dt):
    if kernel == 2 and N != 16:
        pytest.skip("the time-chunked kernel is for dstate 16")
    w = inputs.WORKLOADS["mamba130m"].replace(name=f"z{batch}x{L}x{dim}x{N}{dt}", batch=batch, seqlen=L,
                                              dim=dim, dstate=N, dtype=dt)
    x = inputs.make(w, seed=31, device=DEV)
    _announce(f"kernel={kernel} chunk={chunk} {w.name}")
    for gated in (False, True):
        y, st = pu.gpu_fwd(x, gated, kernel=kernel, chunk_len=chunk, chunk_rows=rows, zoh=True)
        torch.cuda.synchronize()
        _check(x, y, st, gated, what=f"{w.name} gated={gated}")


def _wide_range_inputs(batch, L, dim, seed):
    """Step sizes from ~1e-6 to ~5 and |A| from 1e-4 to 20, so dt*A runs from ~1e-10 to
    ~100 across the series / difference switch at 1/16; a few A are exactly 0 (limit dt)
    and a few small positive A grow the state."""
    g = inputs.HostStream(seed)
    N = 16
    u = g.randn((batch, L, dim), DEV)
    delta = g.rand((batch, L, dim), DEV) * 15.0 - 13.0       # softplus: ~2e-6 .. ~2
    B = g.randn((batch, L, N), DEV)
    C = g.randn((batch, L, N), DEV)
    z = g.randn((batch, L, dim), DEV)
    A = -torch.pow(10.0, g.rand((dim, N), DEV) * 5.3 - 4.0)   # -1e-4 .. -20
    A[::7, 3] = 0.0
    A[1::11, 5] = 0.002
    D = g.randn((dim,), DEV)
    bias = g.rand((dim,), DEV) * 2.0 - 1.0
    return dict(u=u, delta=delta, z=z, B=B, C=C, A=A.contiguous(), D=D, delta_bias=bias)


@pytest.mark.parametrize("kernel,chunk,rows", KERNELS)
def test_zoh_step_sizes_across_the_series_switch(kernel, chunk, rows):
    x = _wide_range_inputs(2, 400, 96, seed=32)
    _announce(f"wide-range dt*A kernel={kernel} chunk={chunk}")
    y, st = pu.gpu_fwd(x, True, kernel=kernel, chunk_len=chunk, chunk_rows=rows, zoh=True)
    torch.cuda.synchronize()
    _check(x, y, st, True, what="wide range")


@pytest.mark.parametrize("kernel,chunk,rows", KERNELS)
def test_zoh_initial_state(kernel, chunk, rows):
    w = inputs.WORKLOADS["mamba1.4b"].replace(name="zh0", batch=2, seqlen=333, dim=80)
    x = inputs.make(w, seed=33, device=DEV)
    h0 = inputs.HostStream(86).randn((2, 80, 16), DEV)
    y, st = pu.gpu_fwd(x, True, kernel=kernel, chunk_len=chunk, chunk_rows=rows, zoh=True, h0=h0)
    torch.cuda.synchronize()
    _check(x, y, st, True, h0=h0, what="zoh from h0")


def test_zoh_mamba130m_full_every_element():
    x = inputs.make(inputs.WORKLOADS["mamba130m"], seed=34, device=DEV)
    for gated in (False, True):
        _announce(f"mamba130m full zoh gated={gated}")
        y, st = pu.gpu_fwd(x, gated, zoh=True)
        torch.cuda.synchronize()
        _check(x, y, st, gated, what=f"mamba130m gated={gated}")


def test_zoh_mamba3b_long_full_size_sampled():
    w = inputs.WORKLOADS["mamba3b-long"]
    _announce(f"{w.name} zoh sampled")
    x = inputs.make(w, seed=35, device=DEV)
    y, st = pu.gpu_fwd(x, True, zoh=True)
    torch.cuda.synchronize()
    chans = pu.sample_channels(w.batch, w.dim, 32, seed=35)
    yg, sg = pu.gpu_channels(y, st, chans)
    yr, sr = pu.oracle_channels(x, chans, gated=True, zoh=True)
    tol = pu.tol_of(x)
    assert pu.scaled_err(yg, yr) <= tol
    assert pu.scaled_err(sg, sr) <= tol


def test_zoh_differs_from_default_input_term():
    """The option changes the result (by about dt*A/2 relative), so it is really applied."""
    w = inputs.WORKLOADS["mamba130m"].replace(name="zdiff", batch=1, seqlen=256, dim=64)
    x = inputs.make(w, seed=36, device=DEV)
    y0, _ = pu.gpu_fwd(x, False)
    y1, _ = pu.gpu_fwd(x, False, zoh=True)
    torch.cuda.synchronize()
    assert ((y1 - y0).abs() / (1 + y0.abs())).max().item() > 1e-3


@pytest.mark.parametrize("N,dt", [(16, "f32"), (5, "bf16")])
def test_zoh_decode_stream_matches_oracle_and_forward(N, dt):
    """ss_step_ex(zoh) token by token equals the oracle's zoh steps and ss_fwd_ex(zoh)."""
    w = inputs.WORKLOADS["decode"].replace(name=f"zdec{N}{dt}", batch=3, seqlen=50, dim=128, dstate=N,
                                           dtype=dt)
    x = inputs.make(w, seed=37, device=DEV, time_major=True)
    L, batch, dim = x["u"].shape
    state = torch.zeros((batch, dim, N), dtype=torch.float32, device=DEV)
    ys = []
    for t in range(L):
        ys.append(ss.step(state, x["u"][t], x["delta"][t], x["A"], x["B"][t], x["C"][t], D=x["D"],
                          z=x["z"][t], delta_bias=x["delta_bias"], zoh=True))
    xb = {k: (v.transpose(0, 1).contiguous() if k in ("u", "delta", "z", "B", "C") else v)
          for k, v in x.items()}
    y_fwd, st_fwd = pu.gpu_fwd(xb, True, zoh=True)
    torch.cuda.synchronize()
    y_step = torch.stack(ys, dim=1)
    tol = pu.tol_of(x)
    n = {k: inputs.to_numpy(v) for k, v in x.items()}
    ref = np.zeros((batch, dim, N))
    for t in range(L):
        yr = oracle.step(ref, n["u"][t], n["delta"][t], n["A"], n["B"][t], n["C"][t], D=n["D"], z=n["z"][t],
                         delta_bias=n["delta_bias"], zoh=True)
        assert pu.scaled_err(y_step[:, t].double().cpu().numpy(), yr) <= tol, f"step {t}"
    assert pu.scaled_err(state.double().cpu().numpy(), ref) <= tol
    assert ((y_step - y_fwd).abs() / (1 + y_fwd.abs())).max().item() <= tol
    assert ((state - st_fwd).abs() / (1 + st_fwd.abs())).max().item() <= tol
