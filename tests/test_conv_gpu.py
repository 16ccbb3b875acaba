"""GPU parity of ss_fwd_conv (the scan with the conv1d + SiLU prologue fused in) against
the oracle's fwd_conv (the fp64 prologue followed by the fp64 scan), element by element:
y, the final state and the prologue output u, with |gpu - ref| <= tol * (1 + |ref|),
tol = 1e-4 for fp32 inputs and 2e-3 for bf16 inputs.
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
    print(f"\n[conv] {msg}", flush=True)


def conv_params(batch, dim, K, seed, bias=True, state=True):
    g = inputs.HostStream(seed)
    w = (g.randn((dim, K), DEV) * 0.5).contiguous()
    b = g.randn((dim,), DEV) * 0.1 if bias else None
    st = g.randn((batch, dim, K - 1), DEV) if state and K > 1 else None
    return w, b, st


def gpu_conv(x, w, b, st, gated=True, h0=None, **kw):
    return ss.fwd_conv(x["u"], w, x["delta"], x["A"], x["B"], x["C"], conv_b=b, conv_state=st, D=x["D"],
                       z=x["z"] if gated else None, delta_bias=x["delta_bias"], h0=h0, u_out=True, **kw)


def oracle_conv(x, w, b, st, gated=True, h0=None, zoh=False):
    n = {k: inputs.to_numpy(v) for k, v in x.items()}
    return oracle.fwd_conv(n["u"], w.cpu().numpy(), n["delta"], n["A"], n["B"], n["C"],
                           conv_b=None if b is None else b.cpu().numpy(),
                           conv_state=None if st is None else st.cpu().numpy(), D=n["D"],
                           z=n["z"] if gated else None, delta_bias=n["delta_bias"],
                           h0=None if h0 is None else h0.double().cpu().numpy(), zoh=zoh)


def check(x, got, ref, what):
    tol = pu.tol_of(x)
    for name, g, r in zip(("y", "state", "u"), got, ref):
        err = pu.scaled_err(g.double().cpu().numpy(), r)
        assert err <= tol, f"{what}: {name} max scaled error {err:.3e} > {tol}"


@pytest.mark.parametrize("kernel,chunk,rows", KERNELS)
@pytest.mark.parametrize("batch,L,dim,N,dt,K", [(2, 37, 40, 16, "f32", 4), (1, 129, 33, 16, "bf16", 4),
                                                (2, 300, 70, 16, "f32", 3), (3, 64, 20, 5, "f32", 4),
                                                (1, 777, 130, 16, "bf16", 2), (2, 50, 16, 16, "f32", 1),
                                                (1, 2, 24, 16, "f32", 4)])
def test_conv_every_kernel_choice(kernel, chunk, rows, batch, L, dim, N, dt, K):
    if kernel == 2 and N != 16:
        pytest.skip("the time-chunked kernel is for dstate 16")
    w = inputs.WORKLOADS["mamba130m"].replace(name=f"c{batch}x{L}x{dim}x{N}{dt}k{K}", batch=batch, seqlen=L,
                                              dim=dim, dstate=N, dtype=dt)
    x = inputs.make(w, seed=81, device=DEV)
    _announce(f"kernel={kernel} chunk={chunk} {w.name}")
    for gated, bias, state in ((True, True, True), (False, False, False)):
        cw, cb, cs = conv_params(batch, dim, K, 82, bias, state)
        got = gpu_conv(x, cw, cb, cs, gated, kernel=kernel, chunk_len=chunk, chunk_rows=rows)
        torch.cuda.synchronize()
        check(x, got, oracle_conv(x, cw, cb, cs, gated), f"{w.name} gated={gated}")


def test_conv_with_initial_state_and_zoh():
    w = inputs.WORKLOADS["mamba130m"].replace(name="cz", batch=2, seqlen=200, dim=48)
    x = inputs.make(w, seed=83, device=DEV)
    cw, cb, cs = conv_params(2, 48, 4, 84)
    h0 = inputs.HostStream(82).randn((2, 48, 16), DEV)
    got = gpu_conv(x, cw, cb, cs, True, h0=h0, zoh=True)
    torch.cuda.synchronize()
    check(x, got, oracle_conv(x, cw, cb, cs, True, h0=h0, zoh=True), "h0 + zoh")


def test_conv_prefill_split_continues():
    """Two calls, the second from the first's final state and with the last 3 inputs as
    conv state, equal one call."""
    w = inputs.WORKLOADS["mamba1.4b"].replace(name="csplit", batch=2, seqlen=1000, dim=96)
    x = inputs.make(w, seed=85, device=DEV)
    cw, cb, _ = conv_params(2, 96, 4, 86, state=False)
    y, st, u = gpu_conv(x, cw, cb, None)
    t0 = 333
    part = lambda sl: {k: (v[:, sl].contiguous() if k in ("u", "delta", "z", "B", "C") else v) for k, v in x.items()}
    y1, s1, u1 = gpu_conv(part(slice(0, t0)), cw, cb, None)
    cs = x["u"][:, t0 - 3:t0].transpose(1, 2).float().contiguous()
    y2, s2, u2 = gpu_conv(part(slice(t0, None)), cw, cb, cs, h0=s1)
    torch.cuda.synchronize()
    tol = pu.tol_of(x)
    assert ((torch.cat([y1, y2], 1) - y).abs() / (1 + y.abs())).max().item() <= tol
    assert ((s2 - st).abs() / (1 + st.abs())).max().item() <= tol
    assert torch.equal(torch.cat([u1, u2], 1), u)


def test_conv_mamba130m_full_every_element():
    wl = inputs.WORKLOADS["mamba130m"]
    x = inputs.make(wl, seed=87, device=DEV)
    cw, cb, _ = conv_params(wl.batch, wl.dim, 4, 88, state=False)
    for gated in (False, True):
        _announce(f"mamba130m full conv gated={gated}")
        got = gpu_conv(x, cw, cb, None, gated)
        torch.cuda.synchronize()
        check(x, got, oracle_conv(x, cw, cb, None, gated), f"mamba130m gated={gated}")


def test_conv_mamba3b_long_full_size_sampled():
    wl = inputs.WORKLOADS["mamba3b-long"]
    _announce(f"{wl.name} conv sampled")
    x = inputs.make(wl, seed=89, device=DEV)
    cw, cb, _ = conv_params(wl.batch, wl.dim, 4, 90, state=False)
    y, st, u = gpu_conv(x, cw, cb, None, True)
    torch.cuda.synchronize()
    chans = pu.sample_channels(wl.batch, wl.dim, 24, seed=89)
    d = torch.as_tensor(chans[:, 1], device=DEV)
    # batch is 1: the sampled channels form a (1, L, k) problem of their own
    sub = {k: (v[:, :, d].contiguous() if k in ("u", "delta", "z") else v) for k, v in x.items()}
    sub.update(A=x["A"][d].contiguous(), D=x["D"][d].contiguous(), delta_bias=x["delta_bias"][d].contiguous())
    ref = oracle_conv(sub, cw[d].contiguous(), cb[d].contiguous(), None, True)
    got = (y[:, :, d], st[:, d], u[:, :, d])
    check(x, got, ref, wl.name)
