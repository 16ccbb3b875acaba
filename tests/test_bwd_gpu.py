"""GPU parity of ss_bwd (the backward of the scan) against the fp64 oracle's backward.

Every gradient is compared element by element, |gpu - ref| <= tol * (1 + |ref|), with
tol = 1e-4 for fp32 inputs and 2e-3 for bf16 inputs (the oracle gets the identical bf16
values and the same fp32 dy), up to the full 3B long-context size (every channel there too,
the oracle run on slices of channels).
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
KEYS = ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0")


def _announce(msg):
    print(f"\n[bwd] {msg}", flush=True)


def _dy(shape, seed):
    g = inputs.HostStream(seed)
    return g.randn(shape, DEV)


def _oracle(x, dy, gated=True, use_D=True, use_bias=True, softplus=True, h0=None, dlast=None, channels=None):
    n = {k: inputs.to_numpy(v) for k, v in x.items()}
    return oracle.bwd(n["u"], n["delta"], n["A"], n["B"], n["C"], dy.cpu().numpy(),
                      D=n["D"] if use_D else None, z=n["z"] if gated else None,
                      delta_bias=n["delta_bias"] if use_bias else None, softplus=softplus,
                      h0=None if h0 is None else h0.double().cpu().numpy(),
                      dlast=None if dlast is None else dlast.cpu().numpy(), channels=channels)


def _gpu(x, dy, gated=True, use_D=True, use_bias=True, softplus=True, h0=None, dlast=None):
    return ss.bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"] if use_D else None,
                  z=x["z"] if gated else None, delta_bias=x["delta_bias"] if use_bias else None,
                  softplus=softplus, h0=h0, dlast=dlast)


def _compare(g, r, tol, what, keys=KEYS):
    for k in keys:
        if g.get(k) is None or r.get(k) is None:
            continue
        err = pu.scaled_err(g[k].double().cpu().numpy(), r[k])
        assert err <= tol, f"{what}: {k} max scaled error {err:.3e} > {tol}"


SHAPES = [(2, 37, 40, 16, "f32"), (1, 129, 33, 16, "bf16"), (3, 64, 20, 5, "f32"),
          (2, 300, 70, 16, "f32"), (1, 1, 16, 16, "f32"), (2, 1000, 130, 16, "f32"),
          (1, 777, 257, 16, "bf16"), (2, 31, 16, 1, "f32"), (1, 33, 48, 16, "f32"),
          (2, 200, 240, 16, "bf16")]  # 15 channel groups: the dB/dC sum's 8-group step and a 7-group tail


@pytest.mark.parametrize("batch,L,dim,N,dt", SHAPES)
@pytest.mark.parametrize("gated", [False, True])
def test_bwd_matches_oracle(batch, L, dim, N, dt, gated):
    w = inputs.WORKLOADS["mamba130m"].replace(name=f"b{batch}x{L}x{dim}x{N}{dt}", batch=batch, seqlen=L,
                                              dim=dim, dstate=N, dtype=dt)
    x = inputs.make(w, seed=51, device=DEV)
    dy = _dy((batch, L, dim), 52)
    _announce(f"{w.name} gated={gated}")
    g = _gpu(x, dy, gated)
    torch.cuda.synchronize()
    _compare(g, _oracle(x, dy, gated), pu.tol_of(x), w.name)


@pytest.mark.parametrize("batch,L,dim,N", [(2, 100, 40, 16), (1, 65, 24, 7)])
def test_bwd_initial_state_and_final_state_gradient(batch, L, dim, N):
    w = inputs.WORKLOADS["mamba130m"].replace(name="bh0", batch=batch, seqlen=L, dim=dim, dstate=N)
    x = inputs.make(w, seed=53, device=DEV)
    dy = _dy((batch, L, dim), 54)
    h0 = _dy((batch, dim, N), 55)
    dlast = _dy((batch, dim, N), 56)
    g = _gpu(x, dy, True, h0=h0, dlast=dlast)
    torch.cuda.synchronize()
    _compare(g, _oracle(x, dy, True, h0=h0, dlast=dlast), pu.tol_of(x), "h0 + dlast")


@pytest.mark.parametrize("use_D,use_bias,softplus", [(False, False, True), (True, False, False),
                                                     (False, True, True)])
def test_bwd_optional_arguments(use_D, use_bias, softplus):
    w = inputs.WORKLOADS["mamba130m"].replace(name="bopt", batch=2, seqlen=90, dim=48)
    x = inputs.make(w, seed=57, device=DEV)
    if not softplus:  # keep the steps positive without softplus
        x["delta"] = x["delta"].abs() * 0.05
    dy = _dy((2, 90, 48), 58)
    g = _gpu(x, dy, True, use_D, use_bias, softplus)
    torch.cuda.synchronize()
    assert (g["dD"] is None) == (not use_D) and (g["ddelta_bias"] is None) == (not use_bias)
    _compare(g, _oracle(x, dy, True, use_D, use_bias, softplus), pu.tol_of(x), "optional arguments")


def test_bwd_empty_sequence():
    w = inputs.WORKLOADS["mamba130m"].replace(name="bempty", batch=2, seqlen=0, dim=40)
    x = inputs.make(w, seed=59, device=DEV)
    dy = torch.empty((2, 0, 40), device=DEV)
    dlast = _dy((2, 40, 16), 60)
    g = _gpu(x, dy, True, dlast=dlast)
    torch.cuda.synchronize()
    assert torch.equal(g["dh0"], dlast)
    assert not g["dA"].any() and not g["dD"].any() and not g["ddelta_bias"].any()


def test_bwd_deterministic():
    w = inputs.WORKLOADS["mamba130m"].replace(name="bdet", batch=2, seqlen=500, dim=96)
    x = inputs.make(w, seed=61, device=DEV)
    dy = _dy((2, 500, 96), 62)
    g1 = _gpu(x, dy)
    g2 = _gpu(x, dy)
    torch.cuda.synchronize()
    for k in KEYS:
        assert torch.equal(g1[k], g2[k]), k


def test_bwd_mamba130m_full_every_element():
    w = inputs.WORKLOADS["mamba130m"]
    x = inputs.make(w, seed=63, device=DEV)
    dy = _dy((w.batch, w.seqlen, w.dim), 64)
    for gated in (False, True):
        _announce(f"mamba130m full gated={gated}")
        g = _gpu(x, dy, gated)
        torch.cuda.synchronize()
        _compare(g, _oracle(x, dy, gated), pu.tol_of(x), f"mamba130m gated={gated}")


def test_bwd_mamba3b_long_every_channel():
    """Full 3B long-context shape: every gradient of all 5120 channels against the oracle,
    element by element. The oracle runs on slices of 640 channels; its channel-summed dB and
    dC add up the slices in fp64."""
    w = inputs.WORKLOADS["mamba3b-long"]
    _announce(f"{w.name} backward, every channel")
    x = inputs.make(w, seed=65, device=DEV)
    dy = _dy((w.batch, w.seqlen, w.dim), 66)
    g = _gpu(x, dy, True)
    torch.cuda.synchronize()
    tol = pu.tol_of(x)
    n = {k: inputs.to_numpy(v) for k, v in x.items()}
    dyn = dy.cpu().numpy()
    del dy
    dB = np.zeros((w.batch, w.seqlen, w.dstate))
    dC = np.zeros_like(dB)
    step = 640
    for b in range(w.batch):
        for d0 in range(0, w.dim, step):
            d1 = min(w.dim, d0 + step)
            ch = np.stack([np.full(d1 - d0, b, np.int64), np.arange(d0, d1, dtype=np.int64)], axis=1)
            r = oracle.bwd(n["u"], n["delta"], n["A"], n["B"], n["C"], dyn, D=n["D"], z=n["z"],
                           delta_bias=n["delta_bias"], channels=ch)
            dB += r["dB"]
            dC += r["dC"]
            for k in ("du", "ddelta", "dz"):
                got = g[k][b, :, d0:d1].t().contiguous().double().cpu().numpy()
                err = pu.scaled_err(got, r[k])
                assert err <= tol, f"{k} channels {d0}..{d1}: {err:.3e}"
            # dA, dD, dbias sum over batch rows; batch is 1 here, so the channels' own terms
            for k in ("dA", "dD", "ddelta_bias"):
                err = pu.scaled_err(g[k][d0:d1].double().cpu().numpy(), r[k])
                assert err <= tol, f"{k} channels {d0}..{d1}: {err:.3e}"
            err = pu.scaled_err(g["dh0"][b, d0:d1].double().cpu().numpy(), r["dh0"])
            assert err <= tol, f"dh0 channels {d0}..{d1}: {err:.3e}"
            print(f"[bwd]   channels {d0}..{d1} ok", flush=True)
    for k, ref in (("dB", dB), ("dC", dC)):
        err = pu.scaled_err(g[k].double().cpu().numpy(), ref)
        assert err <= tol, f"{k}: {err:.3e}"
