"""Seeded random configurations of the forward and the backward against the fp64 oracle.

Each case draws batch, sequence length, channels, states, input dtype, gate, D, bias,
softplus, initial state, discretization, kernel, chunk length, tile rows and sequence parts
from a fixed generator, so every run checks the same ~60 combinations (including ragged
channel groups, partial tiles, one-token sequences and parts that do not divide the
sequence). Tolerance per element as everywhere: |err| <= tol * (1 + |ref|), tol = 1e-4 for
fp32 inputs and 2e-3 for bf16 inputs (the oracle gets the identical bf16 values).
"""
import random

import pytest
import torch

import oracle
import selective_state_space_86_amd as ss
from selective_state_space_86_amd import inputs
from tests import parity_util as pu

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(seed):
    r = random.Random(1000 + seed)
    N = r.choice([1, 3, 4, 8, 15, 16, 16, 16, 16])
    c = dict(batch=r.randint(1, 3), L=r.choice([1, 2, 5, 31, 64, 100, 257, 640, 1001]),
             dim=r.choice([1, 7, 16, 17, 40, 96, 130, 200]), N=N, dt=r.choice(["f32", "bf16"]),
             gated=r.random() < 0.5, use_D=r.random() < 0.7, use_bias=r.random() < 0.7,
             softplus=r.random() < 0.85, h0=r.random() < 0.4, zoh=r.random() < 0.25)
    kernels = [0, 1] + ([2, 2, 2] if N == 16 else []) + ([3] if not c["zoh"] else [])
    c["kernel"] = r.choice(kernels)
    if c["kernel"] == 2:
        c["chunk"] = r.choice([0, 4, 8])
        c["rows"] = r.choice([0, 16, 32] + ([12] if c["chunk"] != 8 else []))
        c["parts"] = r.choice([0, 1, 2, 3, 5])
    else:
        c["chunk"], c["rows"], c["parts"] = 0, 0, 0
    return c


def _inputs(c, seed):
    w = inputs.WORKLOADS["mamba130m"].replace(name=f"rnd{seed}", batch=c["batch"], seqlen=c["L"], dim=c["dim"],
                                              dstate=c["N"], dtype=c["dt"])
    x = inputs.make(w, seed=seed, device=DEV)
    if not c["softplus"]:  # the raw step (plus bias) is used as is: keep it positive and small
        x["delta"] = (x["delta"].float().abs() * 0.05).to(x["delta"].dtype)
        x["delta_bias"] = x["delta_bias"].abs() * 0.01
    g = inputs.HostStream(seed)
    h0 = g.randn((c["batch"], c["dim"], c["N"]), DEV) if c["h0"] else None
    return x, h0


@pytest.mark.parametrize("seed", range(48))
def test_random_forward_case(seed):
    c = _case(seed)
    print(f"\n[random] fwd seed={seed} {c}", flush=True)
    x, h0 = _inputs(c, seed)
    y, st = ss.fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"] if c["use_D"] else None,
                   z=x["z"] if c["gated"] else None, delta_bias=x["delta_bias"] if c["use_bias"] else None,
                   softplus=c["softplus"], h0=h0, zoh=c["zoh"], kernel=c["kernel"], chunk_len=c["chunk"],
                   chunk_rows=c["rows"], split_parts=c["parts"])
    torch.cuda.synchronize()
    y_ref, st_ref = pu.oracle_full(x, c["gated"], c["use_D"], c["use_bias"], c["softplus"], zoh=c["zoh"], h0=h0)
    tol = pu.tol_of(x)
    ey = pu.scaled_err(y.double().cpu().numpy(), y_ref)
    es = pu.scaled_err(st.double().cpu().numpy(), st_ref)
    assert ey <= tol and es <= tol, f"seed {seed}: y {ey:.3e}, state {es:.3e} > {tol}"


@pytest.mark.parametrize("seed", range(16))
def test_random_backward_case(seed):
    c = _case(100 + seed)
    c["zoh"] = False  # the backward is of the default input term
    print(f"\n[random] bwd seed={seed} {c}", flush=True)
    x, h0 = _inputs(c, 100 + seed)
    g = inputs.HostStream(200 + seed)
    dy = g.randn((c["batch"], c["L"], c["dim"]), DEV)
    dlast = g.randn((c["batch"], c["dim"], c["N"]), DEV) if seed % 2 else None
    got = ss.bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"] if c["use_D"] else None,
                 z=x["z"] if c["gated"] else None, delta_bias=x["delta_bias"] if c["use_bias"] else None,
                 softplus=c["softplus"], h0=h0, dlast=dlast)
    torch.cuda.synchronize()
    n = {k: inputs.to_numpy(v) for k, v in x.items()}
    ref = oracle.bwd(n["u"], n["delta"], n["A"], n["B"], n["C"], dy.cpu().numpy(),
                     D=n["D"] if c["use_D"] else None, z=n["z"] if c["gated"] else None,
                     delta_bias=n["delta_bias"] if c["use_bias"] else None, softplus=c["softplus"],
                     h0=None if h0 is None else h0.double().cpu().numpy(),
                     dlast=None if dlast is None else dlast.cpu().numpy())
    tol = pu.tol_of(x)
    for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0"):
        if got.get(k) is None or ref.get(k) is None:
            continue
        err = pu.scaled_err(got[k].double().cpu().numpy(), ref[k])
        assert err <= tol, f"seed {seed}: {k} max scaled error {err:.3e} > {tol}"
