"""GPU parity of ss_proj (the input projections on the matrix cores) against the fp64
oracle's proj, element by element, for delta_raw, B and C. fp32 operands and outputs:
|gpu - ref| <= 1e-4 (1 + |ref|). bf16 operands give bf16 outputs, and a bf16 value keeps 8
significant bits, so its rounding alone reaches 2^-8 relative (more than 2e-3 (1 + |ref|) for
|ref| in [2, 4)); the rule there is the correctly rounded exact value up to the same fp32
accumulation allowance: |gpu - ref| <= ulp_bf16(ref) / 2 + 1e-4 (1 + |ref|). The oracle gets
the identical inputs. Shapes cover several token tiles with a ragged last one, channel counts that are
not multiples of the 32-channel groups, dstate below 16, every instantiated count of step
tiles (rank 8 .. 256), the token-split kernel taken for large token counts, and the full
130M-layer size; at the 1.4B and 3B sizes tokens are sampled (the projections are per token, so
a sample is its own problem).
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


def _announce(msg):
    print(f"\n[proj] {msg}", flush=True)


def half_ulp_bf16(r):
    """Half the spacing of bf16 values around |r| (8 significant bits)."""
    a = np.maximum(np.abs(r), 2.0 ** -126)
    return np.ldexp(1.0, (np.floor(np.log2(a)) - 8).astype(np.int64))


def excess(got, ref, bf16):
    """max over elements of the error divided by what the rule allows (<= 1 passes)."""
    got = np.asarray(got, np.float64)
    if got.size == 0:
        return 0.0
    allow = 1e-4 * (1.0 + np.abs(ref))
    if bf16:
        allow = allow + half_ulp_bf16(ref)
    return float(np.max(np.abs(got - ref) / allow))


def oracle_proj(x, rank, N, tokens=None):
    u = x["u"]
    if tokens is not None:  # (batch, token) pairs as a (1, k, dim) problem of their own
        u = u[tokens[:, 0], tokens[:, 1]].unsqueeze(0)
    n = lambda t: inputs.to_numpy(t)
    return oracle.proj(n(u), n(x["W_x"]), n(x["W_dt"]), rank, N)


def check(got, ref, dtype, what, tokens=None):
    for name, g, r in zip(("delta_raw", "B", "C"), got, ref):
        if tokens is not None:
            g = g[tokens[:, 0], tokens[:, 1]].unsqueeze(0)
        x = excess(g.double().cpu().numpy(), r, dtype == torch.bfloat16)
        assert x <= 1.0, f"{what}: {name} error is {x:.3f} times the allowance"


def run_case(batch, L, dim, N, rank, dt, seed):
    w = inputs.WORKLOADS["mamba130m"].replace(name=f"p{batch}x{L}x{dim}x{N}r{rank}{dt}", batch=batch, seqlen=L,
                                              dim=dim, dstate=N, dtype=dt)
    x = inputs.make_proj(w, rank, seed=seed, device=DEV)
    _announce(w.name)
    got = ss.proj(x["u"], x["W_x"], x["W_dt"], rank)
    torch.cuda.synchronize()
    check(got, oracle_proj(x, rank, N), x["u"].dtype, w.name)


@pytest.mark.parametrize("batch,L,dim,N,rank,dt", [
    (1, 37, 64, 16, 16, "f32"), (2, 100, 136, 16, 48, "f32"), (1, 65, 256, 5, 8, "bf16"),
    (3, 129, 1536, 16, 48, "f32"), (1, 200, 520, 16, 160, "bf16"), (2, 130, 64, 16, 256, "f32"),
    (1, 1, 8, 1, 8, "f32"), (2, 300, 96, 16, 24, "bf16"), (1, 77, 200, 16, 96, "f32"),
    (2, 50, 40, 16, 128, "bf16"), (1, 33, 1032, 7, 192, "f32"), (1, 64, 4096, 16, 128, "bf16"),
])
def test_proj_matches_oracle(batch, L, dim, N, rank, dt):
    run_case(batch, L, dim, N, rank, dt, seed=101)


@pytest.mark.parametrize("rank", [8, 40, 72, 104, 136, 168, 200, 256])
def test_proj_every_step_tile_count(rank):
    """rank -> 2, 3 (fp32; bf16 rounds up to 4), 4, 6, 8, 10, 12 or 16 step tiles of 16
    (zero-padded beyond rank)."""
    run_case(1, 48, 72, 16, rank, "f32", seed=102)
    run_case(1, 48, 72, 16, rank, "bf16", seed=103)


@pytest.mark.parametrize("dt,rank,dim,N,L", [("f32", 48, 64, 16, 40000), ("bf16", 48, 64, 16, 40000),
                                              ("f32", 160, 64, 16, 40000), ("f32", 40, 136, 16, 35001),
                                              ("bf16", 152, 200, 7, 35001), ("bf16", 8, 1032, 16, 33333),
                                              ("f32", 96, 520, 5, 33000)])
def test_proj_token_split_kernel(dt, rank, dim, N, L):
    """Enough tokens (two sequences of L, at least 256 per CU) for the token-split kernel, up to
    10 step tiles: ragged channel groups and lines, dstate below 16, a ragged last workgroup."""
    w = inputs.WORKLOADS["mamba130m"].replace(name=f"ptok{dt}{rank}x{dim}", batch=2, seqlen=L, dim=dim, dstate=N,
                                              dtype=dt)
    x = inputs.make_proj(w, rank, seed=104, device=DEV)
    _announce(w.name)
    got = ss.proj(x["u"], x["W_x"], x["W_dt"], rank)
    torch.cuda.synchronize()
    check(got, oracle_proj(x, rank, N), x["u"].dtype, w.name)


def test_proj_empty_sequence():
    w = inputs.WORKLOADS["mamba130m"].replace(name="p0", batch=2, seqlen=0, dim=64)
    x = inputs.make_proj(w, 16, device=DEV)
    dr, B, C = ss.proj(x["u"], x["W_x"], x["W_dt"], 16)
    torch.cuda.synchronize()
    assert dr.numel() == 0 and B.numel() == 0 and C.numel() == 0


def test_proj_deterministic():
    w = inputs.WORKLOADS["mamba130m"].replace(name="pdet", batch=2, seqlen=300, dim=256)
    x = inputs.make_proj(w, 48, seed=105, device=DEV)
    a = ss.proj(x["u"], x["W_x"], x["W_dt"], 48)
    b = ss.proj(x["u"], x["W_x"], x["W_dt"], 48)
    torch.cuda.synchronize()
    for p, q in zip(a, b):
        assert torch.equal(p, q)


def test_proj_130m_full_every_element():
    w = inputs.WORKLOADS["mamba130m"]
    rank = inputs.proj_rank(w.dim)
    _announce(f"{w.name} full, rank {rank}")
    x = inputs.make_proj(w, rank, seed=106, device=DEV)
    got = ss.proj(x["u"], x["W_x"], x["W_dt"], rank)
    torch.cuda.synchronize()
    check(got, oracle_proj(x, rank, w.dstate), x["u"].dtype, w.name)


@pytest.mark.parametrize("name", ["mamba1.4b", "mamba3b-long"])
def test_proj_full_size_sampled_tokens(name):
    w = inputs.WORKLOADS[name]
    rank = inputs.proj_rank(w.dim)
    _announce(f"{name} sampled tokens, rank {rank}")
    x = inputs.make_proj(w, rank, seed=107, device=DEV)
    got = ss.proj(x["u"], x["W_x"], x["W_dt"], rank)
    torch.cuda.synchronize()
    rng = np.random.default_rng(107)
    k = 96
    tokens = np.stack([rng.integers(0, w.batch, k), rng.integers(0, w.seqlen, k)], axis=1)
    tokens[0] = (w.batch - 1, w.seqlen - 1)  # the very last token, in the last workgroup
    t = torch.as_tensor(tokens, device=DEV)
    check(got, oracle_proj(x, rank, w.dstate, tokens=t), x["u"].dtype, name, tokens=t)


def test_proj_then_scan_matches_oracle():
    """The projections feed the scan: ss_proj then ss_fwd against oracle.proj then oracle.fwd."""
    w = inputs.WORKLOADS["mamba130m"].replace(name="pscan", batch=2, seqlen=257, dim=96)
    rank = 16
    x = inputs.make_proj(w, rank, seed=108, device=DEV)
    s = inputs.make(w, seed=108, device=DEV)
    dr, B, C = ss.proj(x["u"], x["W_x"], x["W_dt"], rank)
    y, st = ss.fwd(x["u"], dr, s["A"], B, C, D=s["D"], z=s["z"], delta_bias=s["delta_bias"])
    torch.cuda.synchronize()
    n = inputs.to_numpy
    odr, oB, oC = oracle_proj(x, rank, w.dstate)
    y_ref, st_ref = oracle.fwd(n(x["u"]).astype(np.float64), odr, n(s["A"]), oB, oC, D=n(s["D"]),
                               z=n(s["z"]).astype(np.float64), delta_bias=n(s["delta_bias"]))
    # the GPU scan sees the fp32-rounded projections; the oracle the exact ones
    assert pu.scaled_err(y.double().cpu().numpy(), y_ref) <= 1e-4
    assert pu.scaled_err(st.double().cpu().numpy(), st_ref) <= 1e-4


# ---- the fused prologue (ss_proj_conv) ----------------------------------------------------------

def conv_params(batch, dim, K, seed, bias=True, state=True):
    g = inputs.HostStream(seed)
    w = (g.randn((dim, K), DEV) * 0.5).contiguous()
    b = g.randn((dim,), DEV) * 0.1 if bias else None
    st = g.randn((batch, dim, K - 1), DEV) if state and K > 1 else None
    return w, b, st


def oracle_proj_conv(x, rank, N, w, b, st):
    n = inputs.to_numpy
    return oracle.proj(n(x["u"]), n(x["W_x"]), n(x["W_dt"]), rank, N, conv_w=w.cpu().numpy(),
                       conv_b=None if b is None else b.cpu().numpy(),
                       conv_state=None if st is None else st.cpu().numpy())


def run_conv_case(batch, L, dim, N, rank, dt, K, seed, bias=True, state=True):
    w = inputs.WORKLOADS["mamba130m"].replace(name=f"pc{batch}x{L}x{dim}x{N}r{rank}{dt}k{K}", batch=batch,
                                              seqlen=L, dim=dim, dstate=N, dtype=dt)
    x = inputs.make_proj(w, rank, seed=seed, device=DEV)
    cw, cb, cs = conv_params(batch, dim, K, seed, bias, state)
    _announce(f"{w.name} bias={bias} state={state}")
    got = ss.proj_conv(x["u"], cw, x["W_x"], x["W_dt"], rank, conv_b=cb, conv_state=cs)
    torch.cuda.synchronize()
    check(got, oracle_proj_conv(x, rank, N, cw, cb, cs), x["u"].dtype, w.name)


@pytest.mark.parametrize("batch,L,dim,N,rank,dt,K", [
    (2, 37, 64, 16, 16, "f32", 4), (3, 20, 136, 16, 48, "f32", 4), (1, 65, 256, 5, 8, "bf16", 4),
    (2, 129, 520, 16, 64, "bf16", 3), (4, 1, 40, 16, 16, "f32", 4), (5, 2, 72, 16, 24, "bf16", 4),
    (2, 3, 96, 16, 32, "f32", 2), (1, 300, 1032, 7, 160, "bf16", 4), (2, 77, 200, 16, 96, "f32", 1),
    (3, 50, 64, 16, 200, "bf16", 4), (1, 40, 48, 16, 256, "f32", 3), (2, 100, 4096, 16, 128, "bf16", 4),
])
def test_proj_conv_matches_oracle(batch, L, dim, N, rank, dt, K):
    """Sequences shorter than the window, sequence starts inside a strip, every kconv, ragged
    channel counts, and one case of each strip count (4 strips up to 4 step tiles, 2 up to 10, 1
    beyond)."""
    run_conv_case(batch, L, dim, N, rank, dt, K, seed=201)


@pytest.mark.parametrize("bias,state", [(False, False), (True, False), (False, True)])
def test_proj_conv_optional_bias_and_state(bias, state):
    run_conv_case(3, 45, 96, 16, 48, "f32", 4, seed=202, bias=bias, state=state)
    run_conv_case(3, 45, 96, 16, 48, "bf16", 4, seed=203, bias=bias, state=state)


def test_proj_conv_130m_full_every_element():
    w = inputs.WORKLOADS["mamba130m"]
    rank = inputs.proj_rank(w.dim)
    _announce(f"{w.name} conv full, rank {rank}")
    x = inputs.make_proj(w, rank, seed=204, device=DEV)
    cw, cb, cs = conv_params(w.batch, w.dim, 4, 204)
    got = ss.proj_conv(x["u"], cw, x["W_x"], x["W_dt"], rank, conv_b=cb, conv_state=cs)
    torch.cuda.synchronize()
    check(got, oracle_proj_conv(x, rank, w.dstate, cw, cb, cs), x["u"].dtype, w.name)


@pytest.mark.parametrize("name", ["mamba1.4b", "mamba3b-long"])
def test_proj_conv_full_size_sampled_tokens(name):
    """At full size the oracle takes each sampled token's window on its own: the convolution
    is causal with kconv = 4, so token t >= 3 depends on x[t-3 .. t] only, a sequence of
    four tokens whose last output is the token's; the first tokens of each sequence are
    checked against the oracle on a prefix of the sequences with the conv state."""
    w = inputs.WORKLOADS[name]
    rank = inputs.proj_rank(w.dim)
    _announce(f"{name} conv sampled tokens, rank {rank}")
    x = inputs.make_proj(w, rank, seed=205, device=DEV)
    cw, cb, cs = conv_params(w.batch, w.dim, 4, 205)
    got = ss.proj_conv(x["u"], cw, x["W_x"], x["W_dt"], rank, conv_b=cb, conv_state=cs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(205)
    k = 64
    tokens = np.stack([rng.integers(0, w.batch, k), rng.integers(3, w.seqlen, k)], axis=1)
    tokens[0] = (w.batch - 1, w.seqlen - 1)
    t = torch.as_tensor(tokens, device=DEV)
    win = torch.stack([x["u"][b, s - 3:s + 1] for b, s in tokens.tolist()])  # (k, 4, dim)
    n = inputs.to_numpy
    ref = oracle.proj(n(win), n(x["W_x"]), n(x["W_dt"]), rank, w.dstate, conv_w=cw.cpu().numpy(),
                      conv_b=cb.cpu().numpy())
    ref = tuple(r[:, 3:4].reshape(1, k, -1) for r in ref)
    check(got, ref, x["u"].dtype, name, tokens=t)
    # the first 40 tokens of every sequence, with the conv state
    P = 40
    ref = oracle.proj(n(x["u"][:, :P]), n(x["W_x"]), n(x["W_dt"]), rank, w.dstate, conv_w=cw.cpu().numpy(),
                      conv_b=cb.cpu().numpy(), conv_state=cs.cpu().numpy())
    check(tuple(g[:, :P] for g in got), ref, x["u"].dtype, name + " prefix")


def test_proj_conv_then_scan_matches_oracle():
    """The block's SSM path from its input: ss_proj_conv then ss_fwd_conv (both form u from x)
    against the oracle's proj with the prologue, then its fwd_conv."""
    w = inputs.WORKLOADS["mamba130m"].replace(name="pcscan", batch=2, seqlen=203, dim=96)
    rank = 16
    x = inputs.make_proj(w, rank, seed=206, device=DEV)
    s = inputs.make(w, seed=206, device=DEV)
    cw, cb, cs = conv_params(w.batch, w.dim, 4, 206)
    dr, B, C = ss.proj_conv(x["u"], cw, x["W_x"], x["W_dt"], rank, conv_b=cb, conv_state=cs)
    y, st = ss.fwd_conv(x["u"], cw, dr, s["A"], B, C, conv_b=cb, conv_state=cs, D=s["D"], z=s["z"],
                        delta_bias=s["delta_bias"])
    torch.cuda.synchronize()
    n = inputs.to_numpy
    odr, oB, oC = oracle_proj_conv(x, rank, w.dstate, cw, cb, cs)
    y_ref, st_ref, _ = oracle.fwd_conv(n(x["u"]).astype(np.float64), cw.cpu().numpy(), odr, n(s["A"]), oB, oC,
                                       conv_b=cb.cpu().numpy(), conv_state=cs.cpu().numpy(), D=n(s["D"]),
                                       z=n(s["z"]).astype(np.float64), delta_bias=n(s["delta_bias"]))
    assert pu.scaled_err(y.double().cpu().numpy(), y_ref) <= 1e-4
    assert pu.scaled_err(st.double().cpu().numpy(), st_ref) <= 1e-4


def test_proj_conv_deterministic():
    w = inputs.WORKLOADS["mamba130m"].replace(name="pcdet", batch=2, seqlen=300, dim=256, dtype="bf16")
    x = inputs.make_proj(w, 48, seed=207, device=DEV)
    cw, cb, cs = conv_params(2, 256, 4, 207)
    a = ss.proj_conv(x["u"], cw, x["W_x"], x["W_dt"], 48, conv_b=cb, conv_state=cs)
    b = ss.proj_conv(x["u"], cw, x["W_x"], x["W_dt"], 48, conv_b=cb, conv_state=cs)
    torch.cuda.synchronize()
    for p, q in zip(a, b):
        assert torch.equal(p, q)
