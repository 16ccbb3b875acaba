"""Out-of-bounds writes: every output of the forward (y, the final state, the conv prologue's
u), of the decode step (the state, updated in place, and y), of the backward (every gradient)
and of the projections (delta_raw, B, C), and the caller's workspace, is carved out of a larger
buffer whose padding holds a sentinel bit pattern. After each call the padding must still
hold it, every output element must have been written (no sentinel left inside), and the
result must be bit-identical to the same call on buffers of their own.

Shapes: ragged channel counts (not a multiple of the 16-channel groups), ragged sequence
tails, dstate 16 and below, every forward kernel and tile plan, the sequence split (with its
workspace padded too), the two-row decode layout and the general one.
"""
import math

import pytest
import torch

import selective_state_space_86_amd as ss
from selective_state_space_86_amd import inputs
from tests import parity_util as pu

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PAD = 16384  # elements of padding on each side
SENT = {torch.float32: (torch.int32, 0x7FA5A5A5), torch.bfloat16: (torch.int16, 0x7FA5),
        torch.uint8: (torch.uint8, 0xA5)}  # a NaN payload no kernel writes


def _announce(msg):
    print(f"\n[canary] {msg}", flush=True)


class Padded:
    """A tensor of `shape` in the middle of a sentinel-filled buffer; `init` (optional)
    becomes its contents (for in-place outputs such as the decode state)."""

    def __init__(self, shape, dtype=torch.float32, init=None):
        self.n = math.prod(shape)
        ity, self.s = SENT[dtype]
        self.buf = torch.empty(2 * PAD + self.n, dtype=dtype, device=DEV)
        self.bits = self.buf.view(ity)
        self.bits.fill_(self.s)
        self.t = self.buf[PAD:PAD + self.n].view(shape)
        if init is not None:
            self.t.copy_(init)

    def check(self, what, written=True):
        torch.cuda.synchronize()
        assert bool((self.bits[:PAD] == self.s).all()), f"{what}: write before the buffer"
        assert bool((self.bits[PAD + self.n:] == self.s).all()), f"{what}: write past the buffer"
        if written:
            assert not bool((self.bits[PAD:PAD + self.n] == self.s).any()), f"{what}: element left unwritten"


def same_bits(a, b, what):
    ity = SENT[a.dtype][0]
    assert torch.equal(a.view(ity), b.view(ity)), f"{what}: differs from the call on plain buffers"


def _make(batch, L, dim, N, dt, seed):
    w = inputs.WORKLOADS["mamba130m"].replace(name=f"c{batch}x{L}x{dim}x{N}{dt}", batch=batch, seqlen=L,
                                              dim=dim, dstate=N, dtype=dt)
    return inputs.make(w, seed=seed, device=DEV)


FWD_SHAPES = [(2, 300, 40, 16, "f32"), (1, 1000, 130, 16, "bf16"), (3, 77, 20, 5, "f32"),
              (1, 4100, 48, 16, "f32"), (2, 1, 17, 16, "bf16")]
# (kernel, chunk_len, chunk_rows, split_parts)
FWD_PLANS = [(0, 0, 0, 0), (1, 0, 0, 0), (3, 0, 0, 0), (2, 4, 16, 0), (2, 8, 32, 0), (2, 4, 12, 0),
             (2, 8, 16, 3), (2, 4, 32, 2)]


@pytest.mark.parametrize("plan", FWD_PLANS)
@pytest.mark.parametrize("batch,L,dim,N,dt", FWD_SHAPES)
def test_forward_outputs_stay_in_bounds(batch, L, dim, N, dt, plan):
    kernel, chunk, rows, parts = plan
    if kernel == 2 and N != 16:
        pytest.skip("the chunked kernel is for dstate 16")
    x = _make(batch, L, dim, N, dt, seed=501)
    _announce(f"fwd {batch}x{L}x{dim}x{N} {dt} plan={plan}")
    h0 = inputs.HostStream(500, L).randn((batch, dim, N), DEV) if L % 2 else None
    kw = dict(kernel=kernel, chunk_len=chunk, chunk_rows=rows, split_parts=parts, h0=h0)
    y_ref, st_ref = pu.gpu_fwd(x, True, **kw)
    need = ss.fwd_workspace_size(batch, L, dim, N, x["u"].dtype, kernel=kernel, chunk_len=chunk,
                                 chunk_rows=rows, split_parts=parts)
    ws = Padded((max(need, 1),), torch.uint8)
    y = Padded((batch, L, dim))
    st = Padded((batch, dim, N))
    pu.gpu_fwd(x, True, y=y.t, last_state=st.t, workspace=ws.t, **kw)
    y.check("y")
    st.check("last_state")
    ws.check("workspace", written=False)
    same_bits(y.t, y_ref, "y")
    same_bits(st.t, st_ref, "last_state")


@pytest.mark.parametrize("kernel,chunk,rows,parts", [(1, 0, 0, 0), (2, 4, 16, 0), (2, 8, 32, 2)])
@pytest.mark.parametrize("batch,L,dim,N,dt,K", [(2, 300, 40, 16, "f32", 4), (1, 777, 130, 16, "bf16", 3)])
def test_conv_forward_outputs_stay_in_bounds(batch, L, dim, N, dt, K, kernel, chunk, rows, parts):
    x = _make(batch, L, dim, N, dt, seed=502)
    _announce(f"fwd_conv {batch}x{L}x{dim}x{N} {dt} K={K} plan={(kernel, chunk, rows, parts)}")
    g = inputs.HostStream(503)
    w = (g.randn((dim, K), DEV) * 0.5).contiguous()
    b = g.randn((dim,), DEV) * 0.1
    cs = g.randn((batch, dim, K - 1), DEV)

    def run(**out):
        return ss.fwd_conv(x["u"], w, x["delta"], x["A"], x["B"], x["C"], conv_b=b, conv_state=cs, D=x["D"],
                           z=x["z"], delta_bias=x["delta_bias"], kernel=kernel, chunk_len=chunk,
                           chunk_rows=rows, split_parts=parts, **out)

    y_ref, st_ref, u_ref = run(u_out=True)
    y, st, u = Padded((batch, L, dim)), Padded((batch, dim, N)), Padded((batch, L, dim))
    run(y=y.t, last_state=st.t, u_out=u.t)
    for p, r, name in ((y, y_ref, "y"), (st, st_ref, "last_state"), (u, u_ref, "u_out")):
        p.check(name)
        same_bits(p.t, r, name)


@pytest.mark.parametrize("batch,dim,N,dt,zoh", [(2, 128, 16, "bf16", False), (4, 192, 16, "f32", True),
                                               (3, 100, 16, "f32", False), (5, 130, 16, "bf16", True),
                                               (2, 64, 5, "f32", False), (1, 1, 16, "f32", False)])
def test_decode_step_outputs_stay_in_bounds(batch, dim, N, dt, zoh):
    w = inputs.WORKLOADS["decode"].replace(name=f"cd{batch}x{dim}x{N}{dt}", batch=batch, seqlen=5, dim=dim,
                                           dstate=N, dtype=dt)
    x = inputs.make(w, seed=504, device=DEV, time_major=True)
    _announce(f"step {batch}x{dim}x{N} {dt} zoh={zoh}")
    st0 = inputs.HostStream(505).randn((batch, dim, N), DEV)
    ref = st0.clone()
    st = Padded((batch, dim, N), init=st0)
    for t in range(x["u"].shape[0]):
        args = (x["u"][t], x["delta"][t], x["A"], x["B"][t], x["C"][t])
        kw = dict(D=x["D"], z=x["z"][t], delta_bias=x["delta_bias"], zoh=zoh)
        y_ref = ss.step(ref, *args, **kw)
        y = Padded((batch, dim))
        ss.step(st.t, *args, y=y.t, **kw)
        y.check(f"y at step {t}")
        st.check(f"state at step {t}")
        same_bits(y.t, y_ref, f"y at step {t}")
        same_bits(st.t, ref, f"state at step {t}")


BWD_KEYS = ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0")


@pytest.mark.parametrize("batch,L,dim,N,dt", [(2, 300, 40, 16, "f32"), (1, 777, 130, 16, "bf16"),
                                              (3, 64, 20, 5, "f32"), (2, 1, 16, 16, "f32")])
def test_backward_gradients_stay_in_bounds(batch, L, dim, N, dt):
    x = _make(batch, L, dim, N, dt, seed=505)
    _announce(f"bwd {batch}x{L}x{dim}x{N} {dt}")
    g = inputs.HostStream(506)
    dy = g.randn((batch, L, dim), DEV)
    h0 = g.randn((batch, dim, N), DEV)
    dlast = g.randn((batch, dim, N), DEV)

    def run(**kw):
        return ss.bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"],
                      delta_bias=x["delta_bias"], h0=h0, dlast=dlast, **kw)

    ref = run()
    shapes = dict(du=(batch, L, dim), ddelta=(batch, L, dim), dz=(batch, L, dim), dA=(dim, N),
                  dB=(batch, L, N), dC=(batch, L, N), dD=(dim,), ddelta_bias=(dim,), dh0=(batch, dim, N))
    pads = {k: Padded(s) for k, s in shapes.items()}
    ws = Padded((max(ss.bwd_workspace_size(batch, L, dim, N), 1),), torch.uint8)
    run(out={k: p.t for k, p in pads.items()}, workspace=ws.t)
    for k in BWD_KEYS:
        pads[k].check(k)
        same_bits(pads[k].t, ref[k], k)
    ws.check("workspace", written=False)


def test_backward_split_gradients_stay_in_bounds():
    """~1.2 channel groups per CU: 8-wave tiles and the sequence split in both of the
    backward's scans, whose hand-off region lives in the (padded) workspace."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    batch, L, dim, N = 1, 700, 16 * int(cus * 1.2) - 5, 16
    x = _make(batch, L, dim, N, "bf16", seed=507)
    _announce(f"bwd split {batch}x{L}x{dim}x{N}")
    dy = inputs.HostStream(507).randn((batch, L, dim), DEV)

    def run(**kw):
        return ss.bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"],
                      delta_bias=x["delta_bias"], **kw)

    ref = run()
    shapes = dict(du=(batch, L, dim), ddelta=(batch, L, dim), dz=(batch, L, dim), dA=(dim, N),
                  dB=(batch, L, N), dC=(batch, L, N), dD=(dim,), ddelta_bias=(dim,), dh0=(batch, dim, N))
    pads = {k: Padded(s) for k, s in shapes.items()}
    ws = Padded((ss.bwd_workspace_size(batch, L, dim, N),), torch.uint8)
    run(out={k: p.t for k, p in pads.items()}, workspace=ws.t)
    for k in BWD_KEYS:
        pads[k].check(k)
        same_bits(pads[k].t, ref[k], k)
    ws.check("workspace", written=False)


@pytest.mark.parametrize("batch,L,dim,N,rank,dt,K", [
    (2, 100, 136, 16, 48, "f32", 0), (1, 65, 256, 5, 8, "bf16", 0), (2, 40000, 64, 16, 48, "bf16", 0),
    (3, 20, 136, 16, 48, "f32", 4), (1, 300, 1032, 7, 160, "bf16", 4),
])
def test_projection_outputs_stay_in_bounds(batch, L, dim, N, rank, dt, K):
    w = inputs.WORKLOADS["mamba130m"].replace(name=f"cp{batch}x{L}x{dim}x{N}r{rank}{dt}", batch=batch,
                                              seqlen=L, dim=dim, dstate=N, dtype=dt)
    x = inputs.make_proj(w, rank, seed=508, device=DEV)
    _announce(f"proj {w.name} K={K}")
    tdt = x["u"].dtype
    if K:
        g = inputs.HostStream(509)
        cw = (g.randn((dim, K), DEV) * 0.5).contiguous()

        def run(**o):
            return ss.proj_conv(x["u"], cw, x["W_x"], x["W_dt"], rank, **o)
    else:
        def run(**o):
            return ss.proj(x["u"], x["W_x"], x["W_dt"], rank, **o)
    ref = run()
    pads = [Padded((batch, L, dim), tdt), Padded((batch, L, N), tdt), Padded((batch, L, N), tdt)]
    run(delta_raw=pads[0].t, B=pads[1].t, C=pads[2].t)
    for p, r, name in zip(pads, ref, ("delta_raw", "B", "C")):
        p.check(name)
        same_bits(p.t, r, name)
