"""Seeded synthetic inputs for the selective-scan workloads.

This module draws random tensors and nothing else: it holds none of the scan's
arithmetic, so both the GPU path and the fp64 oracle can consume what it produces.
Draws use ``torch.Generator`` on the requested device, in a fixed order
(u, delta, z, B, C, D, bias), from a seed derived from the workload name and a
caller seed. bf16 tensors are fp32 draws rounded to nearest even.

Workload shapes are the per-layer scan shapes of Mamba models (d_inner channels,
d_state = 16): 130M (batch 8, L 2048, 1536 ch), 1.4B (batch 4, L 4096, 4096 ch) and
3B long context (batch 1, L 131072, 5120 ch), plus a tiny case and a decode stream.
Value ranges: u, B, C, z, D ~ N(0, 1); raw step ~ N(-2, 1) (N(-4, 1) for the long
context, so that exp(dt*A) stays close to 1); bias ~ U(log(e^0.001 - 1), log(e^0.1 - 1))
so that softplus(bias) spans 0.001 .. 0.1; A[d, n] = -(n + 1).
"""
from __future__ import annotations

import dataclasses
import math
import zlib

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    dim: int
    dstate: int
    dtype: str  # "f32" or "bf16": element type of u, delta, z, B, C
    gated: bool
    delta_dist: tuple  # ("normal", mean, std) or ("uniform", lo, hi)
    bias: str  # "range" (softplus(bias) in 0.001..0.1), "zero" or "none"
    lti: bool = False  # delta[b,:,d], B[b,:,:], C[b,:,:] held constant over t
    steps: int = 0  # > 0: a decode stream of this many single-token steps

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def elems(self) -> int:
        return self.batch * self.seqlen * self.dim


BIAS_LO = math.log(math.expm1(0.001))
BIAS_HI = math.log(math.expm1(0.1))

WORKLOADS = {
    "tiny": Workload("tiny", 1, 64, 16, 4, "f32", True, ("uniform", -4.0, -1.0), "zero"),
    "tiny-lti": Workload("tiny-lti", 1, 64, 16, 4, "f32", True, ("uniform", -4.0, -1.0), "zero",
                         lti=True),
    "mamba130m": Workload("mamba130m", 8, 2048, 1536, 16, "f32", False, ("normal", -2.0, 1.0),
                          "range"),
    "mamba130m-gated": Workload("mamba130m-gated", 8, 2048, 1536, 16, "f32", True,
                                ("normal", -2.0, 1.0), "range"),
    "mamba1.4b": Workload("mamba1.4b", 4, 4096, 4096, 16, "bf16", True, ("normal", -2.0, 1.0),
                          "range"),
    "mamba3b-long": Workload("mamba3b-long", 1, 131072, 5120, 16, "bf16", True,
                             ("normal", -4.0, 1.0), "range"),
    "decode": Workload("decode", 256, 1024, 5120, 16, "f32", True, ("normal", -2.0, 1.0), "range",
                       steps=1024),
}


def sweep_workload(seqlen: int) -> Workload:
    """The long-context shape (batch 1, 5120 channels, bf16, gated) at another length."""
    return WORKLOADS["mamba3b-long"].replace(name=f"mamba3b-L{seqlen}", seqlen=seqlen)


def _seed(name: str, seed: int) -> int:
    return (zlib.crc32(name.encode()) * 1000003 + 86 * 7919 + seed) % (2 ** 62)


def make(w: Workload, seed: int = 0, device="cpu", time_major: bool = False) -> dict:
    """Draw every tensor of workload ``w``.

    Returns a dict with u, delta, z, B, C (w.dtype) and A, D, delta_bias (float32).
    With ``time_major`` the per-token tensors are laid out (seqlen, batch, dim) and
    (seqlen, batch, dstate) so that step t is a contiguous slice (decode streams);
    otherwise (batch, seqlen, dim) and (batch, seqlen, dstate).
    delta_bias is None when w.bias == "none"; z is always drawn (pass it or not).
    """
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(_seed(w.name, seed))
    b, L, d, n = w.batch, w.seqlen, w.dim, w.dstate
    tok = (L, b, d) if time_major else (b, L, d)
    st = (L, b, n) if time_major else (b, L, n)
    f32 = dict(dtype=torch.float32, device=dev, generator=g)

    def normal(shape, mean=0.0, std=1.0):
        return torch.randn(shape, **f32) * std + mean

    def delta_draw(shape):
        kind, p, q = w.delta_dist
        if kind == "normal":
            return normal(shape, p, q)
        return torch.rand(shape, **f32) * (q - p) + p

    if w.lti:
        # one draw per (b, d) / (b, n), repeated along t
        u = normal(tok)
        if time_major:
            delta = delta_draw((1, b, d)).expand(tok).contiguous()
        else:
            delta = delta_draw((b, 1, d)).expand(tok).contiguous()
        z = normal(tok)
        one = (1, b, n) if time_major else (b, 1, n)
        B = normal(one).expand(st).contiguous()
        C = normal(one).expand(st).contiguous()
    else:
        u = normal(tok)
        delta = delta_draw(tok)
        z = normal(tok)
        B = normal(st)
        C = normal(st)
    D = normal((d,))
    if w.bias == "range":
        bias = torch.rand((d,), **f32) * (BIAS_HI - BIAS_LO) + BIAS_LO
    elif w.bias == "zero":
        bias = torch.zeros((d,), dtype=torch.float32, device=dev)
    else:
        bias = None
    A = -torch.arange(1, n + 1, dtype=torch.float32, device=dev).repeat(d, 1).contiguous()
    out = dict(u=u, delta=delta, z=z, B=B, C=C, A=A, D=D, delta_bias=bias)
    if w.dtype == "bf16":
        for k in ("u", "delta", "z", "B", "C"):
            out[k] = out[k].to(torch.bfloat16)
    return out


def proj_rank(dim: int) -> int:
    """Rank of the step projection in the projection workloads: dim / 32 rounded up to a
    multiple of 8 (1536 -> 48, 4096 -> 128, 5120 -> 160)."""
    return max(8, -(-dim // 256) * 8)


def make_proj(w: Workload, rank: int, seed: int = 0, device="cpu") -> dict:
    """Inputs of the projections for workload ``w``: u (batch, seqlen, dim) ~ N(0, 1),
    W_x (rank + 2 dstate, dim) ~ N(0, 1/dim) and W_dt (dim, rank) ~ N(0, 1/rank), so every
    output is O(1); all in w.dtype (bf16: fp32 draws rounded to nearest even)."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(_seed(w.name + "/proj", seed))
    f32 = dict(dtype=torch.float32, device=dev, generator=g)
    d, n = w.dim, w.dstate
    out = dict(u=torch.randn((w.batch, w.seqlen, d), **f32),
               W_x=torch.randn((rank + 2 * n, d), **f32) / math.sqrt(d),
               W_dt=torch.randn((d, rank), **f32) / math.sqrt(rank))
    if w.dtype == "bf16":
        out = {k: v.to(torch.bfloat16) for k, v in out.items()}
    return out


def to_numpy(t):
    """A host numpy view of a tensor for the oracle: float32 stays float32, bfloat16
    becomes uint16 bit patterns. None stays None."""
    if t is None:
        return None
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")
