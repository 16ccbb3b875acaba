"""Seeded synthetic inputs for the selective-scan workloads.

This module draws random tensors and nothing else: it holds none of the scan's
arithmetic, so both the GPU path and the fp64 oracle can consume what it produces.

Draws (the same on every host): numpy PCG64 streams keyed by
``SeedSequence([86, config, tensor, chunk])`` (a caller seed other than 0 is appended),
in the order u, delta, z, B, C, D, bias (tensor ids 0..6). Per-token tensors are drawn in
chunks of 4096 tokens of one batch row (chunk = row * chunks_per_row + index), each chunk
as (tokens, width) in token-major order, so a draw does not depend on how the tokens are
later grouped into calls or launches, and a shorter sequence draws a prefix of a longer
one. Values are drawn in fp64, rounded to fp32 (nearest even) and, for bf16 tensors, to
bf16 (nearest even). Every length is drawn this way, the longest sweep point (2^20 tokens of
5120 channels) included, chunks in parallel on up to 16 host threads. The projection inputs
(``make_proj``) follow the same recipe with tensor ids 7..9.

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
import os
import zlib
from concurrent.futures import ThreadPoolExecutor

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


# configuration ids of the seed key: the tiny case 1, 130M 2, 1.4B 3, 3B long context 4 (and
# its length sweep, which draws prefixes of the same streams), decode 5; other shapes (tests)
# a number derived from their name
CONFIG_IDS = {"tiny": 1, "tiny-lti": 1, "mamba130m": 2, "mamba130m-gated": 2, "mamba1.4b": 3,
              "mamba3b-long": 4, "decode": 5}
TENSOR_IDS = {"u": 0, "delta": 1, "z": 2, "B": 3, "C": 4, "D": 5, "bias": 6,
              "proj_u": 7, "W_x": 8, "W_dt": 9}
CHUNK = 4096


def config_id(w: Workload) -> int:
    if w.name in CONFIG_IDS:
        return CONFIG_IDS[w.name]
    if w.name.startswith("mamba3b-L"):
        return 4
    return 1000 + zlib.crc32(w.name.encode()) % 1_000_000


def _rng(cfg: int, tensor: str, chunk: int, seed: int) -> np.random.Generator:
    key = [86, cfg, TENSOR_IDS[tensor], chunk] + ([seed] if seed else [])
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def _draw(rng, dist, count):
    """fp64 draws rounded to fp32 (nearest even)."""
    kind, p, q = dist
    v = rng.standard_normal(count) * q + p if kind == "normal" else rng.uniform(p, q, count)
    return v.astype(np.float32)


def _bf16_bits(f32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, rounded to nearest even (finite inputs)."""
    b = f32.view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _host_tokens(w: Workload, cfg: int, tensor: str, dist, width: int, seed: int, pool) -> np.ndarray:
    """A per-token tensor (batch, seqlen, width), drawn chunk by chunk, in the workload's
    element type (bf16 as uint16 bit patterns)."""
    b, L = w.batch, w.seqlen
    nch = -(-L // CHUNK)
    out = np.empty((b, L, width), dtype=np.uint16 if w.dtype == "bf16" else np.float32)

    def one(job):
        r, c = job
        t0, t1 = c * CHUNK, min(L, (c + 1) * CHUNK)
        v = _draw(_rng(cfg, tensor, r * nch + c, seed), dist, (t1 - t0) * width).reshape(t1 - t0, width)
        out[r, t0:t1] = _bf16_bits(v) if w.dtype == "bf16" else v

    list(pool.map(one, [(r, c) for r in range(b) for c in range(nch)]))
    return out


def _host_rows(w: Workload, cfg: int, tensor: str, dist, width: int, seed: int) -> np.ndarray:
    """One draw per batch row, (batch, width) fp32 (the LTI case's per-row values)."""
    return np.stack([_draw(_rng(cfg, tensor, r, seed), dist, width) for r in range(w.batch)])


def _torch_of(a: np.ndarray, bf16: bool, dev) -> torch.Tensor:
    t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if bf16 else torch.from_numpy(a)
    return t.to(dev)


def make(w: Workload, seed: int = 0, device="cpu", time_major: bool = False) -> dict:
    """Draw every tensor of workload ``w``.

    Returns a dict with u, delta, z, B, C (w.dtype) and A, D, delta_bias (float32).
    With ``time_major`` the per-token tensors are laid out (seqlen, batch, dim) and
    (seqlen, batch, dstate) so that step t is a contiguous slice (decode streams);
    otherwise (batch, seqlen, dim) and (batch, seqlen, dstate). The values do not depend
    on the layout. delta_bias is None when w.bias == "none"; z is always drawn (pass it
    or not).
    """
    dev = torch.device(device)
    cfg = config_id(w)
    b, L, d, n = w.batch, w.seqlen, w.dim, w.dstate
    bf = w.dtype == "bf16"
    normal = ("normal", 0.0, 1.0)
    out = {}
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as pool:
        if w.lti:
            # one draw per (b, d) / (b, n), repeated along t
            out["u"] = _host_tokens(w, cfg, "u", normal, d, seed, pool)
            rows = {"delta": (w.delta_dist, d), "B": (normal, n), "C": (normal, n)}
            for k in ("delta", "z", "B", "C"):
                if k == "z":
                    out[k] = _host_tokens(w, cfg, "z", normal, d, seed, pool)
                    continue
                dist, width = rows[k]
                v = np.ascontiguousarray(np.broadcast_to(_host_rows(w, cfg, k, dist, width, seed)[:, None, :],
                                                         (b, L, width)))
                out[k] = _bf16_bits(v) if bf else v
        else:
            out["u"] = _host_tokens(w, cfg, "u", normal, d, seed, pool)
            out["delta"] = _host_tokens(w, cfg, "delta", w.delta_dist, d, seed, pool)
            out["z"] = _host_tokens(w, cfg, "z", normal, d, seed, pool)
            out["B"] = _host_tokens(w, cfg, "B", normal, n, seed, pool)
            out["C"] = _host_tokens(w, cfg, "C", normal, n, seed, pool)
    res = {}
    for k in ("u", "delta", "z", "B", "C"):
        a = out[k]
        if time_major:
            a = np.ascontiguousarray(a.transpose(1, 0, 2))
        res[k] = _torch_of(a, bf, dev)
    res["D"] = torch.from_numpy(_draw(_rng(cfg, "D", 0, seed), normal, d)).to(dev)
    if w.bias == "range":
        res["delta_bias"] = torch.from_numpy(_draw(_rng(cfg, "bias", 0, seed), ("uniform", BIAS_LO, BIAS_HI),
                                                   d)).to(dev)
    elif w.bias == "zero":
        res["delta_bias"] = torch.zeros((d,), dtype=torch.float32, device=dev)
    else:
        res["delta_bias"] = None
    res["A"] = -torch.arange(1, n + 1, dtype=torch.float32, device=dev).repeat(d, 1).contiguous()
    return {k: res[k] for k in ("u", "delta", "z", "B", "C", "A", "D", "delta_bias")}


def proj_rank(dim: int) -> int:
    """Rank of the step projection in the projection workloads: dim / 32 rounded up to a
    multiple of 8 (1536 -> 48, 4096 -> 128, 5120 -> 160)."""
    return max(8, -(-dim // 256) * 8)


def make_proj(w: Workload, rank: int, seed: int = 0, device="cpu") -> dict:
    """Inputs of the projections for workload ``w``: u (batch, seqlen, dim) ~ N(0, 1),
    W_x (rank + 2 dstate, dim) ~ N(0, 1/dim) and W_dt (dim, rank) ~ N(0, 1/rank), so every
    output is O(1); all in w.dtype (bf16: fp32 draws rounded to nearest even). Host PCG64
    streams as in ``make`` (u in 4096-token chunks, tensor ids 7, 8, 9; each weight matrix
    one stream, row-major)."""
    dev = torch.device(device)
    cfg = config_id(w)
    d, n = w.dim, w.dstate
    bf = w.dtype == "bf16"
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as pool:
        u = _host_tokens(w, cfg, "proj_u", ("normal", 0.0, 1.0), d, seed, pool)
    wx = _draw(_rng(cfg, "W_x", 0, seed), ("normal", 0.0, 1.0 / math.sqrt(d)),
               (rank + 2 * n) * d).reshape(rank + 2 * n, d)
    wdt = _draw(_rng(cfg, "W_dt", 0, seed), ("normal", 0.0, 1.0 / math.sqrt(rank)), d * rank).reshape(d, rank)
    if bf:
        wx, wdt = _bf16_bits(wx), _bf16_bits(wdt)
    return dict(u=_torch_of(u, bf, dev), W_x=_torch_of(wx, bf, dev), W_dt=_torch_of(wdt, bf, dev))


class HostStream:
    """A seeded host stream for a test's own extra tensors (initial states, output
    gradients, conv taps, shapes of its own): numpy PCG64 keyed by
    ``SeedSequence([86, 99, *key])``, drawn in fp64 and rounded to fp32, then copied to the
    device, so every such draw is also the same on every host. Successive calls continue
    the one stream in call order."""

    def __init__(self, *key: int):
        self._rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([86, 99, *key])))

    def _out(self, v: np.ndarray, shape, device) -> torch.Tensor:
        return torch.from_numpy(v.astype(np.float32).reshape(shape)).to(device)

    def randn(self, shape, device="cpu") -> torch.Tensor:
        """N(0, 1) values of the given shape, float32."""
        return self._out(self._rng.standard_normal(math.prod(shape)), shape, device)

    def rand(self, shape, device="cpu") -> torch.Tensor:
        """U[0, 1) values of the given shape, float32."""
        return self._out(self._rng.random(math.prod(shape)), shape, device)


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
