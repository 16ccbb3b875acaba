"""Pins for the oracle's input projections (ss_oracle_proj): xp = W_x u_t, delta_raw =
W_dt xp[:rank], B = xp[rank:rank+N], C = xp[rank+N:rank+2N], each checked against
something other than the oracle's own loops: numpy's matrix product taken in the other
association order, selection matrices (whose products are exact), rank-1 closed forms,
scaling, exact bf16 widening, and the conv prologue composed with the plain projection.
"""
import numpy as np
import pytest

from tests.test_oracle_pins import assert_close


def f64(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def proj_case(seed, batch=2, L=7, dim=11, N=3, rank=4):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((batch, L, dim)).astype(np.float32)
    W_x = (rng.standard_normal((rank + 2 * N, dim)) / np.sqrt(dim)).astype(np.float32)
    W_dt = (rng.standard_normal((dim, rank)) / np.sqrt(rank)).astype(np.float32)
    return u, W_x, W_dt


def test_matches_numpy_product_other_association(oracle_lib):
    """delta_raw = u (W_dt W_x[:rank])^T: the two maps multiplied first, by numpy."""
    N, rank = 3, 4
    u, W_x, W_dt = proj_case(90, N=N, rank=rank)
    dr, B, C = oracle_lib.proj(u, W_x, W_dt, rank, N)
    Wd = f64(W_dt) @ f64(W_x)[:rank]                   # (dim, dim), then applied to u
    assert_close(dr, f64(u) @ Wd.T, 1e-13, "delta_raw")
    xp = np.einsum("bld,od->blo", f64(u), f64(W_x))
    assert_close(B, xp[..., rank:rank + N], 1e-13, "B")
    assert_close(C, xp[..., rank + N:], 1e-13, "C")


def test_selection_matrices_are_exact(oracle_lib):
    """W_x rows and W_dt rows are unit vectors: every output is one input value, exactly."""
    rng = np.random.default_rng(91)
    batch, L, dim, N, rank = 2, 5, 9, 2, 3
    u = rng.standard_normal((batch, L, dim)).astype(np.float32)
    pick = rng.permutation(dim)[:rank + 2 * N]          # W_x row o selects channel pick[o]
    W_x = np.zeros((rank + 2 * N, dim), np.float32)
    W_x[np.arange(rank + 2 * N), pick] = 1.0
    sel = rng.integers(0, rank, dim)                    # W_dt row d selects xp[sel[d]]
    W_dt = np.zeros((dim, rank), np.float32)
    W_dt[np.arange(dim), sel] = 1.0
    dr, B, C = oracle_lib.proj(u, W_x, W_dt, rank, N)
    uf = f64(u)
    assert np.array_equal(dr, uf[..., pick[sel]])
    assert np.array_equal(B, uf[..., pick[rank:rank + N]])
    assert np.array_equal(C, uf[..., pick[rank + N:]])


def test_rank_one_closed_form(oracle_lib):
    """rank 1: delta_raw[d] = W_dt[d, 0] * <W_x[0], u>."""
    u, W_x, W_dt = proj_case(92, rank=1, N=2)
    dr, _, _ = oracle_lib.proj(u, W_x, W_dt, 1, 2)
    s = np.array([[sum(float(W_x[0, d]) * float(u[b, t, d]) for d in range(u.shape[2]))
                   for t in range(u.shape[1])] for b in range(u.shape[0])])
    assert_close(dr, s[..., None] * f64(W_dt)[:, 0][None, None, :], 1e-13, "rank 1")


def test_scaling_and_additivity(oracle_lib):
    """Linear in u: proj(2 u1 - 3 u2) = 2 proj(u1) - 3 proj(u2) (no bias, no nonlinearity)."""
    N, rank = 2, 3
    u1, W_x, W_dt = proj_case(93, N=N, rank=rank)
    u2, _, _ = proj_case(94, N=N, rank=rank)
    a = oracle_lib.proj(u1, W_x, W_dt, rank, N)
    b = oracle_lib.proj(u2, W_x, W_dt, rank, N)
    c = oracle_lib.proj(2 * f64(u1) - 3 * f64(u2), W_x, W_dt, rank, N)
    for x, y, z, name in zip(a, b, c, ("delta_raw", "B", "C")):
        assert_close(z, 2 * x - 3 * y, 1e-12, name)


def test_bf16_inputs_widen_exactly(oracle_lib):
    N, rank = 2, 3
    u, W_x, W_dt = proj_case(95, N=N, rank=rank)
    hi = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)
    r16 = oracle_lib.proj(hi(u), hi(W_x), hi(W_dt), rank, N)
    r32 = oracle_lib.proj(f64(hi(u)), f64(hi(W_x)).astype(np.float32), f64(hi(W_dt)).astype(np.float32), rank, N)
    for x, y in zip(r16, r32):
        assert np.array_equal(x, y)


def test_conv_prologue_then_projection(oracle_lib):
    """With conv weights, the projection applies to silu(conv(x) + b)."""
    from tests.test_oracle_conv_pins import conv_case, np_conv_silu
    N, rank = 2, 3
    x, w, b, st = conv_case(96, batch=2, L=9, dim=5, K=4)
    _, W_x, W_dt = proj_case(97, dim=5, N=N, rank=rank)
    got = oracle_lib.proj(x, W_x, W_dt, rank, N, conv_w=w, conv_b=b, conv_state=st)
    ref = oracle_lib.proj(np_conv_silu(x, w, b, st), W_x, W_dt, rank, N)
    for g, r, name in zip(got, ref, ("delta_raw", "B", "C")):
        assert_close(g, r, 1e-14, name)


def test_rejects_bad_shapes(oracle_lib):
    u, W_x, W_dt = proj_case(98)
    with pytest.raises(ValueError):
        oracle_lib.proj(u, W_x, W_dt, 5, 3)
