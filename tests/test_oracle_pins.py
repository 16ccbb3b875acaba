"""Pins for the fp64 oracle: each test checks it against something other than itself.

- LTI case equals the explicit causal convolution with K_k = sum_n C[n] abar[n]^k dt B[n]
  (page "架构变体：Mamba/SSM", section "并行卷积", and its Python demo);
- a zero step leaves the state unchanged and a huge step resets it (page
  "从RNN到Mamba…", section 2, the two limits of the step size);
- constant inputs follow the geometric series;
- tiny cases equal the fully unrolled double sum;
- the page-5 demo values (exact decimals, tests/golden);
- splitting the sequence, stepping token by token, causality and linearity in u;
- the exact zero-order-hold option: the exact solution of h' = A h + B u for inputs held
  constant over each step (page "架构变体：Mamba/SSM", section "离散化"), so it matches
  the continuous-time solution for any step sizes and two half steps equal one step.
Reference numbers here come from numpy/scipy formulas written independently of the
oracle's loop (convolution, closed forms, explicit sums), never from the oracle itself.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def softplus_ref(x):
    return np.logaddexp(0.0, x)


def silu_ref(z):
    return z * expit(z)


def rand_case(rng, batch=2, L=17, dim=3, N=5, lti=False, gated=True, with_D=True, bias=True):
    f = np.float32
    u = rng.standard_normal((batch, L, dim)).astype(f)
    if lti:
        delta = np.repeat(rng.uniform(-3, 0.5, (batch, 1, dim)), L, axis=1).astype(f)
        B = np.repeat(rng.standard_normal((batch, 1, N)), L, axis=1).astype(f)
        C = np.repeat(rng.standard_normal((batch, 1, N)), L, axis=1).astype(f)
    else:
        delta = rng.uniform(-3, 0.5, (batch, L, dim)).astype(f)
        B = rng.standard_normal((batch, L, N)).astype(f)
        C = rng.standard_normal((batch, L, N)).astype(f)
    # channel-dependent, non-square A so a transposed index cannot go unnoticed
    A = (-rng.uniform(0.2, 2.0, (dim, N))).astype(f)
    D = rng.standard_normal(dim).astype(f) if with_D else None
    z = rng.standard_normal((batch, L, dim)).astype(f) if gated else None
    bias_v = rng.uniform(-1.0, 0.5, dim).astype(f) if bias else None
    return dict(u=u, delta=delta, A=A, B=B, C=C, D=D, z=z, delta_bias=bias_v)


def f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def bf16_bits_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def step_sizes(c, softplus=True):
    x = f64(c["delta"]) + (0.0 if c["delta_bias"] is None else f64(c["delta_bias"])[None, None, :])
    return softplus_ref(x) if softplus else x


def zoh_coef(dt, A):
    """(exp(dt A) - 1) / A, with its A -> 0 limit dt (numpy expm1; broadcasts)."""
    A = np.asarray(A, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.expm1(dt * A) / A
    return np.where(A == 0.0, dt, q)


def brute_force(c, softplus=True, zoh=False):
    """Unrolled closed form: y_t = sum_{s<=t} sum_n C_t[n] exp(A[d,n] sum_{r=s+1..t} dt_r)
    bbar_s[n] B_s[n] u_s + D u_t, times silu(z_t); also the final state. bbar_s = dt_s, or
    the exact zero-order-hold (exp(dt_s A) - 1)/A with zoh."""
    u, B, C, A = f64(c["u"]), f64(c["B"]), f64(c["C"]), f64(c["A"])
    dt = step_sizes(c, softplus)
    batch, L, dim = u.shape
    N = A.shape[1]
    y = np.zeros((batch, L, dim))
    last = np.zeros((batch, dim, N))
    for b in range(batch):
        for d in range(dim):
            cum = np.concatenate([[0.0], np.cumsum(dt[b, :, d])])  # cum[k] = sum_{r<k} dt_r
            for t in range(L):
                tot = 0.0
                for s in range(t + 1):
                    decay = np.exp(A[d] * (cum[t + 1] - cum[s + 1]))  # sum_{r=s+1..t} dt_r
                    coef = zoh_coef(dt[b, s, d], A[d]) if zoh else dt[b, s, d]
                    tot += np.sum(C[b, t] * decay * coef * B[b, s] * u[b, s, d])
                if c["D"] is not None:
                    tot += f64(c["D"])[d] * u[b, t, d]
                if c["z"] is not None:
                    tot *= silu_ref(f64(c["z"])[b, t, d])
                y[b, t, d] = tot
            for s in range(L):
                decay = np.exp(A[d] * (cum[L] - cum[s + 1]))
                coef = zoh_coef(dt[b, s, d], A[d]) if zoh else dt[b, s, d]
                last[b, d] += decay * coef * B[b, s] * u[b, s, d]
    return y, last


def assert_close(got, ref, rtol, what=""):
    scale = 1.0 + np.abs(ref)
    err = np.max(np.abs(got - ref) / scale) if ref.size else 0.0
    assert err <= rtol, f"{what}: max scaled error {err:.3e} > {rtol:.1e}"


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("with_D", [False, True])
def test_brute_force_unrolled_sum(oracle_lib, gated, with_D):
    rng = np.random.default_rng(1)
    c = rand_case(rng, gated=gated, with_D=with_D)
    y, last = oracle_lib.fwd(**c, softplus=True)
    y_ref, last_ref = brute_force(c, softplus=True)
    assert_close(y, y_ref, 1e-12, "y")
    assert_close(last, last_ref, 1e-12, "last_state")


def test_brute_force_no_softplus_no_bias(oracle_lib):
    rng = np.random.default_rng(2)
    c = rand_case(rng, bias=False)
    c["delta"] = rng.uniform(0.01, 0.8, c["delta"].shape).astype(np.float32)
    y, last = oracle_lib.fwd(**c, softplus=False)
    y_ref, last_ref = brute_force(c, softplus=False)
    assert_close(y, y_ref, 1e-12, "y")
    assert_close(last, last_ref, 1e-12, "last_state")


def test_brute_force_bf16_inputs(oracle_lib):
    """bf16 bit patterns decode exactly: same unrolled sum on the decoded values."""
    rng = np.random.default_rng(3)
    c = rand_case(rng)
    cb = dict(c)
    for k in ("u", "delta", "B", "C", "z"):
        bits = (c[k].view(np.uint32) >> 16).astype(np.uint16)  # truncation is fine for a test
        cb[k] = bits
    y, last = oracle_lib.fwd(**cb, softplus=True)
    cf = dict(c)
    for k in ("u", "delta", "B", "C", "z"):
        cf[k] = bf16_bits_to_f64(cb[k])
    y_ref, last_ref = brute_force(cf, softplus=True)
    assert_close(y, y_ref, 1e-12, "y")
    assert_close(last, last_ref, 1e-12, "last_state")


@pytest.mark.parametrize("gated", [False, True])
def test_lti_equals_convolution(oracle_lib, gated):
    """Page 5, section '并行卷积': with constant dt, B, C the scan is a causal convolution
    with kernel K_k = sum_n C[n] abar[n]^k dt B[n] (np.convolve as in the page's demo)."""
    rng = np.random.default_rng(4)
    c = rand_case(rng, batch=2, L=96, dim=4, N=6, lti=True, gated=gated)
    y, _ = oracle_lib.fwd(**c, softplus=True)
    dt = step_sizes(c)
    A = f64(c["A"])
    L = c["u"].shape[1]
    k = np.arange(L)
    for b in range(2):
        for d in range(4):
            dtv = dt[b, 0, d]
            abar = np.exp(dtv * A[d])
            K = np.sum(f64(c["C"])[b, 0][None, :] * abar[None, :] ** k[:, None] * dtv *
                       f64(c["B"])[b, 0][None, :], axis=1)
            uu = f64(c["u"])[b, :, d]
            yr = np.convolve(K, uu)[:L] + f64(c["D"])[d] * uu
            if gated:
                yr = yr * silu_ref(f64(c["z"])[b, :, d])
            assert_close(y[b, :, d], yr, 1e-11, f"conv b={b} d={d}")


def test_geometric_series_constant_inputs(oracle_lib):
    """Constant u, dt, B, C: h_t[n] = dt B[n] u (1 - abar^(t+1)) / (1 - abar)."""
    L, dim, N = 200, 2, 5
    f = np.float32
    u = np.full((1, L, dim), 0.75, f)
    delta = np.full((1, L, dim), -1.5, f)
    B = np.tile(np.array([0.3, -1.1, 0.7, 2.0, -0.4], f), (1, L, 1))
    C = np.tile(np.array([1.2, 0.5, -0.9, 0.25, 1.7], f), (1, L, 1))
    A = np.array([[-0.5, -1.0, -1.5, -2.0, -3.0], [-0.1, -0.2, -0.3, -0.4, -0.5]], f)
    D = np.array([0.6, -1.3], f)
    z = np.full((1, L, dim), 0.4, f)
    y, last = oracle_lib.fwd(u, delta, A, B, C, D=D, z=z, softplus=True)
    t = np.arange(L)[:, None]
    for d in range(dim):
        dt = math.log1p(math.exp(-1.5))
        la = dt * f64(A[d])  # log of abar
        bu = dt * f64(B[0, 0]) * 0.75
        h = bu[None, :] * (-np.expm1((t + 1) * la[None, :])) / (-np.expm1(la))[None, :]
        zv = float(z[0, 0, 0])  # the fp32 rounding of 0.4 that the oracle receives
        yr = (h @ f64(C[0, 0]) + f64(D[d]) * 0.75) * zv * expit(zv)
        assert_close(y[0, :, d], yr, 1e-12, "geometric y")
        assert_close(last[0, d], h[-1], 1e-12, "geometric state")


def test_zero_step_keeps_state_exactly(oracle_lib):
    """Softplus off, delta = bias = 0: abar = exp(0) = 1 and the input term is 0, so the
    state stays h0 bit for bit and y_t = (C_t . h0 + D u_t) silu(z_t)."""
    rng = np.random.default_rng(5)
    c = rand_case(rng, bias=False)
    c["delta"] = np.zeros_like(c["delta"])
    h0 = rng.standard_normal((2, 3, 5))
    y, last = oracle_lib.fwd(**c, softplus=False, h0=h0)
    assert np.array_equal(last, h0)
    yr = np.einsum("btn,bdn->btd", f64(c["C"]), h0) + f64(c["D"])[None, None, :] * f64(c["u"])
    yr *= silu_ref(f64(c["z"]))
    assert_close(y, yr, 1e-13, "y with frozen state")
    # the decode step with a zero step size leaves a carried state unchanged as well
    st = h0.copy()
    oracle_lib.step(st, c["u"][:, 0], c["delta"][:, 0], c["A"], c["B"][:, 0], c["C"][:, 0],
                    D=c["D"], z=c["z"][:, 0], softplus=False)
    assert np.array_equal(st, h0)


def test_tiny_softplus_step_changes_state_negligibly(oracle_lib):
    rng = np.random.default_rng(6)
    c = rand_case(rng, bias=False)
    c["delta"] = np.full_like(c["delta"], -50.0)  # softplus(-50) ~ 2e-22
    h0 = rng.standard_normal((2, 3, 5))
    _, last = oracle_lib.fwd(**c, softplus=True, h0=h0)
    assert np.max(np.abs(last - h0)) < 1e-19


def test_huge_step_resets_state(oracle_lib):
    """Softplus off, step 1e4: exp(dt*A) underflows to 0, so h_t = (dt B_t) u_t exactly."""
    rng = np.random.default_rng(7)
    c = rand_case(rng, bias=False, gated=False)
    c["delta"] = np.full_like(c["delta"], 1.0e4)
    h0 = rng.standard_normal((2, 3, 5))
    y, last = oracle_lib.fwd(**c, softplus=False, h0=h0)
    hlast = (1.0e4 * f64(c["B"])[:, -1, None, :]) * f64(c["u"])[:, -1, :, None]
    assert np.array_equal(last, hlast)
    hall = (1.0e4 * f64(c["B"])[:, :, None, :]) * f64(c["u"])[:, :, :, None]  # (b,t,d,n)
    yr = np.einsum("btn,btdn->btd", f64(c["C"]), hall) + f64(c["D"]) * f64(c["u"])
    assert_close(y, yr, 1e-13, "reset y")


def test_page5_worked_example(oracle_lib):
    """The page-5 LTI demo through the S6 interface (exact decimal results)."""
    g = json.load(open(os.path.join(GOLDEN, "page5_lti_example.json")))
    x = np.array([float(v) for v in g["x"]], np.float32)
    L = len(x)
    u = x.reshape(1, L, 1)
    delta = np.ones((1, L, 1), np.float32)
    A = np.array([[math.log(0.9)]], np.float32)
    B = np.full((1, L, 1), 0.2, np.float32)
    C = np.full((1, L, 1), 1.0, np.float32)
    y, last = oracle_lib.fwd(u, delta, A, B, C, softplus=False)
    # the fp32 inputs (0.2, x, ln 0.9) are roundings of the page's decimals: 1e-6 relative
    want = np.array([float(Fraction(v)) for v in g["y"]])
    assert np.max(np.abs(y[0, :, 0] - want)) < 2e-7
    assert abs(last[0, 0, 0] - want[-1]) < 2e-7
    # the page's own check: the same numbers from the convolution with K_k = C B A^k
    K = np.array([float(Fraction(v)) for v in g["conv_kernel"]])
    assert np.allclose(np.convolve(K, [float(Fraction(v)) for v in g["x"]])[:L], want, rtol=0, atol=1e-15)
    # exact rational recurrence from the page's decimals reproduces the stored values
    h = Fraction(0)
    for xv, yv in zip(g["x"], g["y"]):
        h = Fraction(g["A_decay"]) * h + Fraction(g["B"]) * Fraction(xv)
        assert Fraction(g["C"]) * h == Fraction(yv)


def _load_selective_generator():
    import importlib.util
    spec = importlib.util.spec_from_file_location("make_page5_selective",
                                                  os.path.join(GOLDEN, "make_page5_selective.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_page5_selective_example(oracle_lib):
    """The page-5 selective demo (write weight B_t = B_base * sigmoid(x_t), so B changes every
    step) through the S6 interface, against 50-digit decimal values of its definition."""
    g = json.load(open(os.path.join(GOLDEN, "page5_selective_example.json")))
    # the stored values are the definition's: the generator re-derives them digit for digit
    gen = _load_selective_generator()
    b, y = gen.derive(g["x"])
    assert [f"{v:.30g}" for v in b] == g["B_t"] and [f"{v:.30g}" for v in y] == g["y"]
    L = len(g["x"])
    u = np.array([float(v) for v in g["x"]], np.float64).reshape(1, L, 1)
    delta = np.ones((1, L, 1), np.float64)
    B = np.array([float(v) for v in g["B_t"]], np.float64).reshape(1, L, 1)
    C = np.full((1, L, 1), float(g["C"]), np.float64)
    A = np.array([[math.log(0.9)]], np.float32)
    y_or, last = oracle_lib.fwd(u, delta, A, B, C, softplus=False)
    want = np.array([float(v) for v in g["y"]])
    # A = ln 0.9 rounded to fp32 (within 3.8e-9): exp(A) is 0.9 to 4e-9 relative, which moves
    # y_t by at most t * 4e-9 * sum|terms| < 5e-9 here; the fp64 inputs and arithmetic add ~1e-16
    assert np.max(np.abs(y_or[0, :, 0] - want)) < 1e-8
    assert abs(last[0, 0, 0] - want[-1]) < 1e-8


def test_split_sequence_matches_one_pass(oracle_lib):
    """Associativity of the update: [0, t0) then [t0, L) from the carried state is
    bit-identical to one pass."""
    rng = np.random.default_rng(8)
    c = rand_case(rng, L=40)
    y, last = oracle_lib.fwd(**c)
    t0 = 13
    c1 = {k: (v[:, :t0] if k in ("u", "delta", "B", "C", "z") and v is not None else v) for k, v in c.items()}
    c2 = {k: (v[:, t0:] if k in ("u", "delta", "B", "C", "z") and v is not None else v) for k, v in c.items()}
    y1, s1 = oracle_lib.fwd(**c1)
    y2, s2 = oracle_lib.fwd(**c2, h0=s1)
    assert np.array_equal(np.concatenate([y1, y2], axis=1), y)
    assert np.array_equal(s2, last)


def test_step_by_step_matches_forward(oracle_lib):
    rng = np.random.default_rng(9)
    c = rand_case(rng, L=25)
    y, last = oracle_lib.fwd(**c)
    st = np.zeros((2, 3, 5))
    for t in range(25):
        yt = oracle_lib.step(st, c["u"][:, t], c["delta"][:, t], c["A"], c["B"][:, t], c["C"][:, t],
                             D=c["D"], z=c["z"][:, t], delta_bias=c["delta_bias"])
        assert np.array_equal(yt, y[:, t])
    assert np.array_equal(st, last)


def test_causality(oracle_lib):
    rng = np.random.default_rng(10)
    c = rand_case(rng, L=30)
    y, _ = oracle_lib.fwd(**c)
    c2 = dict(c)
    c2["u"] = c["u"].copy()
    c2["u"][:, 17] += 3.0
    y2, _ = oracle_lib.fwd(**c2)
    assert np.array_equal(y[:, :17], y2[:, :17])
    assert not np.array_equal(y[:, 17:], y2[:, 17:])


def test_linearity_in_u(oracle_lib):
    rng = np.random.default_rng(11)
    c = rand_case(rng, gated=False)
    # values on a 2^-10 grid below 2^4 in magnitude, so a*u1 + b*u2 is exact in fp32
    u1 = (np.round(rng.standard_normal(c["u"].shape) * 1024) / 1024).astype(np.float32)
    u2 = (np.round(rng.standard_normal(c["u"].shape) * 1024) / 1024).astype(np.float32)
    a, b = 0.5, -2.0
    u3 = (a * u1.astype(np.float64) + b * u2.astype(np.float64)).astype(np.float32)
    y1, s1 = oracle_lib.fwd(**dict(c, u=u1))
    y2, s2 = oracle_lib.fwd(**dict(c, u=u2))
    y3, s3 = oracle_lib.fwd(**dict(c, u=u3))
    assert_close(y3, a * y1 + b * y2, 1e-12, "linearity y")
    assert_close(s3, a * s1 + b * s2, 1e-12, "linearity state")


def test_channel_subset_matches_full(oracle_lib):
    rng = np.random.default_rng(12)
    c = rand_case(rng, batch=3, L=21, dim=5, N=4)
    h0 = rng.standard_normal((3, 5, 4))
    y, last = oracle_lib.fwd(**c, h0=h0)
    ch = np.array([[2, 4], [0, 0], [1, 3], [2, 1]])
    ys, ls = oracle_lib.fwd(**c, h0=h0, channels=ch)
    for i, (b, d) in enumerate(ch):
        assert np.array_equal(ys[i], y[b, :, d])
        assert np.array_equal(ls[i], last[b, d])


def test_thread_count_does_not_change_results(oracle_lib):
    rng = np.random.default_rng(13)
    c = rand_case(rng, batch=2, L=50, dim=16, N=8)
    y1, s1 = oracle_lib.fwd(**c, nthreads=1)
    y4, s4 = oracle_lib.fwd(**c, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(s1, s4)


def test_rejects_bad_arguments(oracle_lib):
    rng = np.random.default_rng(14)
    c = rand_case(rng)
    with pytest.raises(TypeError):
        oracle_lib.fwd(**dict(c, u=c["u"].astype(np.float64)))
    with pytest.raises(ValueError):
        oracle_lib.fwd(**dict(c, A=c["A"][:, :3]))
    with pytest.raises(ValueError):
        oracle_lib.fwd(**c, channels=np.array([[5, 0]]))


# ---- exact zero-order hold (zoh=True) ----------------------------------------------------
# Page "架构变体：Mamba/SSM", section "离散化": the continuous system h' = A h + B u is
# discretised by holding the input constant over each step of length dt. The resulting
# update is the exact solution of the ODE for piecewise-constant input, which gives pins
# that hold for any sequence of step sizes.


def test_zoh_matches_continuous_solution(oracle_lib):
    """Constant u and B, arbitrary positive steps: after steps dt_1..dt_t the state is the
    ODE solution e^{A S} h0 + (e^{A S} - 1)/A B u at S = dt_1 + .. + dt_t, however S was cut
    into steps (A = 0 integrates: h0 + S B u; a positive A grows)."""
    rng = np.random.default_rng(21)
    batch, L, dim, N = 2, 60, 3, 5
    f = np.float32
    u = np.repeat(rng.standard_normal((batch, 1, dim)), L, axis=1).astype(f)
    B = np.repeat(rng.standard_normal((batch, 1, N)), L, axis=1).astype(f)
    C = rng.standard_normal((batch, L, N)).astype(f)
    delta = rng.uniform(0.001, 0.4, (batch, L, dim)).astype(f)  # the steps (softplus off)
    A = (-rng.uniform(0.2, 3.0, (dim, N))).astype(f)
    A[1, 2] = 0.0
    A[2, 4] = 0.05
    h0 = rng.standard_normal((batch, dim, N))
    y, last = oracle_lib.fwd(u, delta, A, B, C, softplus=False, h0=h0, zoh=True)
    S = np.cumsum(f64(delta), axis=1)
    Af = f64(A)
    for b in range(batch):
        for d in range(dim):
            St = S[b, :, d][:, None]
            h = np.exp(Af[d] * St) * h0[b, d] + zoh_coef(St, Af[d]) * f64(B[b, 0]) * f64(u[b, 0, d])
            assert_close(y[b, :, d], np.sum(f64(C[b]) * h, axis=1), 1e-12, f"zoh y b={b} d={d}")
            assert_close(last[b, d], h[-1], 1e-12, f"zoh state b={b} d={d}")


def test_zoh_half_steps_compose(oracle_lib):
    """Holding an input for dt equals holding it for dt/2 twice: repeating every token with
    half the step gives the same states, and every second output equals the original's
    (time-varying u, B, C; halving a float is exact)."""
    rng = np.random.default_rng(22)
    c = rand_case(rng, L=30, bias=False, gated=False, with_D=False)
    c["delta"] = rng.uniform(0.01, 0.6, c["delta"].shape).astype(np.float32)
    y, last = oracle_lib.fwd(**c, softplus=False, zoh=True)
    c2 = dict(c)
    for k in ("u", "B", "C"):
        c2[k] = np.repeat(c[k], 2, axis=1)
    c2["delta"] = np.repeat(c["delta"] * np.float32(0.5), 2, axis=1)
    y2, last2 = oracle_lib.fwd(**c2, softplus=False, zoh=True)
    assert_close(y2[:, 1::2], y, 1e-12, "half-step outputs")
    assert_close(last2, last, 1e-12, "half-step state")


@pytest.mark.parametrize("gated", [False, True])
def test_zoh_brute_force_unrolled_sum(oracle_lib, gated):
    rng = np.random.default_rng(23)
    c = rand_case(rng, gated=gated)
    c["A"][0, 1] = 0.0  # the A -> 0 limit of the input term
    y, last = oracle_lib.fwd(**c, softplus=True, zoh=True)
    y_ref, last_ref = brute_force(c, softplus=True, zoh=True)
    assert_close(y, y_ref, 1e-12, "y")
    assert_close(last, last_ref, 1e-12, "last_state")


def test_zoh_step_by_step_matches_forward(oracle_lib):
    rng = np.random.default_rng(24)
    c = rand_case(rng, L=20)
    y, last = oracle_lib.fwd(**c, zoh=True)
    st = np.zeros((2, 3, 5))
    for t in range(20):
        yt = oracle_lib.step(st, c["u"][:, t], c["delta"][:, t], c["A"], c["B"][:, t], c["C"][:, t],
                             D=c["D"], z=c["z"][:, t], delta_bias=c["delta_bias"], zoh=True)
        assert np.array_equal(yt, y[:, t])
    assert np.array_equal(st, last)
