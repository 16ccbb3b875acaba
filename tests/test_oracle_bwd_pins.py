"""Pins for the oracle's backward (reverse-mode derivative of the forward), each against
something other than the backward itself:

- central finite differences of an independent fp64 numpy forward (itself checked against
  the oracle forward), for every input element, with and without softplus;
- adjoint identities: the loss is linear (affine) in u, B, C, D and h0, so the gradient
  paired with any direction v equals the change of the loss computed by the oracle forward;
- the LTI case (constant dt, B, C): du is the correlation of dy with the convolution
  kernel K_k = sum_n C abar^k dt B (page "架构变体：Mamba/SSM", section "并行卷积");
- a zero step (softplus off, dt = 0): the state is frozen, so dh0, ddelta and dB have
  closed forms;
- linearity in dy, channel subsets, thread count.
"""
import numpy as np
import pytest
from scipy.special import expit

from tests.test_oracle_pins import rand_case, f64, assert_close, silu_ref

GRAD_KEYS = ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias", "dh0")


def np_forward(p, softplus=True):
    """Plain fp64 forward on float64 parameters (vectorised over batch and channel):
    returns y (batch, L, dim) and the final state (batch, dim, N)."""
    u, delta, A, B, C = p["u"], p["delta"], p["A"], p["B"], p["C"]
    batch, L, dim = u.shape
    N = A.shape[1]
    x = delta + (p["delta_bias"][None, None, :] if p.get("delta_bias") is not None else 0.0)
    dt = np.logaddexp(0.0, x) if softplus else x
    h = np.zeros((batch, dim, N)) if p.get("h0") is None else p["h0"].copy()
    y = np.zeros((batch, L, dim))
    for t in range(L):
        abar = np.exp(dt[:, t, :, None] * A[None])
        h = abar * h + dt[:, t, :, None] * B[:, t, None, :] * u[:, t, :, None]
        s = np.einsum("bdn,bn->bd", h, C[:, t])
        if p.get("D") is not None:
            s = s + p["D"][None] * u[:, t]
        if p.get("z") is not None:
            s = s * silu_ref(p["z"][:, t])
        y[:, t] = s
    return y, h


def loss(p, dy, dlast, softplus=True):
    y, h = np_forward(p, softplus)
    val = np.sum(dy * y)
    if dlast is not None:
        val += np.sum(dlast * h)
    return val


def case(seed, softplus=True, gated=True, with_D=True, bias=True, h0=True, dlast=True, batch=2, L=7,
         dim=3, N=4):
    rng = np.random.default_rng(seed)
    c = rand_case(rng, batch=batch, L=L, dim=dim, N=N, gated=gated, with_D=with_D, bias=bias)
    if not softplus:
        c["delta"] = rng.uniform(0.05, 0.7, c["delta"].shape).astype(np.float32)
    dy = rng.standard_normal(c["u"].shape).astype(np.float32)
    h0v = rng.standard_normal((batch, dim, N)) if h0 else None
    dl = rng.standard_normal((batch, dim, N)).astype(np.float32) if dlast else None
    return c, dy, h0v, dl


def params64(c, h0):
    p = {k: (None if v is None else f64(v)) for k, v in c.items()}
    p["h0"] = None if h0 is None else np.array(h0, dtype=np.float64)
    return p


def test_numpy_forward_matches_oracle(oracle_lib):
    c, _, h0, _ = case(40)
    y, st = oracle_lib.fwd(**c, h0=h0)
    y2, st2 = np_forward(params64(c, h0))
    assert_close(y2, y, 1e-13, "y")
    assert_close(st2, st, 1e-13, "state")


@pytest.mark.parametrize("softplus", [True, False])
def test_backward_matches_finite_differences(oracle_lib, softplus):
    c, dy, h0, dl = case(41, softplus=softplus, bias=softplus)
    g = oracle_lib.bwd(**c, dy=dy, softplus=softplus, h0=h0, dlast=dl)
    p = params64(c, h0)
    dy64, dl64 = f64(dy), f64(dl)
    names = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz",
             "delta_bias": "ddelta_bias", "h0": "dh0"}
    for pname, gname in names.items():
        if p.get(pname) is None:
            continue
        base = p[pname]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            eps = 1e-6 * max(1.0, abs(base[idx]))
            old = base[idx]
            base[idx] = old + eps
            lp = loss(p, dy64, dl64, softplus)
            base[idx] = old - eps
            lm = loss(p, dy64, dl64, softplus)
            base[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        assert_close(g[gname], fd, 2e-7, f"d{pname} vs finite differences")


def _oracle_loss(oracle_lib, c, dy, dl, h0=None, softplus=True):
    y, st = oracle_lib.fwd(**c, h0=h0, softplus=softplus)
    val = float(np.sum(f64(dy) * y))
    if dl is not None:
        val += float(np.sum(f64(dl) * st))
    return val


@pytest.mark.parametrize("which", ["u", "B", "C", "D", "h0"])
def test_adjoint_identity_for_linear_arguments(oracle_lib, which):
    """L is affine in u (h0 = 0), B (h0 = 0), C, D and h0: <grad, v> = L(v) - L(0)."""
    rng = np.random.default_rng(42)
    c, dy, h0, dl = case(42, h0=(which == "h0"))
    if which in ("u", "B"):
        h0 = None
    g = oracle_lib.bwd(**c, dy=dy, h0=h0, dlast=dl)
    if which == "h0":
        v = rng.standard_normal(h0.shape)
        lv = _oracle_loss(oracle_lib, c, dy, dl, h0=v)
        l0 = _oracle_loss(oracle_lib, c, dy, dl, h0=np.zeros_like(v))
        got = float(np.sum(g["dh0"] * v))
    else:
        v = rng.standard_normal(c[which].shape).astype(np.float32)
        lv = _oracle_loss(oracle_lib, dict(c, **{which: v}), dy, dl, h0=h0)
        l0 = _oracle_loss(oracle_lib, dict(c, **{which: np.zeros_like(v)}), dy, dl, h0=h0)
        got = float(np.sum(g["d" + which] * f64(v)))
    assert abs(got - (lv - l0)) <= 1e-12 * (1 + abs(lv - l0)), (got, lv - l0)


def test_lti_du_is_correlation_with_kernel(oracle_lib):
    """Constant dt, B, C and no gate: y = K * u + D u, so du_s = sum_{t>=s} K_{t-s} dy_t + D dy_s."""
    rng = np.random.default_rng(43)
    c = rand_case(rng, batch=2, L=40, dim=3, N=5, lti=True, gated=False)
    dy = rng.standard_normal(c["u"].shape).astype(np.float32)
    g = oracle_lib.bwd(**c, dy=dy)
    x = f64(c["delta"]) + f64(c["delta_bias"])[None, None, :]
    dt = np.logaddexp(0.0, x)
    A = f64(c["A"])
    L = c["u"].shape[1]
    k = np.arange(L)
    for b in range(2):
        for d in range(3):
            abar = np.exp(dt[b, 0, d] * A[d])
            K = np.sum(f64(c["C"])[b, 0] * abar[None, :] ** k[:, None] * dt[b, 0, d] * f64(c["B"])[b, 0], axis=1)
            dyv = f64(dy)[b, :, d]
            ref = np.array([np.dot(K[:L - s], dyv[s:]) for s in range(L)]) + f64(c["D"])[d] * dyv
            assert_close(g["du"][b, :, d], ref, 1e-12, f"lti du b={b} d={d}")


def test_zero_step_closed_forms(oracle_lib):
    """softplus off, delta = bias = 0: abar = 1 and no input enters, so h_t = h0 for all t.
    Then lam_t = sum_{s>=t} ds_s C_s + dlast, dh0 = lam_0, dB = 0 and
    ddelta_t = sum_n lam_t[n] (B_t[n] u_t + A[n] h0[n])."""
    c, dy, h0, dl = case(44, softplus=False, bias=False)
    c["delta"] = np.zeros_like(c["delta"])
    g = oracle_lib.bwd(**c, dy=dy, softplus=False, h0=h0, dlast=dl)
    u, B, C, A = f64(c["u"]), f64(c["B"]), f64(c["C"]), f64(c["A"])
    s = np.einsum("btn,bdn->btd", C, h0) + f64(c["D"])[None, None, :] * u
    ds = f64(dy) * silu_ref(f64(c["z"]))
    contrib = ds[:, :, :, None] * C[:, :, None, :]                      # (b, t, d, n)
    lam = np.flip(np.cumsum(np.flip(contrib, 1), 1), 1) + f64(dl)[:, None]
    assert_close(g["dh0"], lam[:, 0], 1e-13, "dh0")
    assert np.array_equal(g["dB"], np.zeros_like(g["dB"]))
    ref = np.einsum("btdn,btdn->btd", lam, B[:, :, None, :] * u[:, :, :, None] + A[None, None] * h0[:, None])
    assert_close(g["ddelta"], ref, 1e-13, "ddelta")
    zz = f64(c["z"])
    dsilu = expit(zz) * (1 + zz * (1 - expit(zz)))
    assert_close(g["dz"], f64(dy) * s * dsilu, 1e-13, "dz")


def test_linear_in_dy(oracle_lib):
    c, _, h0, _ = case(45)
    rng = np.random.default_rng(45)
    grid = lambda: (np.round(rng.standard_normal(c["u"].shape) * 1024) / 1024).astype(np.float32)
    dy1, dy2 = grid(), grid()
    dy3 = (0.5 * dy1.astype(np.float64) - 2.0 * dy2.astype(np.float64)).astype(np.float32)
    g1 = oracle_lib.bwd(**c, dy=dy1, h0=h0)
    g2 = oracle_lib.bwd(**c, dy=dy2, h0=h0)
    g3 = oracle_lib.bwd(**c, dy=dy3, h0=h0)
    for k in GRAD_KEYS:
        assert_close(g3[k], 0.5 * g1[k] - 2.0 * g2[k], 1e-12, k)


def test_channel_subset_matches_full(oracle_lib):
    c, dy, h0, dl = case(46, batch=3, dim=5)
    g = oracle_lib.bwd(**c, dy=dy, h0=h0, dlast=dl)
    ch = np.array([[2, 4], [0, 0], [1, 3], [2, 1]])
    gs = oracle_lib.bwd(**c, dy=dy, h0=h0, dlast=dl, channels=ch)
    for i, (b, d) in enumerate(ch):
        for k in ("du", "ddelta", "dz"):
            assert np.array_equal(gs[k][i], g[k][b, :, d])
        assert np.array_equal(gs["dh0"][i], g["dh0"][b, d])
    every = np.array([[b, d] for b in range(3) for d in range(5)])
    ga = oracle_lib.bwd(**c, dy=dy, h0=h0, dlast=dl, channels=every)
    assert_close(ga["dB"], g["dB"], 1e-14, "dB over all channels")
    assert_close(ga["dC"], g["dC"], 1e-14, "dC over all channels")
    # per-channel dA, dD, dbias summed over the batch rows equal the full result
    assert_close(ga["dA"].reshape(3, 5, -1).sum(0), g["dA"], 1e-14, "dA")
    assert_close(ga["dD"].reshape(3, 5).sum(0), g["dD"], 1e-14, "dD")


def test_thread_count_changes_only_rounding(oracle_lib):
    c, dy, h0, dl = case(47, batch=2, L=30, dim=16, N=8)
    g1 = oracle_lib.bwd(**c, dy=dy, h0=h0, dlast=dl, nthreads=1)
    g4 = oracle_lib.bwd(**c, dy=dy, h0=h0, dlast=dl, nthreads=4)
    for k in GRAD_KEYS:
        assert_close(g4[k], g1[k], 1e-14, k)
    for k in ("du", "ddelta", "dz", "dA", "dD", "ddelta_bias", "dh0"):
        assert np.array_equal(g4[k], g1[k])


def test_empty_sequence(oracle_lib):
    c, dy, h0, dl = case(48, L=0)
    g = oracle_lib.bwd(**c, dy=dy, h0=h0, dlast=dl)
    assert np.array_equal(g["dh0"], f64(dl))
    assert g["du"].size == 0 and not g["dA"].any()
