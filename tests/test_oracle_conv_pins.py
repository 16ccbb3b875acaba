"""Pins for the oracle's conv prologue u = silu(causal depthwise conv1d(x) + conv_b) and for
the forward with it, each against something other than the oracle's own loop:
np.convolve (the page-5 demo's tool) for the convolution, closed forms for an impulse and
for a one-tap filter, and continuity across a split with the carried conv state.
"""
import numpy as np
import pytest

from tests.test_oracle_pins import f64, assert_close, silu_ref, rand_case


def conv_case(seed, batch=2, L=23, dim=3, K=4, state=True, bias=True):
    rng = np.random.default_rng(seed)
    f = np.float32
    x = rng.standard_normal((batch, L, dim)).astype(f)
    w = rng.standard_normal((dim, K)).astype(f)
    b = rng.standard_normal(dim).astype(f) if bias else None
    st = rng.standard_normal((batch, dim, K - 1)).astype(f) if state else None
    return x, w, b, st


def np_conv_silu(x, w, b, st):
    batch, L, dim = x.shape
    K = w.shape[1]
    u = np.zeros((batch, L, dim))
    for bb in range(batch):
        for d in range(dim):
            hist = f64(st[bb, d]) if st is not None else np.zeros(K - 1)
            xx = np.concatenate([hist, f64(x[bb, :, d])])
            # causal: pre_t = sum_m w[m] x[t-(K-1)+m]; np.convolve flips its second argument
            pre = np.convolve(xx, f64(w[d])[::-1], mode="valid")
            if b is not None:
                pre = pre + float(b[d])
            u[bb, :, d] = silu_ref(pre)
    return u


@pytest.mark.parametrize("K,state,bias", [(4, True, True), (4, False, True), (3, True, False),
                                          (2, False, False), (1, False, True)])
def test_conv_matches_numpy_convolve(oracle_lib, K, state, bias):
    x, w, b, st = conv_case(70 + K, K=K, state=state and K > 1, bias=bias)
    u = oracle_lib.conv_silu(x, w, b, st)
    assert_close(u, np_conv_silu(x, w, b, st), 1e-14, "conv + silu")


def test_conv_bf16_input(oracle_lib):
    x, w, b, st = conv_case(75)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    xf = (bits.astype(np.uint32) << 16).view(np.float32)
    assert_close(oracle_lib.conv_silu(bits, w, b, st), np_conv_silu(xf, w, b, st), 1e-14, "bf16 x")


def test_impulse_response(oracle_lib):
    """x = 1 at t0, else 0, no state: pre_t = conv_w[K-1-(t-t0)] + b for t0 <= t < t0 + K and
    b elsewhere (the filter read backwards in time)."""
    K, L, t0 = 4, 12, 5
    x = np.zeros((1, L, 2), np.float32)
    x[0, t0, :] = 1.0
    w = np.array([[0.5, -1.25, 2.0, 0.75], [-0.3, 0.1, 0.9, -2.2]], np.float32)
    b = np.array([0.2, -0.4], np.float32)
    u = oracle_lib.conv_silu(x, w, b)
    for d in range(2):
        pre = np.full(L, float(b[d]))
        for t in range(t0, t0 + K):
            pre[t] += float(w[d, K - 1 - (t - t0)])
        assert_close(u[0, :, d], silu_ref(pre), 1e-15, f"impulse d={d}")


def test_one_tap_is_silu(oracle_lib):
    x, _, _, _ = conv_case(76, K=1)
    u = oracle_lib.conv_silu(x, np.ones((3, 1), np.float32))
    assert_close(u, silu_ref(f64(x)), 1e-15, "one tap")


def test_split_continues_with_conv_state(oracle_lib):
    """conv over [0, L) equals conv over [t0, L) with the state holding x[t0-K+1 .. t0-1]."""
    x, w, b, st = conv_case(77, L=30)
    u = oracle_lib.conv_silu(x, w, b, st)
    t0 = 11
    st2 = np.ascontiguousarray(x[:, t0 - 3:t0, :].transpose(0, 2, 1))
    u2 = oracle_lib.conv_silu(np.ascontiguousarray(x[:, t0:]), w, b, st2)
    assert np.array_equal(u2, u[:, t0:])


def test_forward_with_conv_is_forward_on_conv_output(oracle_lib):
    """fwd_conv = conv_silu then the scan on that u: the scan part equals the unrolled sum
    (brute force of the pinned scan) evaluated on the fp64 u."""
    from tests.test_oracle_pins import brute_force
    rng = np.random.default_rng(78)
    c = rand_case(rng)
    x, w, b, st = conv_case(78, batch=2, L=17, dim=3)
    y, last, u = oracle_lib.fwd_conv(x, w, c["delta"], c["A"], c["B"], c["C"], conv_b=b, conv_state=st,
                                     D=c["D"], z=c["z"], delta_bias=c["delta_bias"])
    assert_close(u, np_conv_silu(x, w, b, st), 1e-14, "u")
    y_ref, last_ref = brute_force(dict(c, u=u))
    assert_close(y, y_ref, 1e-12, "y")
    assert_close(last, last_ref, 1e-12, "state")
