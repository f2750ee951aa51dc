"""Pins of the convolution oracle against things other than itself.

* numpy's own convolution: a causal filter is the full linear convolution of the
  series with the kernel, cut to the first L outputs (np.convolve, a library routine).
* The impulse response of the filter is the reversed kernel.
* Splitting the sequence and carrying the state gives the same outputs and final state.
* L single-token updates equal one call over those L tokens.
"""
import numpy as np
import pytest

from oracle.conv_oracle import conv1d, conv1d_update


def _silu(v):
    return v / (1.0 + np.exp(-v))


@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_matches_numpy_convolve(W):
    r = np.random.default_rng(W)
    Bsz, L, D = 2, 37, 5
    x = r.standard_normal((Bsz, L, D))
    w = r.standard_normal((D, W))
    bias = r.standard_normal(D)
    y, _ = conv1d(x, w, bias, silu=True)
    for b in range(Bsz):
        for d in range(D):
            # conv1d weights multiply x[t - W + 1 + k]; np.convolve flips its kernel
            a = np.convolve(x[b, :, d], w[d, ::-1])[:L] + bias[d]
            np.testing.assert_allclose(y[b, :, d], _silu(a), rtol=1e-13, atol=1e-13)


def test_impulse_response_is_reversed_kernel():
    W, L = 4, 10
    w = np.array([[0.5, -1.0, 2.0, 3.0]])
    x = np.zeros((1, L, 1))
    x[0, 2, 0] = 1.0
    y, _ = conv1d(x, w, None, silu=False)
    want = np.zeros(L)
    want[2:2 + W] = w[0, ::-1]
    np.testing.assert_array_equal(y[0, :, 0], want)


@pytest.mark.parametrize("T", [0, 1, 3, 20])
def test_split_with_state_carry(T):
    r = np.random.default_rng(11)
    x = r.standard_normal((3, 20, 4))
    w = r.standard_normal((4, 4))
    s0 = r.standard_normal((3, 4, 3))
    y, s = conv1d(x, w, None, s0)
    y1, s1 = conv1d(x[:, :T], w, None, s0)
    y2, s2 = conv1d(x[:, T:], w, None, s1)
    np.testing.assert_allclose(np.concatenate([y1, y2], axis=1), y, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(s2, s, rtol=0, atol=0)


def test_updates_equal_one_call():
    r = np.random.default_rng(12)
    x = r.standard_normal((2, 9, 6))
    w = r.standard_normal((6, 3))
    bias = r.standard_normal(6)
    y, s = conv1d(x, w, bias)
    st = np.zeros((2, 6, 2))
    for t in range(9):
        yt, st = conv1d_update(st, x[:, t], w, bias)
        np.testing.assert_allclose(yt, y[:, t], rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(st, s)
