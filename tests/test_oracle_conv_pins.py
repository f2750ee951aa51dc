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


# ---- the backward oracle: finite differences of the (pinned) forward, planted mistakes

from oracle.conv_oracle import conv1d_bwd  # noqa: E402


def _conv_problem(seed, Bsz=2, L=7, D=3, W=4, state=True, bias=True):
    r = np.random.default_rng(seed)
    return {"x": r.standard_normal((Bsz, L, D)), "w": r.standard_normal((D, W)),
            "bias": r.standard_normal(D) if bias else None,
            "state": r.standard_normal((Bsz, D, W - 1)) if state else None}, r.standard_normal((Bsz, L, D))


def _fd_worst(fn, seed, W, silu, state=True, bias=True):
    p, dy = _conv_problem(seed, W=W, state=state, bias=bias)
    g = fn(p["x"], p["w"], p["bias"], p["state"], dy, silu)
    names = {"x": "dx", "w": "dw", "bias": "dbias", "state": "dstate"}
    loss = lambda: float((conv1d(p["x"], p["w"], p["bias"], p["state"], silu)[0] * dy).sum())
    worst = 0.0
    for name, arr in p.items():
        if arr is None:
            continue
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            v = arr[idx]
            eps = 1e-6 * max(1.0, abs(v))
            arr[idx] = v + eps
            lp = loss()
            arr[idx] = v - eps
            lm = loss()
            arr[idx] = v
            fd = (lp - lm) / (2 * eps)
            worst = max(worst, abs(fd - g[names[name]][idx]) / max(1.0, abs(fd)))
    return worst


@pytest.mark.parametrize("W,silu,state,bias", [(4, True, True, True), (4, False, False, True), (1, True, False, False),
                                               (3, True, True, False), (2, False, True, True)])
def test_backward_equals_finite_differences(W, silu, state, bias):
    assert _fd_worst(conv1d_bwd, 40 + W, W, silu, state, bias) < 1e-7


def test_backward_is_the_transpose_for_a_linear_filter():
    """With SiLU off the filter is linear in x: <dy, K x> = <K^T dy, x> for any x, dy."""
    p, dy = _conv_problem(3, L=20, state=False, bias=False)
    y, _ = conv1d(p["x"], p["w"], None, None, silu=False)
    g = conv1d_bwd(p["x"], p["w"], None, None, dy, silu=False)
    np.testing.assert_allclose((y * dy).sum(), (g["dx"] * p["x"]).sum(), rtol=1e-12)


_BWD_MUTANTS = {
    "silu_prime_dropped": ("g = dy[:, t, :] * sg * (1.0 + a * (1.0 - sg))", "g = dy[:, t, :] * sg"),
    "tap_off_by_one": ("dxp[:, t + k, :] += w[None, :, k] * g", "dxp[:, t + k, :] += w[None, :, W - 1 - k] * g"),
    "dw_with_wrong_input": ("dw[:, k] += (g * xp[:, t + k, :]).sum(axis=0)", "dw[:, k] += (g * xp[:, t, :]).sum(axis=0)"),
    "bias_ignored_in_a": ("a = np.zeros((Bsz, D)) if bias is None else np.broadcast_to(", "a = np.zeros((Bsz, D)) if True else np.broadcast_to("),
    "state_gradient_shifted": ('"dstate": dxp[:, :W - 1, :]', '"dstate": dxp[:, 1:W, :]'),
}


@pytest.mark.parametrize("kind", sorted(_BWD_MUTANTS))
def test_planted_backward_mistake_is_caught(kind):
    import inspect
    from oracle import conv_oracle
    src = inspect.getsource(conv_oracle.conv1d_bwd)
    old, new = _BWD_MUTANTS[kind]
    assert old in src, kind
    ns = dict(vars(conv_oracle))
    exec(src.replace(old, new), ns)
    assert _fd_worst(ns["conv1d_bwd"], 41, 4, True) > 1e-3, f"mutant {kind} passes the pin"
