"""fp64 oracle of the causal depthwise convolution (+ SiLU) that feeds the scan.

TEST INFRASTRUCTURE ONLY (see the package docstring): only the tests, the package's
smoke check and the bench's CPU-baseline leg use it; it shares no code with the GPU
library.

What it computes (skill page "State Space Models Mamba", MambaBlock listing: a
depthwise Conv1d over the sequence with kernel size d_conv, padding d_conv - 1, the
output cut back to the sequence length -- a causal filter -- then SiLU).  For every
batch row b, channel d and step t, with W = width and the W - 1 inputs before the
sequence taken from state (zeros when there is none):

    xp[b, :, d] = concat(state[b, d, :], x[b, :, d])        (W - 1 + L values)
    a[b, t, d]  = bias[d] + sum_{k < W} w[d, k] * xp[b, t + k, d]
    y[b, t, d]  = silu(a) = a / (1 + exp(-a))                (or a itself, silu off)
    state_out[b, d, :] = the last W - 1 values of xp[b, :, d]

Single-token form (decode): the same with L = 1, state updated in place.

Backward, for a loss with gradient dy = dLoss/dy (the chain rule through the same
definition; the final state is not differentiated):

    g[b, t, d]    = dy * silu'(a) = dy * s (1 + a (1 - s)),  s = 1 / (1 + exp(-a))  (dy, silu off)
    dxp[b, t + k, d] += w[d, k] * g[b, t, d]            for every t < L, k < W
    dx = dxp[:, W - 1:, :],  dstate[b, d, j] = dxp[b, j, d]  (j < W - 1)
    dw[d, k]  = sum_{b, t} g[b, t, d] * xp[b, t + k, d]
    dbias[d]  = sum_{b, t} g[b, t, d]
"""
from __future__ import annotations

import numpy as np


def _silu(v):
    return v / (1.0 + np.exp(-v))


def conv1d(x, w, bias=None, state=None, silu=True):
    """x [B, L, D], w [D, W], bias [D] or None, state [B, D, W-1] or None (float64 or
    anything numpy widens exactly).  Returns (y [B, L, D], state_out [B, D, W-1])."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    Bsz, L, D = x.shape
    W = w.shape[1]
    st = np.zeros((Bsz, D, W - 1)) if state is None else np.asarray(state, dtype=np.float64)
    xp = np.concatenate([st.transpose(0, 2, 1), x], axis=1)       # [B, W-1+L, D]
    y = np.empty((Bsz, L, D))
    for t in range(L):
        acc = np.zeros((Bsz, D)) if bias is None else np.broadcast_to(np.asarray(bias, np.float64), (Bsz, D)).copy()
        for k in range(W):
            acc = acc + w[None, :, k] * xp[:, t + k, :]
        y[:, t, :] = _silu(acc) if silu else acc
    state_out = xp[:, L:, :].transpose(0, 2, 1).copy() if W > 1 else np.zeros((Bsz, D, 0))
    return y, state_out


def conv1d_update(state, x, w, bias=None, silu=True):
    """One token: state [B, D, W-1], x [B, D].  Returns (y [B, D], new state)."""
    y, st = conv1d(np.asarray(x, np.float64)[:, None, :], w, bias, state, silu)
    return y[:, 0, :], st


def conv1d_bwd(x, w, bias=None, state=None, dy=None, silu=True):
    """Gradients of <dy, y> through ``conv1d``: returns a dict dx [B, L, D], dw [D, W],
    dbias [D] and dstate [B, D, W-1] (the gradient with respect to the starting state,
    zeros or not)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    Bsz, L, D = x.shape
    W = w.shape[1]
    st = np.zeros((Bsz, D, W - 1)) if state is None else np.asarray(state, dtype=np.float64)
    xp = np.concatenate([st.transpose(0, 2, 1), x], axis=1)       # [B, W-1+L, D]
    dxp = np.zeros_like(xp)
    dw = np.zeros((D, W))
    dbias = np.zeros(D)
    for t in range(L):
        a = np.zeros((Bsz, D)) if bias is None else np.broadcast_to(np.asarray(bias, np.float64), (Bsz, D)).copy()
        for k in range(W):
            a = a + w[None, :, k] * xp[:, t + k, :]
        if silu:
            sg = 1.0 / (1.0 + np.exp(-a))
            g = dy[:, t, :] * sg * (1.0 + a * (1.0 - sg))
        else:
            g = dy[:, t, :]
        for k in range(W):
            dxp[:, t + k, :] += w[None, :, k] * g
            dw[:, k] += (g * xp[:, t + k, :]).sum(axis=0)
        dbias += g.sum(axis=0)
    return {"dx": dxp[:, W - 1:, :].copy(), "dw": dw, "dbias": dbias,
            "dstate": dxp[:, :W - 1, :].transpose(0, 2, 1).copy()}
