"""Second, independent fp64 oracle of the selective scan, in numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Written separately
from ``ssm_oracle.c`` -- whole [B, D, N] state slabs per time step instead of
one channel at a time -- so that the two can be checked against each other.

Discrete selective SSM per time step t (managen.ai page, "Selective Scan
Algorithm"; skill page, MambaBlock._selective_scan):

    A_bar[b, d, n] = exp(delta[b, t, d] * A[d, n])
    B_bar[b, d, n] = delta[b, t, d] * B[b, t, n]
    h              = A_bar * h + B_bar * x[b, t, d]
    y[b, t, d]     = <h[b, d, :], C[b, t, :]> + D[d] * x[b, t, d]
    y              = y * silu(z[b, t, d])            (when a gate is given)
"""
from __future__ import annotations

import numpy as np


def _silu(v):
    return v / (1.0 + np.exp(-v))


def _softplus(u):
    return np.logaddexp(0.0, u)


def scan_np(x, delta, A, Bm, Cm, Dskip=None, z=None, h0=None, delta_softplus=False):
    """All arrays float64.  x, delta, z: [B, L, D]; A: [D, N]; Bm, Cm: [B, L, N];
    Dskip: [D]; h0: [B, D, N].  Returns y [B, L, D], h_last [B, D, N]."""
    x = np.asarray(x, dtype=np.float64)
    Bsz, L, D = x.shape
    N = A.shape[1]
    dl = np.asarray(delta, dtype=np.float64)
    if delta_softplus:
        dl = _softplus(dl)
    h = np.zeros((Bsz, D, N)) if h0 is None else np.array(h0, dtype=np.float64, copy=True)
    y = np.empty((Bsz, L, D))
    A = np.asarray(A, dtype=np.float64)
    for t in range(L):
        dt = dl[:, t, :][:, :, None]                      # [B, D, 1]
        a_bar = np.exp(dt * A[None, :, :])                 # [B, D, N]
        b_bar = dt * np.asarray(Bm, dtype=np.float64)[:, t, None, :]    # [B, D, N]
        h = a_bar * h + b_bar * x[:, t, :, None]
        yt = np.einsum("bdn,bn->bd", h, np.asarray(Cm, dtype=np.float64)[:, t, :])
        if Dskip is not None:
            yt = yt + np.asarray(Dskip, dtype=np.float64)[None, :] * x[:, t, :]
        if z is not None:
            yt = yt * _silu(np.asarray(z, dtype=np.float64)[:, t, :])
        y[:, t, :] = yt
    return y, h
