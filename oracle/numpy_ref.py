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

with the other discretisations of ``_discretize_slab`` (zero-order hold, bilinear)
in place of A_bar, B_bar, and an optional per-channel bias added to delta before
the softplus.
"""
from __future__ import annotations

import numpy as np


def _silu(v):
    return v / (1.0 + np.exp(-v))


def _softplus(u):
    return np.logaddexp(0.0, u)


def _discretize_slab(kind, dt, A):
    """A_bar and the factor F with B_bar = F * B, as [B, D, N] slabs, for a diagonal A.

    "mamba": exp(dt A) and dt (managen.ai, Selective Scan Algorithm);
    "zoh": exp(dt A) and A^-1 (exp(dt A) - 1), i.e. dt * phi(dt A) with
    phi(u) = (e^u - 1) / u, phi(0) = 1 (skill page "Discretization" docstring;
    brentwoodlivery, From Continuous to Discrete);
    "bilinear": (1 + dt A / 2) / (1 - dt A / 2) and dt / (1 - dt A / 2)
    (chipfoundryservices glossary, Lab 1)."""
    u = dt * A[None, :, :]
    if kind == "bilinear":
        den = 1.0 - 0.5 * u
        return (1.0 + 0.5 * u) / den, dt / den
    a_bar = np.exp(u)
    if kind == "zoh":
        with np.errstate(divide="ignore", invalid="ignore"):
            phi = np.where(u == 0.0, 1.0, np.expm1(u) / np.where(u == 0.0, 1.0, u))
        return a_bar, dt * phi
    return a_bar, np.broadcast_to(dt, a_bar.shape)


def scan_np(x, delta, A, Bm, Cm, Dskip=None, z=None, h0=None, delta_softplus=False,
            discretization="mamba", delta_bias=None):
    """All arrays float64.  x, delta, z: [B, L, D]; A: [D, N]; Bm, Cm: [B, L, N];
    Dskip: [D]; h0: [B, D, N]; delta_bias: [D] (added before the softplus).
    Returns y [B, L, D], h_last [B, D, N]."""
    x = np.asarray(x, dtype=np.float64)
    Bsz, L, D = x.shape
    N = A.shape[1]
    dl = np.asarray(delta, dtype=np.float64)
    if delta_bias is not None:
        dl = dl + np.asarray(delta_bias, dtype=np.float64)[None, None, :]
    if delta_softplus:
        dl = _softplus(dl)
    h = np.zeros((Bsz, D, N)) if h0 is None else np.array(h0, dtype=np.float64, copy=True)
    y = np.empty((Bsz, L, D))
    A = np.asarray(A, dtype=np.float64)
    for t in range(L):
        dt = dl[:, t, :][:, :, None]                      # [B, D, 1]
        a_bar, fac = _discretize_slab(discretization, dt, A)             # [B, D, N]
        b_bar = fac * np.asarray(Bm, dtype=np.float64)[:, t, None, :]    # [B, D, N]
        h = a_bar * h + b_bar * x[:, t, :, None]
        yt = np.einsum("bdn,bn->bd", h, np.asarray(Cm, dtype=np.float64)[:, t, :])
        if Dskip is not None:
            yt = yt + np.asarray(Dskip, dtype=np.float64)[None, :] * x[:, t, :]
        if z is not None:
            yt = yt * _silu(np.asarray(z, dtype=np.float64)[:, t, :])
        y[:, t, :] = yt
    return y, h


def _discretize_grad_slab(kind, dt, A):
    """The operands of ``_discretize_slab`` and their partial derivatives, as slabs:
    (A_bar, F, dA_bar/ddt, dF/ddt, dA_bar/dA, dF/dA), B_bar = F * B.

    mamba: A_bar = e^u (u = dt A), F = dt: derivatives A e^u, 1, dt e^u, 0.
    zoh: F = dt phi(u), phi(u) = (e^u - 1) / u: dF/ddt = e^u, dF/dA = dt^2 psi(u) with
    psi(u) = d phi / du = (u e^u - e^u + 1) / u^2 (1/2 + u/3 + u^2/8 + u^3/30 + u^4/144
    near 0, where the closed form cancels).
    bilinear: with r = 1 / (1 - u/2), A_bar = 2 r - 1, F = r dt: dA_bar/ddt = r^2 A,
    dF/ddt = r^2, dA_bar/dA = r^2 dt, dF/dA = r^2 dt^2 / 2."""
    u = dt * A[None, :, :]
    if kind == "bilinear":
        r = 1.0 / (1.0 - 0.5 * u)
        r2 = r * r
        return (2.0 * r - 1.0, r * dt, r2 * A[None], np.broadcast_to(r2, u.shape) * 1.0, r2 * dt,
                r2 * dt * dt / 2.0)
    e = np.exp(u)
    if kind == "zoh":
        small = np.abs(u) < 1e-2
        us = np.where(small, 1.0, u)
        phi = np.where(u == 0.0, 1.0, np.expm1(u) / np.where(u == 0.0, 1.0, u))
        psi_series = 0.5 + u * (1.0 / 3.0 + u * (1.0 / 8.0 + u * (1.0 / 30.0 + u / 144.0)))
        psi = np.where(small, psi_series, (us * np.exp(us) - np.expm1(us)) / (us * us))
        return e, dt * phi, A[None] * e, e, dt * e, dt * dt * psi
    one = np.ones(u.shape)
    return e, dt * one, A[None] * e, one, dt * e, np.zeros(u.shape)


def scan_bwd_np(x, delta, A, Bm, Cm, Dskip=None, z=None, h0=None, delta_softplus=False,
                gy=None, g_last=None, delta_bias=None, discretization="mamba"):
    """Reverse-mode derivative of ``scan_np`` for the loss <gy, y> + <g_last, h_last>.

    Written as the chain rule through the discretised operands: with
    lam_t = dLoss/dh_t (after step t), the step h_t = A_bar_t h_{t-1} + B_bar_t x_t gives
        dLoss/dA_bar_t = lam_t * h_{t-1},   dLoss/dB_bar_t = lam_t * x_t,
        dLoss/dh_{t-1} = A_bar_t * lam_t (+ the readout of step t-1),
    and the discretisation (A_bar(dt, A), B_bar = F(dt, A) B; see
    ``_discretize_grad_slab``) carries those on to dt, A, B.  All float64;
    shapes as ``scan_np`` plus gy [B, L, D] and g_last [B, D, N] (either may be None
    = zero) and delta_bias [D] (added to delta before the softplus).  Returns a dict dx,
    ddelta, dz, dB, dC, dA, dD, dh0 (dz None without a gate; ddelta with respect to the
    raw input in softplus mode) and ddelta_bias (None without a bias)."""
    x = np.asarray(x, dtype=np.float64)
    Bsz, L, D = x.shape
    A = np.asarray(A, dtype=np.float64)
    N = A.shape[1]
    Bm = np.asarray(Bm, dtype=np.float64)
    Cm = np.asarray(Cm, dtype=np.float64)
    raw = np.asarray(delta, dtype=np.float64)
    if delta_bias is not None:
        raw = raw + np.asarray(delta_bias, dtype=np.float64)[None, None, :]
    dl = _softplus(raw) if delta_softplus else raw
    gy = np.zeros((Bsz, L, D)) if gy is None else np.asarray(gy, dtype=np.float64)
    zz = None if z is None else np.asarray(z, dtype=np.float64)
    # forward slabs: h_{t-1} for every t, and the ungated output
    hs = np.empty((L + 1, Bsz, D, N))
    hs[0] = 0.0 if h0 is None else np.asarray(h0, dtype=np.float64)
    y0 = np.empty((Bsz, L, D))
    for t in range(L):
        a_bar, fac = _discretize_slab(discretization, dl[:, t, :, None], A)[:2]
        hs[t + 1] = a_bar * hs[t] + fac * Bm[:, t, None, :] * x[:, t, :, None]
        y0[:, t, :] = np.einsum("bdn,bn->bd", hs[t + 1], Cm[:, t, :])
        if Dskip is not None:
            y0[:, t, :] += np.asarray(Dskip, dtype=np.float64)[None, :] * x[:, t, :]
    out = {"dx": np.zeros((Bsz, L, D)), "ddelta": np.zeros((Bsz, L, D)),
           "dz": None if zz is None else np.zeros((Bsz, L, D)),
           "dB": np.zeros((Bsz, L, N)), "dC": np.zeros((Bsz, L, N)),
           "dA": np.zeros((D, N)), "dD": np.zeros(D)}
    lam = np.zeros((Bsz, D, N)) if g_last is None else np.array(g_last, dtype=np.float64)
    for t in range(L - 1, -1, -1):
        if zz is not None:
            sg = 1.0 / (1.0 + np.exp(-zz[:, t, :]))
            gy0 = gy[:, t, :] * zz[:, t, :] * sg
            out["dz"][:, t, :] = gy[:, t, :] * y0[:, t, :] * sg * (1.0 + zz[:, t, :] * (1.0 - sg))
        else:
            gy0 = gy[:, t, :]
        if Dskip is not None:
            out["dD"] += (gy0 * x[:, t, :]).sum(axis=0)
            out["dx"][:, t, :] += np.asarray(Dskip, dtype=np.float64)[None, :] * gy0
        # readout y0 = <h_t, C_t>: into C and into the state adjoint
        out["dC"][:, t, :] += np.einsum("bd,bdn->bn", gy0, hs[t + 1])
        lam = lam + gy0[:, :, None] * Cm[:, t, None, :]
        a_bar, fac, da_dt, df_dt, da_dA, df_dA = _discretize_grad_slab(discretization, dl[:, t, :, None], A)
        g_abar = lam * hs[t]                       # dLoss/dA_bar_t
        g_bbar = lam * x[:, t, :, None]            # dLoss/dB_bar_t
        g_fac = g_bbar * Bm[:, t, None, :]         # dLoss/dF_t
        out["dx"][:, t, :] += np.einsum("bdn,bdn->bd", lam, fac * Bm[:, t, None, :])
        g_dt = np.einsum("bdn,bdn->bd", g_abar, da_dt) + np.einsum("bdn,bdn->bd", g_fac, df_dt)
        out["ddelta"][:, t, :] = g_dt / (1.0 + np.exp(-raw[:, t, :])) if delta_softplus else g_dt
        out["dA"] += np.einsum("bdn,bdn->dn", g_abar, da_dA) + np.einsum("bdn,bdn->dn", g_fac, df_dA)
        out["dB"][:, t, :] += np.einsum("bdn,bdn->bn", g_bbar, fac)
        lam = a_bar * lam
    out["dh0"] = lam
    # the bias enters every step's raw delta: its gradient is the sum of those
    out["ddelta_bias"] = None if delta_bias is None else out["ddelta"].sum(axis=(0, 1))
    return out
