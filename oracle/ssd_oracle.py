"""fp64 oracle of the Mamba-2 structured state-space layer's scan (multi-head SSD).

TEST INFRASTRUCTURE ONLY (see the package docstring): only the tests, the package's
smoke check and the bench's CPU-baseline leg use it; it shares no code with the GPU
library.

What the pages give: managen.ai, "Mamba: State Space Models Challenge Transformers",
Mamba2Block listing -- a multi-head structure (n_heads, d_head = 64) around an SSD
layer with d_state = 128, whose body is left out; brentwoodlivery, "State-space models
(Mamba, S4)", section "Mamba 2 and Hybrid Architectures" -- the SSM rewritten as a
structured matrix multiplication, with attention and the SSM as two cases of one
state space duality.  The plainest reading that keeps the S6 recurrence of the same
pages (A_bar = exp(dt A), B_bar = dt B, readout after the update, skip term D x,
gate y * silu(z)):

    per batch row b, head h (P = d_head channels p, N = d_state states n), step t:
        dt         = delta[b, t, h]  (+ bias[h]; softplus of it in softplus mode)
                                                   one step size per head
        A_bar      = exp(dt * a[h])                one scalar decay per head: A = a_h I
        H[p, n]    = A_bar * H[p, n] + dt * B[b, t, n] * x[b, t, h, p]
        y[b,t,h,p] = sum_n C[b, t, n] * H[p, n] + D[h] * x[b, t, h, p]
        y          = y * silu(z[b, t, h, p])       (when a gate is given)

with B and C one vector of width N per token, shared by every head (a single
group).  With G groups (Mamba-2 layers split the heads into groups of consecutive
heads), B and C are [B, L, G, N] and head h reads group h // (H / G): each group is the
single-group map on its own heads with its own B and C.  The structured-matrix form the
page names is the same map written as
y = M (x) with M[t, s] = C_t . B_s * exp(a (cum_t - cum_s)) * dt_s for s <= t
(cum = running sum of dt): a masked, decayed product C B^T, i.e. linear attention
with a decay mask.  The tests check the recurrence below against that form.

The recurrence is written out one time step at a time over whole [B, H, P, N]
slabs; no chunking, no reordering.
"""
from __future__ import annotations

import numpy as np


def _softplus(u):
    return np.logaddexp(0.0, u)


def _silu(v):
    return v / (1.0 + np.exp(-v))


def ssd(x, delta, a, Bm, Cm, D=None, z=None, h0=None, delta_softplus=False, delta_bias=None):
    """All arrays float64 (or anything numpy widens exactly).

    x, z: [B, L, H, P];  delta: [B, L, H];  a: [H];  Bm, Cm: [B, L, N], or [B, L, G, N] for G
    groups of H / G consecutive heads;  D: [H];  h0: [B, H, P, N];  delta_bias: [H].
    Returns y [B, L, H, P] and h_last [B, H, P, N].
    """
    Bm = np.asarray(Bm)
    if Bm.ndim == 4:   # groups: the single-group map per group of heads
        G = Bm.shape[2]
        H = np.asarray(x).shape[2]
        assert H % G == 0, (H, G)
        hg = H // G
        ys, hs = [], []
        for g in range(G):
            sel = slice(g * hg, (g + 1) * hg)
            pick = lambda t, ax: None if t is None else np.take(np.asarray(t), np.arange(g * hg, (g + 1) * hg), axis=ax)
            yg, hlg = ssd(pick(x, 2), pick(delta, 2), np.asarray(a)[sel], Bm[:, :, g], np.asarray(Cm)[:, :, g],
                          None if D is None else np.asarray(D)[sel], pick(z, 2), pick(h0, 1), delta_softplus,
                          None if delta_bias is None else np.asarray(delta_bias)[sel])
            ys.append(yg)
            hs.append(hlg)
        return np.concatenate(ys, axis=2), np.concatenate(hs, axis=1)
    x = np.asarray(x, dtype=np.float64)
    Bsz, L, H, P = x.shape
    Bm = np.asarray(Bm, dtype=np.float64)
    Cm = np.asarray(Cm, dtype=np.float64)
    N = Bm.shape[2]
    a = np.asarray(a, dtype=np.float64)
    dt = np.asarray(delta, dtype=np.float64)
    if delta_bias is not None:
        dt = dt + np.asarray(delta_bias, dtype=np.float64)[None, None, :]
    if delta_softplus:
        dt = _softplus(dt)
    state = np.zeros((Bsz, H, P, N)) if h0 is None else np.array(h0, dtype=np.float64, copy=True)
    y = np.empty((Bsz, L, H, P))
    for t in range(L):
        step = dt[:, t, :]                                            # [B, H]
        decay = np.exp(step * a[None, :])[:, :, None, None]          # [B, H, 1, 1]
        drive = (step[:, :, None] * x[:, t, :, :])[:, :, :, None] * Bm[:, t, None, None, :]
        state = decay * state + drive                                 # [B, H, P, N]
        yt = np.einsum("bhpn,bn->bhp", state, Cm[:, t, :])
        if D is not None:
            yt = yt + np.asarray(D, dtype=np.float64)[None, :, None] * x[:, t, :, :]
        if z is not None:
            yt = yt * _silu(np.asarray(z, dtype=np.float64)[:, t, :, :])
        y[:, t] = yt
    return y, state


def _widen(a, dtype):
    if a is None:
        return None
    if dtype == "bf16":
        return (np.ascontiguousarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)) \
            .view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def ssd_storage(inp: dict, batches=None, heads=None):
    """The oracle on storage-form inputs (a dict from ``synth.ssd_inputs``): bf16 bit
    patterns or float32, widened exactly.  batches / heads select a subset (lists of
    indices); the result then covers only those rows and heads."""
    dt = inp["dtype"]
    if np.asarray(inp["B"]).ndim == 4 and heads is not None:
        # groups and a subset of heads: each selected head with its own group's B and C
        H, G = np.asarray(inp["x"]).shape[2], np.asarray(inp["B"]).shape[2]
        ys, hls = [], []
        for h in heads:
            g = h // (H // G)
            one = dict(inp)
            one["B"] = np.asarray(inp["B"])[:, :, g]
            one["C"] = np.asarray(inp["C"])[:, :, g]
            yh, hh = ssd_storage(one, batches, [h])
            ys.append(yh)
            hls.append(hh)
        return np.concatenate(ys, axis=2), np.concatenate(hls, axis=1)
    bs = slice(None) if batches is None else np.asarray(batches)
    hs = slice(None) if heads is None else np.asarray(heads)
    pick = lambda t: None if t is None else _widen(np.asarray(t)[bs][:, :, hs], dt)
    x = pick(inp["x"])
    z = pick(inp.get("z"))
    delta = pick(inp["delta"])
    Bm = _widen(np.asarray(inp["B"])[bs], dt)
    Cm = _widen(np.asarray(inp["C"])[bs], dt)
    a = np.asarray(inp["A"], dtype=np.float64)[hs]
    D = None if inp.get("Dskip") is None else np.asarray(inp["Dskip"], dtype=np.float64)[hs]
    bias = None if inp.get("delta_bias") is None else np.asarray(inp["delta_bias"], dtype=np.float64)[hs]
    h0 = None if inp.get("h0") is None else np.asarray(inp["h0"], dtype=np.float64)[bs][:, hs]
    return ssd(x, delta, a, Bm, Cm, D, z, h0, inp.get("delta_softplus", False), bias)


def ssd_bwd(x, delta, a, Bm, Cm, D=None, z=None, h0=None, delta_softplus=False, delta_bias=None,
            gy=None, g_last=None):
    """Reverse-mode derivative of ``ssd`` (one B/C group: Bm, Cm [B, L, N]) for the loss
    <gy, y> + <g_last, h_last>, all float64.

    The chain rule through the recurrence above, one step at a time from the last: with
    lam = dLoss/dH after step t ([B, H, P, N]) and gy0 = gy * silu(z):
        lam     += gy0 (x) C_t                                  (the readout of step t)
        dC_t    += sum_{h,p} gy0[h,p] H_t[h,p,:],    dD += sum gy0 x_t,    dx_t = D gy0
        dx_t    += dt sum_n lam B_t,    dB_t += sum_{h,p} lam dt x_t,
        d(dt)    = sum_{p,n} lam (a A_bar H_{t-1} + x_t B_t),   da += sum lam dt A_bar H_{t-1}
        lam      = A_bar lam                                     (to step t - 1)
    d(dt) is taken back through the softplus and the bias to the raw step size; dh0 is the
    final lam, and dz = gy y0 silu'(z) with y0 the ungated output.
    Returns a dict of dx, ddelta, dA, dB, dC, dD, dz, dh0, ddelta_bias (None where the input
    is absent)."""
    x = np.asarray(x, dtype=np.float64)
    Bsz, L, H, P = x.shape
    Bm = np.asarray(Bm, dtype=np.float64)
    Cm = np.asarray(Cm, dtype=np.float64)
    N = Bm.shape[2]
    a = np.asarray(a, dtype=np.float64)
    raw = np.asarray(delta, dtype=np.float64)
    if delta_bias is not None:
        raw = raw + np.asarray(delta_bias, dtype=np.float64)[None, None, :]
    dt = _softplus(raw) if delta_softplus else raw
    Dv = None if D is None else np.asarray(D, dtype=np.float64)
    zz = None if z is None else np.asarray(z, dtype=np.float64)
    gy = np.asarray(gy, dtype=np.float64)
    # forward, keeping every state and the ungated outputs
    states = np.empty((L + 1, Bsz, H, P, N))
    states[0] = 0.0 if h0 is None else np.asarray(h0, dtype=np.float64)
    abar = np.exp(dt * a[None, None, :])                              # [B, L, H]
    y0 = np.empty((Bsz, L, H, P))
    for t in range(L):
        drive = (dt[:, t, :, None] * x[:, t])[:, :, :, None] * Bm[:, t, None, None, :]
        states[t + 1] = abar[:, t, :, None, None] * states[t] + drive
        y0[:, t] = np.einsum("bhpn,bn->bhp", states[t + 1], Cm[:, t])
        if Dv is not None:
            y0[:, t] += Dv[None, :, None] * x[:, t]
    if zz is not None:
        sg = 1.0 / (1.0 + np.exp(-zz))
        gy0 = gy * zz * sg
        dz = gy * y0 * sg * (1.0 + zz * (1.0 - sg))
    else:
        gy0, dz = gy, None
    lam = np.zeros((Bsz, H, P, N)) if g_last is None else np.array(g_last, dtype=np.float64, copy=True)
    dx = np.zeros_like(x)
    ddt = np.zeros((Bsz, L, H))
    da = np.zeros(H)
    dB = np.zeros_like(Bm)
    dC = np.zeros_like(Cm)
    dD = None if Dv is None else np.zeros(H)
    for t in range(L - 1, -1, -1):
        g = gy0[:, t]                                                 # [B, H, P]
        lam = lam + g[:, :, :, None] * Cm[:, t, None, None, :]
        dC[:, t] += np.einsum("bhp,bhpn->bn", g, states[t + 1])
        if Dv is not None:
            dD += np.einsum("bhp,bhp->h", g, x[:, t])
            dx[:, t] += Dv[None, :, None] * g
        st = dt[:, t]                                                 # [B, H]
        dx[:, t] += st[:, :, None] * np.einsum("bhpn,bn->bhp", lam, Bm[:, t])
        dB[:, t] += np.einsum("bhpn,bh,bhp->bn", lam, st, x[:, t])
        hprev = np.einsum("bhpn,bhpn->bh", lam, states[t])           # sum lam H_{t-1}
        ab = abar[:, t]
        ddt[:, t] = a[None, :] * ab * hprev + np.einsum("bhpn,bhp,bn->bh", lam, x[:, t], Bm[:, t])
        da += np.einsum("bh,bh->h", st * ab, hprev)
        lam = ab[:, :, None, None] * lam
    draw = ddt * (1.0 / (1.0 + np.exp(-raw))) if delta_softplus else ddt
    return {"dx": dx, "ddelta": draw, "dA": da, "dB": dB, "dC": dC, "dD": dD, "dz": dz, "dh0": lam,
            "ddelta_bias": None if delta_bias is None else draw.sum(axis=(0, 1))}


def ssd_bwd_storage(inp: dict, gy, g_last=None):
    """``ssd_bwd`` on storage-form inputs (``synth.ssd_inputs``, one B/C group), widened
    exactly; gy in the inputs' storage form, g_last float32 or None."""
    dt = inp["dtype"]
    w = lambda k: None if inp.get(k) is None else _widen(inp[k], dt)
    f = lambda k: None if inp.get(k) is None else np.asarray(inp[k], dtype=np.float64)
    return ssd_bwd(w("x"), w("delta"), f("A"), w("B"), w("C"), f("Dskip"), w("z"), f("h0"),
                   inp.get("delta_softplus", False), f("delta_bias"), _widen(gy, dt),
                   None if g_last is None else np.asarray(g_last, dtype=np.float64))
