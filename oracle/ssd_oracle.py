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
