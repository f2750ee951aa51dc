"""Helpers shared by the GPU parity tests (device upload, the tolerance rule)."""
from __future__ import annotations

import numpy as np

# Parity rule per element: |gpu - oracle| <= max(RTOL * |oracle|, ATOL).
# bf16 inputs with an fp32 state: 1e-2 relative with a 1e-3 absolute floor.
# fp32 inputs (and every fp32 state): 1e-4 relative with a 1e-5 absolute floor.
TOL = {"bf16": (1e-2, 1e-3), "f32": (1e-4, 1e-5)}


def to_dev(a, dtype):
    import torch
    if a is None:
        return None
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_host(t):
    import torch
    return t.float().cpu().numpy().astype(np.float64) if t.dtype != torch.float64 else t.cpu().numpy()


def device_inputs(inp):
    import torch
    dt = inp["dtype"]
    out = {k: to_dev(inp[k], dt) for k in ("x", "delta", "z", "B", "C")}
    out["A"] = torch.from_numpy(inp["A"]).cuda()
    out["D"] = None if inp.get("Dskip") is None else torch.from_numpy(inp["Dskip"]).cuda()
    out["h0"] = None if inp.get("h0") is None else torch.from_numpy(inp["h0"]).cuda()
    return out


def compare(g, r, dtype, what="y", scale_floor=0.0):
    """Returns a stats dict; 'bad' counts elements outside the rule (NaN must match NaN).

    scale_floor > 0 raises the absolute floor to scale_floor * max|r| for inputs whose
    outputs are far from O(1) (the fixed floor assumes O(1) terms)."""
    rtol, atol = TOL[dtype]
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    nan_g, nan_r = np.isnan(g), np.isnan(r)
    both = nan_g & nan_r
    err = np.where(both, 0.0, np.abs(g - r))
    if scale_floor and r.size:
        atol = max(atol, scale_floor * float(np.max(np.abs(np.where(nan_r, 0, r)))))
    lim = np.maximum(rtol * np.abs(np.where(nan_r, 0, r)), atol)
    ratio = np.where(both, 0.0, err / lim)
    ratio = np.where(nan_g ^ nan_r, np.inf, ratio)
    bad = int((ratio > 1.0).sum())
    nz = np.abs(r) > 0
    unfloored = float(np.max(np.where(nz & ~both, err / np.where(nz, np.abs(r), 1), 0))) if g.size else 0.0
    norm = float(np.linalg.norm(np.where(both, 0, g - r)) / max(np.linalg.norm(np.where(nan_r, 0, r)), 1e-300)) if g.size else 0.0
    return {"what": what, "bad": bad, "n": int(g.size),
            "max_abs": float(err.max()) if g.size else 0.0,
            "worst_ratio": float(ratio.max()) if g.size else 0.0,
            "max_rel_unfloored": unfloored, "normwise": norm}


def assert_close(g, r, dtype, what="y", scale_floor=0.0):
    st = compare(g, r, dtype, what, scale_floor)
    assert st["bad"] == 0, f"{what}: {st['bad']}/{st['n']} elements out of tolerance; {st}"
    return st


def sample_channels(batch, dim, n):
    """n distinct (b, d) channels spread over the batch and the channel axis (first and last included)."""
    ch = {(0, 0), (batch - 1, dim - 1)}
    i = 0
    while len(ch) < min(n, batch * dim):
        ch.add((i % batch, (i * 977 + 13) % dim))
        i += 1
    return sorted(ch)


# Backward parity rule per gradient tensor G (the pages state no tolerance for the
# backward; derived from the arithmetic): |gpu - oracle| <= max(RTOL * |oracle|,
# FLOOR * max|oracle over G|).  The floor is relative to the tensor's own scale because
# gradients are sums whose terms cancel (ddelta = sum of terms of both signs; dB, dC sum
# over channels; dA over batch and time): an fp32 sum of K terms of size s carries an
# error of about K * 6e-8 * s that no relative bound on a small result can cover.
# bf16 outputs: RTOL 1e-2 (a bf16 rounding is 2^-8), FLOOR 2e-3.  fp32 outputs: RTOL 1e-3,
# FLOOR 1e-4 (the adjoint runs through L fp32 decays and exps).
BWD_TOL = {"bf16": (1e-2, 2e-3), "f32": (1e-3, 1e-4)}


def assert_close_grad(g, r, dtype, what):
    rtol, floor = BWD_TOL[dtype]
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite gradient"
    scale = float(np.max(np.abs(r))) if r.size else 0.0
    # an all-zero result (e.g. dA with h0 = 0 and one step) keeps a tiny absolute floor
    lim = np.maximum(np.maximum(rtol * np.abs(r), floor * scale), 1e-7)
    err = np.abs(g - r)
    ratio = float(np.max(err / np.where(lim > 0, lim, 1.0))) if r.size else 0.0
    bad = int((err > lim).sum())
    assert bad == 0, f"{what}: {bad}/{r.size} out of tolerance, worst ratio {ratio:.3f}, scale {scale:.3g}"
    return ratio
