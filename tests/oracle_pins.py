"""Pins for the fp64 oracle: facts fixed by the source pages and by mathematics.

Each ``pin_*`` takes a scan function with the signature

    scan_fn(x, delta, A, Bm, Cm, Dskip=None, z=None, h0=None, delta_softplus=False)
        -> (y [B, L, D], h_last [B, D, N])      (all float64)

and returns the largest error it finds (a float; 0 means exact).  The tests
run every pin against both oracles, and against deliberately broken copies of
the numpy oracle to show that each plausible mistake trips at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def c_oracle_scan(x, delta, A, Bm, Cm, Dskip=None, z=None, h0=None, delta_softplus=False):
    import oracle
    x = np.asarray(x, dtype=np.float64)
    Bsz, L, D = x.shape
    N = A.shape[1]
    cb, cd = np.meshgrid(np.arange(Bsz), np.arange(D), indexing="ij")
    cb, cd = cb.reshape(-1), cd.reshape(-1)

    def series(a):
        return None if a is None else np.asarray(a, dtype=np.float64)[cb, :, cd]

    h0c = None if h0 is None else np.asarray(h0, dtype=np.float64).reshape(Bsz * D, N)
    y, h = oracle.scan_f64(series(x), series(delta), A, Bm, Cm, Dskip, series(z), h0c,
                           delta_softplus, cb, cd, nthreads=2)
    return y.reshape(Bsz, D, L).transpose(0, 2, 1), h.reshape(Bsz, D, N)


def numpy_oracle_scan(*args, **kw):
    from oracle.numpy_ref import scan_np
    return scan_np(*args, **kw)


def _rand_problem(seed, Bsz=2, L=23, D=5, N=4, gate=False, h0=False, a_random=True):
    g = np.random.default_rng(seed)
    x = g.standard_normal((Bsz, L, D))
    delta = np.exp(g.uniform(np.log(1e-3), np.log(0.5), (Bsz, L, D)))
    A = -(np.arange(1, N + 1)[None, :] * np.ones((D, 1)))
    if a_random:
        A = A * np.exp(0.5 * g.standard_normal((D, N)))
    Bm = g.standard_normal((Bsz, L, N))
    Cm = g.standard_normal((Bsz, L, N))
    Dskip = 1.0 + 0.3 * g.standard_normal(D)
    z = g.standard_normal((Bsz, L, D)) if gate else None
    hh = g.standard_normal((Bsz, D, N)) if h0 else None
    return dict(x=x, delta=delta, A=A, Bm=Bm, Cm=Cm, Dskip=Dskip, z=z, h0=hh)


def _call(scan_fn, p, **kw):
    args = dict(p)
    args.update(kw)
    return scan_fn(args["x"], args["delta"], args["A"], args["Bm"], args["Cm"], args["Dskip"],
                   args["z"], args["h0"], args.get("delta_softplus", False))


def _relerr(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(1.0, float(np.max(np.abs(b)))))


# -- pages' worked example ---------------------------------------------------
def pin_worked_example(scan_fn):
    """One step with N=2 from h0=(0.3, 0.1): h1=(0.47, 0.45), y1=0.245."""
    with open(os.path.join(GOLDEN, "worked_example_2d.json")) as f:
        g = json.load(f)
    A = np.log(np.array(g["A_bar_diag"]))[None, :]
    x = np.array([[[g["x1"]]]])
    delta = np.ones((1, 1, 1))
    Bm = np.array(g["B_bar"])[None, None, :]
    Cm = np.array(g["C"])[None, None, :]
    h0 = np.array(g["h0"])[None, None, :]
    y, h = scan_fn(x, delta, A, Bm, Cm, np.zeros(1), None, h0, False)
    return max(abs(float(y[0, 0, 0]) - g["expected_y1"]),
               float(np.max(np.abs(h[0, 0] - np.array(g["expected_h1"])))))


# -- convolution view of the time-invariant case -----------------------------
def _lti_problem(seed, Bsz=2, L=40, D=3, N=5):
    g = np.random.default_rng(seed)
    x = g.standard_normal((Bsz, L, D))
    dd = np.exp(g.uniform(np.log(1e-2), np.log(0.5), D))           # one step size per channel
    delta = np.broadcast_to(dd, (Bsz, L, D)).copy()
    A = -np.exp(g.standard_normal((D, N)))
    Bv = g.standard_normal((Bsz, N))
    Cv = g.standard_normal((Bsz, N))
    Bm = np.broadcast_to(Bv[:, None, :], (Bsz, L, N)).copy()
    Cm = np.broadcast_to(Cv[:, None, :], (Bsz, L, N)).copy()
    Dskip = g.standard_normal(D)
    return dict(x=x, delta=delta, A=A, Bm=Bm, Cm=Cm, Dskip=Dskip, z=None, h0=None,
                dd=dd, Bv=Bv, Cv=Cv)


def _lti_kernel(p, b, d, L):
    """K_k = sum_n C_n * A_bar_n**k * B_bar_n  (impulse response; k = 0 .. L-1)."""
    a_bar = np.exp(p["dd"][d] * p["A"][d])                    # [N]
    b_bar = p["dd"][d] * p["Bv"][b]
    k = np.arange(L)[:, None]
    return (p["Cv"][b][None, :] * a_bar[None, :] ** k * b_bar[None, :]).sum(axis=1)


def pin_convolution_bruteforce(scan_fn, seed=11):
    """y_t = sum_{s<=t} K_{t-s} x_s + D x_t  for constant delta, B, C and h0 = 0."""
    p = _lti_problem(seed)
    y, _ = _call(scan_fn, p)
    Bsz, L, D = p["x"].shape
    err = 0.0
    for b in range(Bsz):
        for d in range(D):
            K = _lti_kernel(p, b, d, L)
            ref = np.array([sum(K[t - s] * p["x"][b, s, d] for s in range(t + 1)) for t in range(L)])
            ref = ref + p["Dskip"][d] * p["x"][b, :, d]
            err = max(err, _relerr(y[b, :, d], ref))
    return err


def pin_convolution_fft(scan_fn, seed=12):
    """Same identity evaluated with a zero-padded FFT (length 2L)."""
    p = _lti_problem(seed, L=64)
    y, _ = _call(scan_fn, p)
    Bsz, L, D = p["x"].shape
    err = 0.0
    for b in range(Bsz):
        for d in range(D):
            K = _lti_kernel(p, b, d, L)
            conv = np.fft.irfft(np.fft.rfft(p["x"][b, :, d], 2 * L) * np.fft.rfft(K, 2 * L), 2 * L)[:L]
            err = max(err, _relerr(y[b, :, d], conv + p["Dskip"][d] * p["x"][b, :, d]))
    return err


# -- unrolled time-varying form ----------------------------------------------
def pin_unrolled_time_varying(scan_fn, seed=13):
    """Unrolling the recurrence with time-varying delta, B, C (and a start state):

        y_t = sum_n C_{t,n} [ exp(A_n S_t) h0_n + sum_{s<=t} exp(A_n (S_t - S_s)) delta_s B_{s,n} x_s ]
              + D x_t,      S_t = sum_{r<=t} delta_r

    evaluated by brute force for every (t, s) pair; gate applied afterwards.
    """
    p = _rand_problem(seed, Bsz=2, L=17, D=4, N=3, gate=True, h0=True)
    y, h_last = _call(scan_fn, p)
    Bsz, L, D = p["x"].shape
    N = p["A"].shape[1]
    err = 0.0
    for b in range(Bsz):
        for d in range(D):
            S = np.cumsum(p["delta"][b, :, d])
            for t in range(L):
                hv = np.exp(p["A"][d] * S[t]) * p["h0"][b, d]
                for s in range(t + 1):
                    hv = hv + (np.exp(p["A"][d] * (S[t] - S[s])) * p["delta"][b, s, d]
                               * p["Bm"][b, s] * p["x"][b, s, d])
                ref = float(np.dot(p["Cm"][b, t], hv)) + p["Dskip"][d] * p["x"][b, t, d]
                zt = p["z"][b, t, d]
                ref *= zt / (1.0 + math.exp(-zt))
                err = max(err, abs(y[b, t, d] - ref) / max(1.0, abs(ref)))
                if t == L - 1:
                    err = max(err, _relerr(h_last[b, d], hv))
    assert N == 3
    return err


# -- closed forms and special cases -------------------------------------------
def pin_closed_form_geometric(scan_fn):
    """Constant x, delta, B and h0 = 0: h_{L-1,n} = delta B_n x (1 - a_n^L) / (1 - a_n), a_n = exp(delta A_n)."""
    L, N = 300, 4
    A = -np.array([[0.5, 1.0, 2.0, 7.0]])
    dt, xv = 0.03, 1.7
    Bv = np.array([0.4, -1.2, 2.0, 0.9])
    x = np.full((1, L, 1), xv)
    delta = np.full((1, L, 1), dt)
    Bm = np.broadcast_to(Bv, (1, L, N)).copy()
    Cm = np.ones((1, L, N))
    _, h = scan_fn(x, delta, A, Bm, Cm, None, None, None, False)
    a = np.exp(dt * A[0])
    ref = dt * Bv * xv * (1 - a ** L) / (1 - a)
    return _relerr(h[0, 0], ref)


def pin_delta_zero(scan_fn, seed=14):
    """delta = 0: the state never moves, so h_last = h0 and y_t = C_t . h0 + D x_t."""
    p = _rand_problem(seed, h0=True)
    p["delta"] = np.zeros_like(p["delta"])
    y, h = _call(scan_fn, p)
    ref_y = np.einsum("bln,bdn->bld", p["Cm"], p["h0"]) + p["Dskip"][None, None, :] * p["x"]
    return max(_relerr(h, p["h0"]), _relerr(y, ref_y))


def pin_linearity(scan_fn, seed=15, gate=False):
    """With h0 = 0 and delta, B, C, z fixed, y is linear in x."""
    p = _rand_problem(seed, gate=gate)
    g = np.random.default_rng(seed + 1)
    x1, x2 = g.standard_normal(p["x"].shape), g.standard_normal(p["x"].shape)
    al, be = 0.7, -1.9
    y1, _ = _call(scan_fn, p, x=x1)
    y2, _ = _call(scan_fn, p, x=x2)
    y12, _ = _call(scan_fn, p, x=al * x1 + be * x2)
    return _relerr(y12, al * y1 + be * y2)


def pin_split_resume(scan_fn, seed=16, T=9):
    """Scanning [0, L) equals scanning [T, L) from the state left by [0, T)."""
    p = _rand_problem(seed, gate=True, h0=True)
    y, h = _call(scan_fn, p)
    cut = lambda a, lo, hi: None if a is None else a[:, lo:hi]
    L = p["x"].shape[1]
    ya, ha = _call(scan_fn, p, **{k: cut(p[k], 0, T) for k in ("x", "delta", "Bm", "Cm", "z")})
    yb, hb = _call(scan_fn, p, h0=ha, **{k: cut(p[k], T, L) for k in ("x", "delta", "Bm", "Cm", "z")})
    return max(_relerr(np.concatenate([ya, yb], axis=1), y), _relerr(hb, h))


def pin_carry_algebra(scan_fn, seed=17, T=8):
    """Chunk carry: h_L = P * h_T + H with P_n = exp(A_n * sum_{t in [T, L)} delta_t) and
    H = state reached over [T, L) from zero.  This is the combine (P1, H1) o (P2, H2) =
    (P2 P1, P2 H1 + H2) applied once."""
    p = _rand_problem(seed)
    L = p["x"].shape[1]
    _, hT = _call(scan_fn, p, **{k: p[k][:, :T] for k in ("x", "delta", "Bm", "Cm")})
    _, hL = _call(scan_fn, p)
    _, H = _call(scan_fn, p, **{k: p[k][:, T:] for k in ("x", "delta", "Bm", "Cm")})
    P = np.exp(p["A"][None, :, :] * p["delta"][:, T:, :].sum(axis=1)[:, :, None])
    return _relerr(hL, P * hT + H)


def pin_n_separability(scan_fn, seed=18):
    """y(all N states) = sum_n y(state n alone) - (N - 1) D x   (no gate)."""
    p = _rand_problem(seed, N=5)
    y, _ = _call(scan_fn, p)
    N = p["A"].shape[1]
    acc = np.zeros_like(y)
    for n in range(N):
        yn, _ = _call(scan_fn, p, A=p["A"][:, n:n + 1], Bm=p["Bm"][:, :, n:n + 1], Cm=p["Cm"][:, :, n:n + 1])
        acc += yn
    return _relerr(y, acc - (N - 1) * p["Dskip"][None, None, :] * p["x"])


def pin_textbook_lti(scan_fn, seed=19):
    """Constant delta, B, C reduce to the dense linear recurrence
    state = A_bar @ state + B_bar u_t;  y_t = C @ state + D u_t
    (chipfoundryservices page, Lab 2) with A_bar = diag(exp(delta A)), B_bar = delta B."""
    p = _lti_problem(seed, Bsz=1, L=30, D=1, N=4)
    y, _ = _call(scan_fn, p)
    A_bar = np.diag(np.exp(p["dd"][0] * p["A"][0]))
    B_bar = (p["dd"][0] * p["Bv"][0]).reshape(-1, 1)
    C = p["Cv"][0].reshape(1, -1)
    Dm = np.array([[p["Dskip"][0]]])
    state = np.zeros(4)
    out = []
    for u_t in p["x"][0, :, 0].reshape(-1, 1):
        state = A_bar @ state + (B_bar @ u_t.reshape(-1, 1)).reshape(-1)
        out.append((C @ state + Dm @ u_t.reshape(-1, 1)).item())
    return _relerr(y[0, :, 0], np.array(out))


def pin_softplus_inverse(scan_fn, seed=20):
    """softplus(log(expm1(delta))) = delta: the softplus mode on u equals the plain mode on delta."""
    p = _rand_problem(seed, gate=True, h0=True)
    y_ref, h_ref = _call(scan_fn, p)
    u = np.log(np.expm1(p["delta"]))
    y_sp, h_sp = _call(scan_fn, p, delta=u, delta_softplus=True)
    return max(_relerr(y_sp, y_ref), _relerr(h_sp, h_ref))


def pin_gate_closed_form(scan_fn, seed=21):
    """sigmoid(ln 3) = 3/4, so a gate z = ln 3 scales the ungated output by (3/4) ln 3;
    z = 0 zeroes it."""
    p = _rand_problem(seed, h0=True)
    y0, _ = _call(scan_fn, p)
    yl3, _ = _call(scan_fn, p, z=np.full(p["x"].shape, math.log(3.0)))
    yz, _ = _call(scan_fn, p, z=np.zeros(p["x"].shape))
    return max(_relerr(yl3, 0.75 * math.log(3.0) * y0), float(np.max(np.abs(yz))))


def pin_nan_propagation(scan_fn, seed=22):
    """A NaN in x[b, t, d] poisons y[b, t' >= t, d] and h_last[b, d, :] and nothing else.
    Returns 0 when that holds, 1 otherwise."""
    p = _rand_problem(seed)
    x = p["x"].copy()
    x[1, 7, 2] = np.nan
    y, h = _call(scan_fn, p, x=x)
    bad = np.isnan(y)
    expect = np.zeros_like(bad)
    expect[1, 7:, 2] = True
    hbad = np.isnan(h)
    hexp = np.zeros_like(hbad)
    hexp[1, 2, :] = True
    return 0.0 if (np.array_equal(bad, expect) and np.array_equal(hbad, hexp)) else 1.0


PINS = {
    "worked_example": (pin_worked_example, 1e-15),
    "convolution_bruteforce": (pin_convolution_bruteforce, 1e-12),
    "convolution_fft": (pin_convolution_fft, 1e-12),
    "unrolled_time_varying": (pin_unrolled_time_varying, 1e-12),
    "closed_form_geometric": (pin_closed_form_geometric, 1e-12),
    "delta_zero": (pin_delta_zero, 1e-14),
    "linearity": (pin_linearity, 1e-12),
    "linearity_gated": (lambda f: pin_linearity(f, gate=True), 1e-12),
    "split_resume": (pin_split_resume, 1e-14),
    "carry_algebra": (pin_carry_algebra, 1e-12),
    "n_separability": (pin_n_separability, 1e-12),
    "textbook_lti": (pin_textbook_lti, 1e-12),
    "softplus_inverse": (pin_softplus_inverse, 1e-12),
    "gate_closed_form": (pin_gate_closed_form, 1e-13),
    "nan_propagation": (pin_nan_propagation, 0.5),
}
