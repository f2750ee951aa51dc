"""Pins of the oracle's discretisation variants and of the delta bias.

The scan's default discretisation is the Mamba one (A_bar = exp(dt A), B_bar = dt B).
Two more are defined for a diagonal A:

* zero-order hold, B_bar = A^-1 (exp(dt A) - I) B (skill page "State Space Models
  Mamba", "Discretization" docstring; brentwoodlivery "State-space models (Mamba,
  S4)", "From Continuous to Discrete" and its discretisation flashcard);
* bilinear, A_bar = (I + dt/2 A)(I - dt/2 A)^-1, B_bar = (I - dt/2 A)^-1 dt B
  (chipfoundryservices glossary "State Space Models & Mamba", Lab 1).

The delta bias is the bias of the linear map that produces delta, added before the
softplus (skill page, MambaBlock listing: dt_proj with bias=True, then softplus).

None of the pins below restates the oracle's formulas.  The discretised matrices come
from scipy.signal.cont2discrete (a block matrix exponential for "zoh", a linear solve
for "bilinear"), from integrating the continuous ODE, or from what the continuous
system fixes (its equilibrium).
"""
from __future__ import annotations

import inspect

import numpy as np
import pytest
from scipy.integrate import solve_ivp
from scipy.signal import cont2discrete

import oracle
from oracle import numpy_ref

KINDS = ["mamba", "zoh", "bilinear"]


def _problem(seed, Bsz=2, L=12, D=3, N=4, softplus=False, gate=False):
    rng = np.random.default_rng(seed)
    p = {
        "x": rng.standard_normal((Bsz, L, D)),
        "delta": np.exp(rng.uniform(np.log(1e-3), np.log(0.5), (Bsz, L, D))),
        "A": -np.exp(rng.normal(0.0, 1.0, (D, N))),
        "Bm": rng.standard_normal((Bsz, L, N)),
        "Cm": rng.standard_normal((Bsz, L, N)),
        "Dskip": rng.normal(1.0, 0.1, D),
        "z": rng.standard_normal((Bsz, L, D)) if gate else None,
        "h0": rng.standard_normal((Bsz, D, N)),
    }
    if softplus:
        p["delta"] = np.log(np.expm1(p["delta"]))
    return p


def _run_c(p, kind, softplus=False, delta_bias=None):
    Bsz, L, D = p["x"].shape
    N = p["A"].shape[1]
    cb, cd = np.meshgrid(np.arange(Bsz), np.arange(D), indexing="ij")
    cb, cd = cb.reshape(-1), cd.reshape(-1)
    ser = lambda a: None if a is None else a[cb, :, cd]
    y, h = oracle.scan_f64(ser(p["x"]), ser(p["delta"]), p["A"], p["Bm"], p["Cm"], p["Dskip"],
                           ser(p["z"]), p["h0"][cb, cd, :], softplus, cb, cd, 1, kind, delta_bias)
    return y.reshape(Bsz, D, L).transpose(0, 2, 1), h.reshape(Bsz, D, N)


def _run_np(p, kind, softplus=False, delta_bias=None, fn=None):
    fn = fn or numpy_ref.scan_np
    return fn(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], p["Dskip"], p["z"], p["h0"], softplus,
              discretization=kind, delta_bias=delta_bias)


def _run_scipy(p, kind):
    """The same scan with every step's (A_bar, B_bar) from scipy's cont2discrete on the dense
    diagonal system: a library routine, not the oracle's formula."""
    x, dl, A, Bm, Cm, Dk, h0 = p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], p["Dskip"], p["h0"]
    Bsz, L, D = x.shape
    N = A.shape[1]
    y = np.empty((Bsz, L, D))
    h_last = np.empty((Bsz, D, N))
    for b in range(Bsz):
        for d in range(D):
            h = h0[b, d].copy()
            for t in range(L):
                dt = dl[b, t, d]
                sys_c = (np.diag(A[d]), Bm[b, t][:, None], Cm[b, t][None, :], np.zeros((1, 1)))
                if kind == "mamba":   # exact A_bar, first-order B_bar: not a cont2discrete method
                    Ad = np.diag(np.exp(dt * A[d]))
                    Bd = dt * Bm[b, t][:, None]
                else:
                    Ad, Bd, _, _, _ = cont2discrete(sys_c, dt, method=kind)
                h = Ad @ h + Bd[:, 0] * x[b, t, d]
                y[b, t, d] = Cm[b, t] @ h + Dk[d] * x[b, t, d]
            h_last[b, d] = h
    return y, h_last


@pytest.mark.parametrize("kind", ["zoh", "bilinear"])
@pytest.mark.parametrize("impl", ["c", "numpy"])
def test_matches_scipy_cont2discrete(kind, impl):
    p = _problem(1)
    yr, hr = _run_scipy(p, kind)
    y, h = (_run_c if impl == "c" else _run_np)(p, kind)
    np.testing.assert_allclose(y, yr, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(h, hr, rtol=1e-11, atol=1e-12)


def test_zoh_is_the_exact_ode_solution():
    """Zero-order hold: holding x_t over a step of length dt, the continuous system
    h' = A h + B_t x_t lands exactly on the discrete state."""
    p = _problem(2, Bsz=1, L=5, D=2, N=3)
    y, h_or = _run_c(p, "zoh")
    A, Bm, x, dl = p["A"], p["Bm"], p["x"], p["delta"]
    for d in range(2):
        h = p["h0"][0, d].copy()
        for t in range(5):
            rhs = lambda _s, v, d=d, t=t: A[d] * v + Bm[0, t] * x[0, t, d]
            sol = solve_ivp(rhs, (0.0, dl[0, t, d]), h, method="DOP853", rtol=1e-13, atol=1e-15)
            h = sol.y[:, -1]
        np.testing.assert_allclose(h_or[0, d], h, rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("kind", ["zoh", "bilinear"])
def test_equilibrium_of_the_continuous_system(kind):
    """With x, B held constant the continuous system settles at h* = -A^-1 B x.  Both
    ZOH and the bilinear map keep that fixed point for every step size; the first-order
    B_bar = dt B does not (its fixed point is dt B x / (1 - exp(dt A)))."""
    rng = np.random.default_rng(3)
    D, N, L = 3, 4, 400
    A = -np.exp(rng.normal(0.0, 0.5, (D, N)))
    Bv = rng.standard_normal(N)
    xv = rng.standard_normal(D)
    p = {"x": np.broadcast_to(xv, (1, L, D)).copy(),
         "delta": np.exp(rng.uniform(np.log(0.3), np.log(2.0), (1, L, D))),
         "A": A, "Bm": np.broadcast_to(Bv, (1, L, N)).copy(), "Cm": np.ones((1, L, N)),
         "Dskip": np.zeros(D), "z": None, "h0": np.zeros((1, D, N))}
    star = -Bv[None, :] * xv[:, None] / A
    for fn in (_run_c, _run_np):
        _, h = fn(p, kind)
        np.testing.assert_allclose(h[0], star, rtol=1e-12, atol=1e-13)
    _, h_mamba = _run_c(p, "mamba")
    assert np.max(np.abs(h_mamba[0] - star)) > 1e-2


def test_zoh_with_zero_A_is_the_first_order_step():
    """A = 0: no decay, and B_bar = dt B (the limit of A^-1 (e^{dt A} - 1)); a tiny
    nonzero A lands next to it."""
    p = _problem(4)
    p["A"][:, :2] = 0.0
    y0, h0 = _run_c(p, "zoh")
    q = dict(p)
    q["A"] = p["A"].copy()
    # the zero-A states of the ZOH scan equal those of the first-order scan
    _, hm = _run_c(p, "mamba")
    np.testing.assert_allclose(h0[:, :, :2], hm[:, :, :2], rtol=1e-15, atol=0)
    q["A"][:, :2] = -1e-12
    y1, h1 = _run_c(q, "zoh")
    np.testing.assert_allclose(h1, h0, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(y1, y0, rtol=1e-9, atol=1e-12)
    yn, hn = _run_np(p, "zoh")
    np.testing.assert_allclose(hn, h0, rtol=1e-13, atol=1e-14)


def test_zoh_keeps_precision_for_tiny_steps():
    """dt A of 1e-9: B_bar must still be dt B to 1e-9 relative (a naive exp(u) - 1 would
    lose half of the digits)."""
    p = _problem(5, L=3)
    p["delta"][:] = 1e-9
    p["h0"][:] = 0.0
    y, _ = _run_c(p, "zoh")
    ym, _ = _run_c(p, "mamba")
    np.testing.assert_allclose(y, ym, rtol=1e-8, atol=0)


@pytest.mark.parametrize("kind", ["zoh", "bilinear"])
def test_small_step_limit_is_first_order(kind):
    """All three discretisations agree to first order in dt: the gap to the Mamba scan,
    relative to the output, halves when dt halves."""
    p = _problem(6)
    p["h0"][:] = 0.0
    p["Dskip"][:] = 0.0     # so that the output itself is first order in dt
    gaps = []
    for s in (1e-2, 5e-3, 2.5e-3):
        q = dict(p)
        q["delta"] = p["delta"] * s
        y, _ = _run_c(q, kind)
        ym, _ = _run_c(q, "mamba")
        gaps.append(np.max(np.abs(y - ym)) / np.max(np.abs(ym)))
    r1, r2 = gaps[0] / gaps[1], gaps[1] / gaps[2]
    assert 1.7 < r1 < 2.3 and 1.7 < r2 < 2.3, gaps


@pytest.mark.parametrize("softplus", [False, True])
def test_delta_bias_goes_before_the_softplus(softplus):
    rng = np.random.default_rng(7)
    p = _problem(7, softplus=softplus, gate=True)
    bias = rng.normal(0.0, 0.3, p["x"].shape[2])
    for kind in KINDS:
        y, h = _run_c(p, kind, softplus, bias)
        q = dict(p)
        q["delta"] = p["delta"] + bias[None, None, :]
        yr, hr = _run_c(q, kind, softplus)
        np.testing.assert_allclose(y, yr, rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(h, hr, rtol=1e-14, atol=1e-15)
        yn, hn = _run_np(p, kind, softplus, bias)
        np.testing.assert_allclose(yn, y, rtol=1e-12, atol=1e-13)
    if softplus:
        # a bias added after the softplus is another function
        q = dict(p)
        q["delta"] = np.log1p(np.exp(p["delta"])) + bias[None, None, :]
        yw, _ = _run_c(q, "mamba", False)
        y, _ = _run_c(p, "mamba", True, bias)
        assert np.max(np.abs(yw - y)) > 1e-3


@pytest.mark.parametrize("kind", KINDS)
def test_c_and_numpy_agree(kind):
    p = _problem(8, Bsz=2, L=40, D=5, N=16, softplus=True, gate=True)
    bias = np.random.default_rng(8).normal(0.0, 0.2, 5)
    y, h = _run_c(p, kind, True, bias)
    yn, hn = _run_np(p, kind, True, bias)
    np.testing.assert_allclose(yn, y, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(hn, h, rtol=1e-11, atol=1e-12)


def test_storage_wrapper_passes_variant_keys():
    """oracle.scan reads "discretization" and "delta_bias" from the input dict."""
    rng = np.random.default_rng(9)
    B, L, D, N = 1, 6, 4, 3
    inp = {"dtype": "f32", "x": rng.standard_normal((B, L, D)).astype(np.float32),
           "delta": rng.uniform(0.01, 0.2, (B, L, D)).astype(np.float32),
           "z": None, "A": -np.arange(1, N + 1, dtype=np.float32)[None].repeat(D, 0),
           "B": rng.standard_normal((B, L, N)).astype(np.float32),
           "C": rng.standard_normal((B, L, N)).astype(np.float32), "Dskip": None,
           "discretization": "bilinear", "delta_bias": rng.normal(0, 0.1, D).astype(np.float32)}
    y, h = oracle.scan(inp)
    yr, hr = numpy_ref.scan_np(inp["x"], inp["delta"], inp["A"].astype(np.float64), inp["B"], inp["C"],
                               discretization="bilinear", delta_bias=inp["delta_bias"])
    np.testing.assert_allclose(y, yr, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(h, hr, rtol=1e-12, atol=1e-13)


# plausible mistakes planted in a copy of the numpy discretisation: each must fail a pin
_MUTANTS = {
    "zoh_times_A": ("np.expm1(u) / np.where(u == 0.0, 1.0, u)", "np.expm1(u) * np.where(u == 0.0, 1.0, u)"),
    "zoh_first_order_B": ("return a_bar, dt * phi", "return a_bar, np.broadcast_to(dt, a_bar.shape)"),
    "zoh_exp_without_minus_one": ("np.expm1(u) / np.where", "np.exp(u) / np.where"),
    "bilinear_inverted": ("return (1.0 + 0.5 * u) / den, dt / den", "return den / (1.0 + 0.5 * u), dt / den"),
    "bilinear_B_unscaled": ("return (1.0 + 0.5 * u) / den, dt / den", "return (1.0 + 0.5 * u) / den, dt + 0.0 * den"),
    "bilinear_full_step": ("den = 1.0 - 0.5 * u", "den = 1.0 - u"),
}


def _mutated(kind):
    src = inspect.getsource(numpy_ref._discretize_slab)
    old, new = _MUTANTS[kind]
    assert old in src, kind
    ns = dict(vars(numpy_ref))
    exec(src.replace(old, new), ns)
    scan_src = inspect.getsource(numpy_ref.scan_np)
    exec(scan_src, ns)
    return ns["scan_np"]


@pytest.mark.parametrize("kind", sorted(_MUTANTS))
def test_planted_discretisation_mistake_is_caught(kind):
    fn = _mutated(kind)
    disc = "zoh" if kind.startswith("zoh") else "bilinear"
    p = _problem(1)
    yr, _ = _run_scipy(p, disc)
    y, _ = _run_np(p, disc, fn=fn)
    assert np.max(np.abs(y - yr)) > 1e-6, f"mutant {kind} passes the pin"


def test_unmutated_copy_passes():
    ns = dict(vars(numpy_ref))
    exec(inspect.getsource(numpy_ref._discretize_slab), ns)
    exec(inspect.getsource(numpy_ref.scan_np), ns)
    p = _problem(1)
    for disc in ("zoh", "bilinear"):
        yr, _ = _run_scipy(p, disc)
        y, _ = _run_np(p, disc, fn=ns["scan_np"])
        np.testing.assert_allclose(y, yr, rtol=1e-11, atol=1e-12)
