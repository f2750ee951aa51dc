"""Pins of the backward (adjoint) oracle, against things other than itself.

* Central finite differences of the forward oracle (already pinned by
  tests/test_oracle_pins.py) for every input element of small problems: the
  adjoint must equal the derivative of the forward definition.
* The LTI special case: with constant step size, B and C, no gate and h0 = 0 the
  scan is a causal convolution y = K * x + D x, so dLoss/dx is the correlation of
  dLoss/dy with the same kernel K_k = sum_n C_n exp(dt A_n)^k dt B_n (brentwoodlivery
  "State-space models (Mamba, S4)", section "The Convolution View"), written out by
  brute force.
* Linearity in the incoming gradient, and the two fp64 implementations (C and
  numpy) agreeing.
"""
import numpy as np
import pytest

import oracle
from oracle.numpy_ref import scan_bwd_np, scan_np


def _problem(seed, Bsz=2, L=6, D=3, N=3, gate=True, h0=True, dskip=True, bias=False):
    r = np.random.default_rng(seed)
    p = {
        "x": r.standard_normal((Bsz, L, D)),
        "delta": np.exp(r.uniform(np.log(0.05), np.log(0.5), (Bsz, L, D))),
        "z": r.standard_normal((Bsz, L, D)) if gate else None,
        "B": r.standard_normal((Bsz, L, N)),
        "C": r.standard_normal((Bsz, L, N)),
        "A": -np.exp(r.standard_normal((D, N)) * 0.5),
        "D": r.standard_normal(D) if dskip else None,
        "h0": r.standard_normal((Bsz, D, N)) if h0 else None,
        "bias": r.normal(0.0, 0.3, D) if bias else None,
    }
    gy = r.standard_normal((Bsz, L, D))
    gl = r.standard_normal((Bsz, D, N))
    return p, gy, gl


def _loss(p, gy, gl, sp, disc="mamba"):
    y, h = scan_np(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["h0"], sp,
                   discretization=disc, delta_bias=p.get("bias"))
    return float((y * gy).sum() + (h * gl).sum())


def _c_bwd(p, gy, gl, sp, disc="mamba"):
    """Backward through the C oracle on float64 arrays (channels in (b, d) order)."""
    Bsz, L, D = p["x"].shape
    N = p["A"].shape[1]
    cb, cd = np.meshgrid(np.arange(Bsz), np.arange(D), indexing="ij")
    cb, cd = cb.reshape(-1), cd.reshape(-1)
    ser = lambda a: None if a is None else a[cb, :, cd]
    r = oracle.scan_bwd_f64(ser(p["x"]), ser(p["delta"]), p["A"], p["B"], p["C"], p["D"], ser(p["z"]),
                            None if p["h0"] is None else p["h0"][cb, cd, :], ser(gy),
                            gl[cb, cd, :], sp, cb, cd, nthreads=2, delta_bias=p.get("bias"),
                            discretization=disc)
    back = lambda a: a.reshape(Bsz, D, L).transpose(0, 2, 1)
    return {"x": back(r["dx"]), "delta": back(r["ddelta"]),
            "bias": None if p.get("bias") is None else back(r["ddelta"]).sum(axis=(0, 1)),
            "z": None if r["dz"] is None else back(r["dz"]),
            "B": r["dB_c"].reshape(Bsz, D, L, N).sum(axis=1),
            "C": r["dC_c"].reshape(Bsz, D, L, N).sum(axis=1),
            "A": r["dA_c"].reshape(Bsz, D, N).sum(axis=0),
            "D": r["dD_c"].reshape(Bsz, D).sum(axis=0),
            "h0": r["dh0"].reshape(Bsz, D, N)}


@pytest.mark.parametrize("seed,sp,gate,h0,dskip,bias", [
    (0, False, True, True, True, False), (1, True, True, True, True, False), (2, False, False, False, True, False),
    (3, True, False, True, False, False), (4, True, True, True, True, True), (5, False, True, False, True, True),
])
def test_adjoint_equals_finite_differences(seed, sp, gate, h0, dskip, bias):
    p, gy, gl = _problem(seed, gate=gate, h0=h0, dskip=dskip, bias=bias)
    if sp:
        p["delta"] = np.log(np.expm1(p["delta"]))      # raw input u, dt = softplus(u)
    g = _c_bwd(p, gy, gl, sp)
    worst = 0.0
    for name, arr in p.items():
        if arr is None:
            assert g[name] is None or name in ("D", "h0", "bias")
            continue
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            v = arr[idx]
            eps = 1e-6 * max(1.0, abs(v))
            arr[idx] = v + eps
            lp = _loss(p, gy, gl, sp)
            arr[idx] = v - eps
            lm = _loss(p, gy, gl, sp)
            arr[idx] = v
            fd = (lp - lm) / (2 * eps)
            err = abs(fd - g[name][idx]) / max(1.0, abs(fd))
            worst = max(worst, err)
            assert err < 1e-6, (name, idx, fd, g[name][idx])
    print(f"[pin] finite differences: worst {worst:.2e}")


def test_lti_input_gradient_is_kernel_correlation():
    r = np.random.default_rng(7)
    Bsz, L, D, N = 1, 40, 2, 4
    dt = np.array([0.3, 0.07])
    A = -np.exp(r.standard_normal((D, N)) * 0.5)
    Bv, Cv = r.standard_normal(N), r.standard_normal(N)
    Dk = r.standard_normal(D)
    p = {"x": r.standard_normal((Bsz, L, D)), "delta": np.broadcast_to(dt, (Bsz, L, D)).copy(),
         "z": None, "B": np.broadcast_to(Bv, (Bsz, L, N)).copy(), "C": np.broadcast_to(Cv, (Bsz, L, N)).copy(),
         "A": A, "D": Dk, "h0": None}
    gy = r.standard_normal((Bsz, L, D))
    g = _c_bwd(p, gy, np.zeros((Bsz, D, N)), False)
    for d in range(D):
        K = np.array([np.sum(Cv * np.exp(dt[d] * A[d]) ** k * dt[d] * Bv) for k in range(L)])
        want = np.array([sum(K[t - s] * gy[0, t, d] for t in range(s, L)) + Dk[d] * gy[0, s, d]
                         for s in range(L)])
        np.testing.assert_allclose(g["x"][0, :, d], want, rtol=1e-12, atol=1e-12)


def test_linear_in_incoming_gradient():
    p, gy, gl = _problem(11, L=20, D=4, N=5)
    _, gy2, gl2 = _problem(12, L=20, D=4, N=5)
    a, b = 0.7, -1.3
    g1, g2 = _c_bwd(p, gy, gl, False), _c_bwd(p, gy2, gl2, False)
    g12 = _c_bwd(p, a * gy + b * gy2, a * gl + b * gl2, False)
    for k in g12:
        if g12[k] is not None:
            np.testing.assert_allclose(g12[k], a * g1[k] + b * g2[k], rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("sp,bias,disc", [(False, False, "mamba"), (True, False, "mamba"), (True, True, "mamba"),
                                         (False, False, "zoh"), (True, True, "zoh"), (False, False, "bilinear"),
                                         (True, True, "bilinear")])
def test_c_and_numpy_backward_agree(sp, bias, disc):
    p, gy, gl = _problem(21, Bsz=3, L=50, D=6, N=7, bias=bias)
    # states whose dt A falls in the zero-order hold's series branch, and A = 0
    p["A"][0, 0] = 0.0
    p["A"][1, :3] = -1e-3
    if sp:
        p["delta"] = np.log(np.expm1(p["delta"]))
    g = _c_bwd(p, gy, gl, sp, disc)
    n = scan_bwd_np(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["h0"], sp, gy, gl,
                    delta_bias=p["bias"], discretization=disc)
    names = {"x": "dx", "delta": "ddelta", "z": "dz", "B": "dB", "C": "dC", "A": "dA", "D": "dD", "h0": "dh0"}
    if bias:
        names["bias"] = "ddelta_bias"
    for k, nk in names.items():
        np.testing.assert_allclose(g[k], n[nk], rtol=1e-11, atol=1e-11)


def test_storage_wrapper_matches_core():
    import synth
    inp = synth.scan_inputs(2, 33, 5, 16, "bf16", seed=5, gate=True, d_kind="normal", a_kind="random", h0=True,
                            softplus_input=True)
    inp["delta_bias"] = synth.make_delta_bias(5, 5)
    r = np.random.default_rng(3)
    gy = r.standard_normal((2, 33, 5))
    out = oracle.scan_bwd(inp, gy)
    w = lambda a: synth.to_f64(a, "bf16")
    n = scan_bwd_np(w(inp["x"]), w(inp["delta"]), inp["A"], w(inp["B"]), w(inp["C"]), inp["Dskip"],
                    w(inp["z"]), inp["h0"], True, gy, None, delta_bias=inp["delta_bias"])
    assert n["ddelta_bias"] is not None
    for k in n:
        np.testing.assert_allclose(out[k], n[k], rtol=1e-11, atol=1e-11)


# Planted mistakes in a copy of the numpy backward (or of its discretisation derivatives):
# each must fail the finite-difference pin of its discretisation.
_MUTANTS = {
    # kind: (function, old text, new text, discretisation)
    "silu_prime_dropped": ("scan_bwd_np", "sg * (1.0 + zz[:, t, :] * (1.0 - sg))", "sg", "mamba"),
    "readout_dropped": ("scan_bwd_np", "lam = lam + gy0[:, :, None] * Cm[:, t, None, :]", "lam = lam", "mamba"),
    "dA_without_dt": ("_discretize_grad_slab", "one, dt * e, np.zeros(u.shape)", "one, e, np.zeros(u.shape)",
                      "mamba"),
    "dx_without_the_factor": ("scan_bwd_np", "lam, fac * Bm[:, t, None, :])", "lam, Bm[:, t, None, :])", "mamba"),
    "ddelta_without_A": ("_discretize_grad_slab", "A[None] * e, one,", "e, one,", "mamba"),
    "dh0_not_decayed": ("scan_bwd_np", "        lam = a_bar * lam\n", "        lam = lam\n", "mamba"),
    "dB_with_wrong_input": ("scan_bwd_np", "g_bbar = lam * x[:, t, :, None]", "g_bbar = lam * hs[t]", "mamba"),
    "softplus_chain_dropped": ("scan_bwd_np", "g_dt / (1.0 + np.exp(-raw[:, t, :]))", "g_dt", "mamba"),
    "dC_with_old_state": ("scan_bwd_np", "gy0, hs[t + 1])", "gy0, hs[t])", "mamba"),
    "bias_ignored": ("scan_bwd_np", "raw = raw + np.asarray(delta_bias", "raw = raw + 0.0 * np.asarray(delta_bias",
                     "mamba"),
    "bias_gradient_of_one_row": ("scan_bwd_np", 'out["ddelta"].sum(axis=(0, 1))', 'out["ddelta"][0].sum(axis=0)',
                                 "mamba"),
    "zoh_dF_dA_dropped": ("_discretize_grad_slab", "dt * e, dt * dt * psi", "dt * e, 0.0 * psi", "zoh"),
    "zoh_dF_ddt_as_mamba": ("_discretize_grad_slab", "A[None] * e, e, dt * e", "A[None] * e, 1.0 + 0.0 * e, dt * e",
                            "zoh"),
    "zoh_psi_sign": ("_discretize_grad_slab", "(us * np.exp(us) - np.expm1(us))", "(us * np.exp(us) + np.expm1(us))",
                     "zoh"),
    "bilinear_r_not_squared": ("_discretize_grad_slab", "r2 = r * r", "r2 = r", "bilinear"),
    "bilinear_dF_dA_halved_twice": ("_discretize_grad_slab", "r2 * dt * dt / 2.0)", "r2 * dt * dt / 4.0)", "bilinear"),
}


def _mutated_bwd(kind):
    import inspect
    from oracle import numpy_ref
    fname, old, new, _ = _MUTANTS[kind]
    src = inspect.getsource(getattr(numpy_ref, fname))
    assert src.count(old) == 1, kind
    ns = dict(vars(numpy_ref))
    exec(src.replace(old, new), ns)
    if fname != "scan_bwd_np":   # re-bind the backward to the mutated helper
        exec(inspect.getsource(numpy_ref.scan_bwd_np), ns)
    return ns["scan_bwd_np"]


def _fd_worst(fn, seed, sp, disc="mamba"):
    # the softplus case also carries a delta bias
    p, gy, gl = _problem(seed, bias=sp)
    if sp:
        p["delta"] = np.log(np.expm1(p["delta"]))
    g = fn(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["h0"], sp, gy, gl,
           delta_bias=p["bias"], discretization=disc)
    names = {"x": "dx", "delta": "ddelta", "z": "dz", "B": "dB", "C": "dC", "A": "dA", "D": "dD", "h0": "dh0",
             "bias": "ddelta_bias"}
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
            lp = _loss(p, gy, gl, sp, disc)
            arr[idx] = v - eps
            lm = _loss(p, gy, gl, sp, disc)
            arr[idx] = v
            fd = (lp - lm) / (2 * eps)
            worst = max(worst, abs(fd - g[names[name]][idx]) / max(1.0, abs(fd)))
    return worst


@pytest.mark.parametrize("kind", sorted(_MUTANTS))
def test_planted_backward_mistake_is_caught(kind):
    fn = _mutated_bwd(kind)
    disc = _MUTANTS[kind][3]
    assert max(_fd_worst(fn, 30, False, disc), _fd_worst(fn, 31, True, disc)) > 1e-3, f"mutant {kind} passes the pin"


@pytest.mark.parametrize("disc", ["mamba", "zoh", "bilinear"])
def test_unmutated_backward_copy_passes(disc):
    assert max(_fd_worst(scan_bwd_np, 30, False, disc), _fd_worst(scan_bwd_np, 31, True, disc)) < 1e-6


def test_zoh_backward_through_tiny_and_zero_steps_times_A():
    """The zero-order hold's series branch (|dt A| < 1e-2, and A = 0 exactly) against
    finite differences of the forward oracle."""
    p, gy, gl = _problem(33)
    p["A"][:, 0] = 0.0
    p["A"][:, 1] = -1e-4
    p["delta"][0, :2] = 1e-3
    g = scan_bwd_np(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["h0"], False, gy, gl,
                    discretization="zoh")
    for (d, n) in ((0, 0), (1, 1), (2, 0), (0, 2)):
        eps = 1e-6
        v = p["A"][d, n]
        p["A"][d, n] = v + eps
        lp = _loss(p, gy, gl, False, "zoh")
        p["A"][d, n] = v - eps
        lm = _loss(p, gy, gl, False, "zoh")
        p["A"][d, n] = v
        fd = (lp - lm) / (2 * eps)
        assert abs(fd - g["dA"][d, n]) <= 1e-6 * max(1.0, abs(fd)), (d, n, fd, g["dA"][d, n])
