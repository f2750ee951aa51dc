"""Pins of the multi-head SSD (Mamba-2 layer) oracle, ``oracle/ssd_oracle.py``.

None of them restates the oracle's loop:

* the S6 oracle in C (pinned on its own by the worked example, the convolution view,
  brute-force unrolling, ...) run on the H * P channels with A[d, n] = a_h for every
  state and the head's step size broadcast over its channels;
* the structured-matrix ("dual", attention-like) form the brentwoodlivery page names:
  y = M x with M[t, s] = (C_t . B_s) exp(a (cum_t - cum_s)) dt_s for s <= t, built as a
  dense matrix by brute force;
* a = 0: the state is the running sum of dt_s x_s B_s^T, a closed form;
* splitting the sequence and carrying the state; heads are independent of each other;
* planted mistakes in a copy of the oracle each fail one of the above.
"""
from __future__ import annotations

import inspect

import numpy as np
import pytest

import oracle
import synth
from oracle import ssd_oracle


def _problem(seed, Bsz=2, L=20, H=3, P=4, N=5, gate=False, softplus=False, bias=False, h0=True):
    rng = np.random.default_rng(seed)
    p = {
        "x": rng.standard_normal((Bsz, L, H, P)),
        "delta": np.exp(rng.uniform(np.log(1e-3), np.log(0.5), (Bsz, L, H))),
        "a": -np.exp(rng.uniform(0.0, np.log(16.0), H)),
        "Bm": rng.standard_normal((Bsz, L, N)),
        "Cm": rng.standard_normal((Bsz, L, N)),
        "D": rng.normal(1.0, 0.1, H),
        "z": rng.standard_normal((Bsz, L, H, P)) if gate else None,
        "h0": rng.standard_normal((Bsz, H, P, N)) if h0 else None,
        "bias": rng.normal(0.0, 0.3, H) if bias else None,
    }
    if softplus:
        p["delta"] = np.log(np.expm1(p["delta"]))
    return p


def _run(p, fn=None, softplus=False):
    fn = fn or ssd_oracle.ssd
    return fn(p["x"], p["delta"], p["a"], p["Bm"], p["Cm"], p["D"], p["z"], p["h0"], softplus, p["bias"])


def _via_s6(p, softplus=False):
    """The S6 C oracle on channels d = h * P + p."""
    x, dl, a = p["x"], p["delta"], p["a"]
    Bsz, L, H, P = x.shape
    N = p["Bm"].shape[2]
    D = H * P
    xs = x.reshape(Bsz, L, D)
    ds = np.repeat(dl, P, axis=2)
    A = np.repeat(a, P)[:, None] * np.ones((1, N))
    Dk = np.repeat(p["D"], P)
    zs = None if p["z"] is None else p["z"].reshape(Bsz, L, D)
    bias = None if p["bias"] is None else np.repeat(p["bias"], P)
    h0 = None if p["h0"] is None else p["h0"].reshape(Bsz, D, N)
    cb, cd = np.meshgrid(np.arange(Bsz), np.arange(D), indexing="ij")
    cb, cd = cb.reshape(-1), cd.reshape(-1)
    ser = lambda t: None if t is None else t[cb, :, cd]
    y, hl = oracle.scan_f64(ser(xs), ser(ds), A, p["Bm"], p["Cm"], Dk, ser(zs),
                            None if h0 is None else h0[cb, cd, :], softplus, cb, cd, 1, "mamba", bias)
    return (y.reshape(Bsz, D, L).transpose(0, 2, 1).reshape(Bsz, L, H, P),
            hl.reshape(Bsz, H, P, N))


def _dual(p):
    """y = M x with M[t, s] = (C_t . B_s) exp(a (cum_t - cum_s)) dt_s (s <= t), plus the
    start state's share exp(a cum_t) C_t . H0[p, :] and D x.  No gate, no softplus."""
    x, dl, a, Bm, Cm = p["x"], p["delta"], p["a"], p["Bm"], p["Cm"]
    Bsz, L, H, P = x.shape
    y = np.zeros((Bsz, L, H, P))
    for b in range(Bsz):
        CB = Cm[b] @ Bm[b].T                                          # [L, L]
        for h in range(H):
            cum = np.cumsum(dl[b, :, h])
            M = np.zeros((L, L))
            for t in range(L):
                for s in range(t + 1):
                    M[t, s] = CB[t, s] * np.exp(a[h] * (cum[t] - cum[s])) * dl[b, s, h]
            y[b, :, h, :] = M @ x[b, :, h, :]
            if p["h0"] is not None:
                y[b, :, h, :] += np.exp(a[h] * cum)[:, None] * (Cm[b] @ p["h0"][b, h].T)
            y[b, :, h, :] += p["D"][h] * x[b, :, h, :]
    return y


@pytest.mark.parametrize("gate,softplus,bias", [(False, False, False), (True, False, False),
                                                (True, True, True), (False, True, False)])
def test_equals_s6_with_a_scalar_decay_per_head(gate, softplus, bias):
    p = _problem(1, gate=gate, softplus=softplus, bias=bias)
    y, h = _run(p, softplus=softplus)
    yr, hr = _via_s6(p, softplus)
    np.testing.assert_allclose(y, yr, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(h, hr, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("h0", [False, True])
def test_structured_matrix_form(h0):
    p = _problem(2, L=24, h0=h0)
    y, _ = _run(p)
    np.testing.assert_allclose(y, _dual(p), rtol=1e-11, atol=1e-12)


def test_no_decay_is_a_running_sum():
    p = _problem(3)
    p["a"][:] = 0.0
    y, h = _run(p)
    x, dl, Bm, Cm = p["x"], p["delta"], p["Bm"], p["Cm"]
    drive = np.einsum("blh,blhp,bln->blhpn", dl, x, Bm)
    states = p["h0"][:, None] + np.cumsum(drive, axis=1)              # [B, L, H, P, N]
    yr = np.einsum("blhpn,bln->blhp", states, Cm) + p["D"][None, None, :, None] * x
    np.testing.assert_allclose(y, yr, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(h, states[:, -1], rtol=1e-12, atol=1e-12)


def test_split_and_carry():
    p = _problem(4, L=30, gate=True)
    y, h = _run(p)
    T = 13
    first = {k: (v[:, :T] if k in ("x", "delta", "Bm", "Cm", "z") and v is not None else v) for k, v in p.items()}
    second = {k: (v[:, T:] if k in ("x", "delta", "Bm", "Cm", "z") and v is not None else v) for k, v in p.items()}
    y1, h1 = _run(first)
    second["h0"] = h1
    y2, h2 = _run(second)
    np.testing.assert_array_equal(np.concatenate([y1, y2], axis=1), y)
    np.testing.assert_array_equal(h2, h)


def test_heads_are_independent():
    p = _problem(5, H=4)
    y, h = _run(p)
    perm = np.array([2, 0, 3, 1])
    q = dict(p)
    q["x"], q["delta"], q["a"], q["D"] = p["x"][:, :, perm], p["delta"][:, :, perm], p["a"][perm], p["D"][perm]
    q["h0"] = p["h0"][:, perm]
    yq, hq = _run(q)
    np.testing.assert_allclose(yq, y[:, :, perm], rtol=1e-14, atol=0)
    np.testing.assert_allclose(hq, h[:, perm], rtol=1e-14, atol=0)


def test_storage_wrapper():
    inp = synth.ssd_inputs(2, 9, 3, 4, 5, "bf16", seed=6, gate=True, softplus_input=True, h0=True,
                           delta_bias=True)
    y, h = ssd_oracle.ssd_storage(inp)
    w = lambda t: synth.to_f64(t, "bf16")
    yr, hr = ssd_oracle.ssd(w(inp["x"]), w(inp["delta"]), inp["A"], w(inp["B"]), w(inp["C"]), inp["Dskip"],
                            w(inp["z"]), inp["h0"], True, inp["delta_bias"])
    np.testing.assert_array_equal(y, yr)
    ys, hs = ssd_oracle.ssd_storage(inp, batches=[1], heads=[2, 0])
    np.testing.assert_array_equal(ys, y[[1]][:, :, [2, 0]])
    np.testing.assert_array_equal(hs, h[[1]][:, [2, 0]])


_MUTANTS = {
    "b_bar_without_dt": ("drive = (step[:, :, None] * x[:, t, :, :])", "drive = (x[:, t, :, :])"),
    "decay_without_dt": ("decay = np.exp(step * a[None, :])", "decay = np.exp(a[None, :] + 0.0 * step)"),
    "readout_before_update": ("state = decay * state + drive                                 # [B, H, P, N]\n        yt = np.einsum(\"bhpn,bn->bhp\", state, Cm[:, t, :])",
                              "yt = np.einsum(\"bhpn,bn->bhp\", state, Cm[:, t, :])\n        state = decay * state + drive"),
    "step_of_head_zero": ("step = dt[:, t, :]  ", "step = np.repeat(dt[:, t, :1], dt.shape[2], axis=1)  "),
    "skip_dropped": ("yt = yt + np.asarray(D, dtype=np.float64)[None, :, None] * x[:, t, :, :]", "yt = yt"),
    "gate_sigmoid": ("yt = yt * _silu(", "yt = yt * (lambda v: 1.0 / (1.0 + np.exp(-v)))("),
}


def _mutated(kind):
    src = inspect.getsource(ssd_oracle.ssd)
    old, new = _MUTANTS[kind]
    assert old in src, kind
    ns = dict(vars(ssd_oracle))
    exec(src.replace(old, new), ns)
    return ns["ssd"]


@pytest.mark.parametrize("kind", sorted(_MUTANTS))
def test_planted_mistake_is_caught(kind):
    fn = _mutated(kind)
    p = _problem(7, gate=True)
    y, _ = _run(p, fn=fn)
    yr, _ = _via_s6(p)
    assert np.max(np.abs(y - yr)) > 1e-6, f"mutant {kind} passes the pin"


def test_unmutated_copy_passes():
    ns = dict(vars(ssd_oracle))
    exec(inspect.getsource(ssd_oracle.ssd), ns)
    p = _problem(7, gate=True)
    y, _ = _run(p, fn=ns["ssd"])
    yr, _ = _via_s6(p)
    np.testing.assert_allclose(y, yr, rtol=1e-12, atol=1e-13)


def _grouped(seed, G, HG, **kw):
    """A problem with G groups of HG heads: B, C [B, L, G, N]."""
    p = _problem(seed, H=G * HG, **kw)
    rng = np.random.default_rng(seed + 1000)
    Bsz, L, N = p["Bm"].shape
    p["Bm"] = rng.standard_normal((Bsz, L, G, N))
    p["Cm"] = rng.standard_normal((Bsz, L, G, N))
    return p


def _group_slice(p, g, HG):
    hs = slice(g * HG, (g + 1) * HG)
    q = dict(p)
    q["x"], q["delta"], q["a"], q["D"] = p["x"][:, :, hs], p["delta"][:, :, hs], p["a"][hs], p["D"][hs]
    q["z"] = None if p["z"] is None else p["z"][:, :, hs]
    q["h0"] = None if p["h0"] is None else p["h0"][:, hs]
    q["bias"] = None if p["bias"] is None else p["bias"][hs]
    q["Bm"], q["Cm"] = p["Bm"][:, :, g], p["Cm"][:, :, g]
    return q


@pytest.mark.parametrize("G,HG,gate", [(2, 2, False), (3, 1, True), (2, 3, True)])
def test_groups_equal_s6_per_group(G, HG, gate):
    """B/C groups: the heads of group g, run through the S6 C oracle with group g's B and C
    rows, give the grouped oracle's outputs for those heads."""
    p = _grouped(11, G, HG, gate=gate)
    y, h = _run(p)
    for g in range(G):
        yr, hr = _via_s6(_group_slice(p, g, HG))
        hs = slice(g * HG, (g + 1) * HG)
        np.testing.assert_allclose(y[:, :, hs], yr, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(h[:, hs], hr, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("old,new", [("Bm[:, :, g], np.asarray(Cm)[:, :, g]", "Bm[:, :, G - 1 - g], np.asarray(Cm)[:, :, g]"),
                                     ("sel = slice(g * hg, (g + 1) * hg)", "sel = slice(0, hg)")])
def test_planted_group_mistake_is_caught(old, new):
    src = inspect.getsource(ssd_oracle.ssd)
    assert old in src
    ns = dict(vars(ssd_oracle))
    exec(src.replace(old, new), ns)
    p = _grouped(12, 2, 2)
    y, _ = _run(p, fn=ns["ssd"])
    yr, _ = _via_s6(_group_slice(p, 1, 2))
    assert np.max(np.abs(y[:, :, 2:4] - yr)) > 1e-6


# ---- the backward (ssd_oracle.ssd_bwd)

def _ssd_loss(p, gy, gl, softplus):
    y, hl = _run(p, softplus=softplus)
    return float((y * gy).sum() + (0.0 if gl is None else (hl * gl).sum()))


def _ssd_bwd_fd_worst(fn, seed, softplus, gate, h0, bias):
    """Largest gap between fn's gradients and central finite differences of the forward
    oracle, element by element over every input (tiny problem)."""
    p = _problem(seed, Bsz=2, L=6, H=2, P=3, N=4, gate=gate, softplus=softplus, bias=bias, h0=h0)
    if bias and not softplus:   # a positive step size (a negative one grows the state without bound)
        p["bias"] = 0.05 * np.abs(p["bias"])
    rng = np.random.default_rng(seed + 7)
    gy = rng.standard_normal(p["x"].shape)
    gl = rng.standard_normal((2, 2, 3, 4))
    g = fn(p["x"], p["delta"], p["a"], p["Bm"], p["Cm"], p["D"], p["z"], p["h0"], softplus, p["bias"], gy, gl)
    names = {"x": "dx", "delta": "ddelta", "a": "dA", "Bm": "dB", "Cm": "dC", "D": "dD", "z": "dz", "h0": "dh0",
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
            lp = _ssd_loss(p, gy, gl, softplus)
            arr[idx] = v - eps
            lm = _ssd_loss(p, gy, gl, softplus)
            arr[idx] = v
            fd = (lp - lm) / (2 * eps)
            worst = max(worst, abs(fd - g[names[name]][idx]) / max(1.0, abs(fd)))
    return worst


@pytest.mark.parametrize("seed,softplus,gate,h0,bias", [(40, False, True, True, False), (41, True, True, False, True),
                                                        (42, False, False, True, True), (43, True, False, False, False)])
def test_ssd_backward_equals_finite_differences(seed, softplus, gate, h0, bias):
    """Every gradient of the SSD backward oracle against central differences of the SSD
    forward oracle (pinned above on its own), element by element."""
    assert _ssd_bwd_fd_worst(ssd_oracle.ssd_bwd, seed, softplus, gate, h0, bias) < 1e-6


def test_ssd_backward_is_the_s6_backward_of_the_expansion():
    """The SSD layer is the S6 scan on the H * P channels with the head's step size, decay and
    D tied over its channels; so its gradients are the S6 oracle's (numpy, pinned on its own
    by finite differences) on that expansion, summed over each head's channels."""
    from oracle.numpy_ref import scan_bwd_np
    p = _problem(44, Bsz=2, L=9, H=3, P=4, N=5, gate=True, softplus=True, bias=True, h0=True)
    rng = np.random.default_rng(45)
    gy = rng.standard_normal(p["x"].shape)
    gl = rng.standard_normal((2, 3, 4, 5))
    g = ssd_oracle.ssd_bwd(p["x"], p["delta"], p["a"], p["Bm"], p["Cm"], p["D"], p["z"], p["h0"], True, p["bias"],
                           gy, gl)
    Bsz, L, H, P = p["x"].shape
    N, D = 5, H * P
    r = scan_bwd_np(p["x"].reshape(Bsz, L, D), np.repeat(p["delta"], P, axis=2),
                    np.repeat(p["a"], P)[:, None] * np.ones((1, N)), p["Bm"], p["Cm"], np.repeat(p["D"], P),
                    p["z"].reshape(Bsz, L, D), p["h0"].reshape(Bsz, D, N), True, gy.reshape(Bsz, L, D),
                    gl.reshape(Bsz, D, N), delta_bias=np.repeat(p["bias"], P))
    np.testing.assert_allclose(g["dx"], r["dx"].reshape(Bsz, L, H, P), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dz"], r["dz"].reshape(Bsz, L, H, P), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["ddelta"], r["ddelta"].reshape(Bsz, L, H, P).sum(axis=3), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dA"], r["dA"].reshape(H, P * N).sum(axis=1), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dB"], r["dB"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dC"], r["dC"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dD"], r["dD"].reshape(H, P).sum(axis=1), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dh0"], r["dh0"].reshape(Bsz, H, P, N), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["ddelta_bias"], r["ddelta_bias"].reshape(H, P).sum(axis=1), rtol=1e-10, atol=1e-12)


# planted mistakes in a copy of ssd_bwd: each must fail the finite-difference pin
_SSD_BWD_MUTANTS = {
    "readout_dropped": ("lam = lam + g[:, :, :, None] * Cm[:, t, None, None, :]", "lam = lam"),
    "decay_term_of_dt_dropped": ("a[None, :] * ab * hprev + np.einsum", "0.0 * hprev + np.einsum"),
    "dA_without_dt": ("np.einsum(\"bh,bh->h\", st * ab, hprev)", "np.einsum(\"bh,bh->h\", ab, hprev)"),
    "dC_with_old_state": ("dC[:, t] += np.einsum(\"bhp,bhpn->bn\", g, states[t + 1])",
                          "dC[:, t] += np.einsum(\"bhp,bhpn->bn\", g, states[t])"),
    "dh0_not_decayed": ("        lam = ab[:, :, None, None] * lam\n", "        lam = lam\n"),
    "softplus_chain_dropped": ("draw = ddt * (1.0 / (1.0 + np.exp(-raw))) if delta_softplus else ddt", "draw = ddt"),
    "silu_prime_dropped": ("dz = gy * y0 * sg * (1.0 + zz * (1.0 - sg))", "dz = gy * y0 * sg"),
}


def _mutated_ssd_bwd(kind):
    old, new = _SSD_BWD_MUTANTS[kind]
    src = inspect.getsource(ssd_oracle.ssd_bwd)
    assert src.count(old) == 1, kind
    ns = dict(vars(ssd_oracle))
    exec(src.replace(old, new), ns)
    return ns["ssd_bwd"]


@pytest.mark.parametrize("kind", sorted(_SSD_BWD_MUTANTS))
def test_planted_ssd_backward_mistake_is_caught(kind):
    fn = _mutated_ssd_bwd(kind)
    worst = max(_ssd_bwd_fd_worst(fn, 40, False, True, True, False), _ssd_bwd_fd_worst(fn, 41, True, True, True, True))
    assert worst > 1e-3, f"mutant {kind} passes the pin"


def test_unmutated_ssd_backward_copy_passes():
    ns = dict(vars(ssd_oracle))
    exec(inspect.getsource(ssd_oracle.ssd_bwd), ns)
    assert _ssd_bwd_fd_worst(ns["ssd_bwd"], 41, True, True, True, True) < 1e-6
