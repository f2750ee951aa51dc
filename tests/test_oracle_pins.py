"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import math

import numpy as np
import pytest

import oracle
import synth
from oracle.numpy_ref import scan_np
from tests import oracle_pins as P

ORACLES = {"c": P.c_oracle_scan, "numpy": P.numpy_oracle_scan}


@pytest.mark.parametrize("pin", sorted(P.PINS))
@pytest.mark.parametrize("impl", sorted(ORACLES))
def test_pin(impl, pin):
    fn, tol = P.PINS[pin]
    err = fn(ORACLES[impl])
    assert err <= tol, f"{impl} oracle fails pin {pin}: err {err:.3e} > {tol:.1e}"


@pytest.mark.parametrize("seed,N,gate,h0,sp", [
    (1, 1, False, False, False), (2, 2, True, False, False), (3, 3, False, True, False),
    (4, 5, True, True, True), (5, 16, True, True, False), (6, 16, False, False, True),
])
def test_two_oracles_agree(seed, N, gate, h0, sp):
    p = P._rand_problem(seed, Bsz=3, L=37, D=6, N=N, gate=gate, h0=h0)
    if sp:
        p["delta"] = np.log(np.expm1(p["delta"]))
    yc, hc = P._call(P.c_oracle_scan, p, delta_softplus=sp)
    yn, hn = P._call(P.numpy_oracle_scan, p, delta_softplus=sp)
    assert P._relerr(yc, yn) < 1e-13 and P._relerr(hc, hn) < 1e-13


def test_storage_wrappers_match_core():
    """oracle.scan on storage-form (bf16) inputs equals the numpy oracle on the widened values."""
    inp = synth.scan_inputs(2, 50, 7, 16, "bf16", seed=3, gate=True, d_kind="normal",
                            a_kind="random", h0=True)
    y, h = oracle.scan(inp)
    w = lambda a: synth.to_f64(a, "bf16")
    yn, hn = scan_np(w(inp["x"]), w(inp["delta"]), inp["A"].astype(np.float64), w(inp["B"]),
                     w(inp["C"]), inp["Dskip"].astype(np.float64), w(inp["z"]),
                     inp["h0"].astype(np.float64))
    assert P._relerr(y, yn) < 1e-13 and P._relerr(h, hn) < 1e-13
    # sampled channels give the same numbers as the full run
    ch = [(1, 3), (0, 0), (1, 6)]
    ys, hs = oracle.scan(inp, channels=ch)
    for i, (b, d) in enumerate(ch):
        assert np.array_equal(ys[i], y[b, :, d]) and np.array_equal(hs[i], h[b, d])


def test_state_update_steps_equal_scan():
    """L single-token updates reproduce one scan (state caching across steps)."""
    Bsz, L, D, N = 2, 12, 5, 4
    inp = synth.scan_inputs(Bsz, L, D, N, "bf16", seed=8, gate=True, d_kind="normal", h0=True)
    y, h = oracle.scan(inp)
    hs = inp["h0"].astype(np.float64)
    for t in range(L):
        step = {k: inp[k][:, t] for k in ("x", "delta", "z", "B", "C")}
        hs, yt = oracle.state_update(hs, step, inp["A"], inp["Dskip"], "bf16")
        assert np.allclose(yt, y[:, t, :], rtol=0, atol=1e-13)
    assert np.allclose(hs, h, rtol=0, atol=1e-13)


def test_empty_and_degenerate_shapes():
    for (Bsz, L, D, N) in [(1, 0, 3, 2), (0, 5, 3, 2), (2, 4, 0, 3), (1, 1, 1, 1)]:
        p = P._rand_problem(0, Bsz=Bsz, L=L, D=D, N=N, h0=True)
        yc, hc = P._call(P.c_oracle_scan, p)
        yn, hn = P._call(P.numpy_oracle_scan, p)
        assert yc.shape == (Bsz, L, D) and hc.shape == (Bsz, D, N)
        assert np.array_equal(yc, yn) or P._relerr(yc, yn) < 1e-14
        if L == 0:
            assert np.array_equal(hc, p["h0"])


# --- planted mistakes: every plausible error in the oracle must trip a pin ---

def _mutant(kind):
    def silu(v):
        return v / (1.0 + np.exp(-v))

    def scan(x, delta, A, Bm, Cm, Dskip=None, z=None, h0=None, delta_softplus=False):
        Bsz, L, D = x.shape
        N = A.shape[1]
        dl = np.logaddexp(0.0, delta) if (delta_softplus and kind != "no_softplus") else delta
        h = np.zeros((Bsz, D, N)) if (h0 is None or kind == "ignore_h0") else np.array(h0, dtype=float)
        y = np.empty((Bsz, L, D))
        Ad = np.broadcast_to(A[0:1], A.shape) if kind == "shared_A" else A
        for t in range(L):
            dt = dl[:, t, :, None]
            sgn = -1.0 if kind == "exp_sign" else 1.0
            a_bar = np.exp(sgn * dt * Ad[None])
            tb = max(t - 1, 0) if kind == "B_shift" else t
            b_bar = (1.0 if kind == "no_delta_B" else dt) * Bm[:, tb, None, :]
            h_new = a_bar * h + b_bar * x[:, t, :, None]
            tc = min(t + 1, L - 1) if kind == "C_shift" else t
            hr = h if kind == "read_before_update" else h_new
            yt = np.einsum("bdn,bn->bd", hr, Cm[:, tc, :])
            h = h_new
            dx = 0.0 if (Dskip is None or kind == "drop_D") else Dskip[None, :] * x[:, t, :]
            if z is not None:
                g = z[:, t, :]
                gate = 1.0 / (1.0 + np.exp(-g)) if kind == "sigmoid_gate" else silu(g)
                yt = yt * gate + dx if kind == "gate_before_D" else (yt + dx) * gate
            else:
                yt = yt + dx
            y[:, t, :] = yt
        return y, h
    return scan


MUTANTS = ["drop_D", "read_before_update", "exp_sign", "no_delta_B", "B_shift", "C_shift",
           "gate_before_D", "sigmoid_gate", "no_softplus", "shared_A", "ignore_h0"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    fn = _mutant(kind)
    failed = [name for name, (pin, tol) in P.PINS.items() if not (pin(fn) <= tol)]
    assert failed, f"mutant {kind} passes every pin"


def test_unmutated_copy_passes():
    fn = _mutant("none")
    for name, (pin, tol) in P.PINS.items():
        assert pin(fn) <= tol, name
