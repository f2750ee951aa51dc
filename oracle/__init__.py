"""fp64 CPU oracle of the Mamba (S6) selective scan and its single-token state update.

TEST INFRASTRUCTURE ONLY.  The product path (the HIP library and its Python
binding) never imports, loads or calls anything in this package; only the
tests, the package's smoke check and the bench's CPU-baseline leg do.  The
oracle shares no code with the GPU path.

Two independent implementations live here:

* ``ssm_oracle.c`` -- plain C, double precision, threads over independent
  channels (built into ``liboracle_ssm.so`` by ``build()``);
* ``numpy_ref.py`` -- a vectorised numpy float64 version written separately,
  used to cross-check the C one on small shapes.

Both compute the definition written out at the top of ``ssm_oracle.c``.
Inputs arrive in storage form (bf16 bit patterns or float32, as produced by
the ``synth`` module) and are widened to float64 exactly before use.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_ssm.so")
_lib = None


def build() -> str:
    """Compile the C oracle (plain gcc, no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-o", _LIB_PATH + ".tmp", _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_scan.argtypes = [I64, I64, I64, P, P, P, P, P, ctypes.c_int, ctypes.c_int, P,
                                P, P, P, P, P, P, P, ctypes.c_int]
    lib.oracle_scan.restype = ctypes.c_int
    lib.oracle_scan_bwd.argtypes = [I64, I64, I64, P, P, P, P, P, ctypes.c_int, ctypes.c_int, P, P, P, P, P, P, P,
                                    P, P, P, P, P, P, P, P, P, ctypes.c_int]
    lib.oracle_scan_bwd.restype = ctypes.c_int
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


DISCRETIZATIONS = {"mamba": 0, "zoh": 1, "bilinear": 2}


def scan_f64(x, delta, A, Bm, Cm, Dskip=None, z=None, h0=None, delta_softplus=False,
             ch_b=None, ch_d=None, nthreads=None, discretization="mamba", delta_bias=None):
    """Core call on float64 arrays.

    x, delta, z : [nchan, L] series of the listed channels (b = ch_b[i], d = ch_d[i])
    Bm, Cm      : [nb, L, N];  A: [nd, N];  Dskip: [nd] or None;  h0: [nchan, N] or None
    discretization: "mamba", "zoh" or "bilinear";  delta_bias: [nd] or None
    Returns (y [nchan, L], h_last [nchan, N]).
    """
    lib = _load()
    disc = DISCRETIZATIONS[discretization]
    dbias = _f64(delta_bias)
    x, delta, z = _f64(x), _f64(delta), _f64(z)
    Bm, Cm, A, Dskip, h0 = _f64(Bm), _f64(Cm), _f64(A), _f64(Dskip), _f64(h0)
    nchan, L = x.shape
    N = A.shape[1]
    assert delta.shape == x.shape and (z is None or z.shape == x.shape)
    assert Bm.shape[1:] == (L, N) and Cm.shape == Bm.shape
    ch_b = np.ascontiguousarray(ch_b, dtype=np.int64)
    ch_d = np.ascontiguousarray(ch_d, dtype=np.int64)
    assert ch_b.shape == (nchan,) and ch_d.shape == (nchan,)
    if nchan:
        assert ch_b.min() >= 0 and ch_b.max() < Bm.shape[0]
        assert ch_d.min() >= 0 and ch_d.max() < A.shape[0]
    if h0 is not None:
        assert h0.shape == (nchan, N)
    y = np.empty((nchan, L), dtype=np.float64)
    h_last = np.empty((nchan, N), dtype=np.float64)
    if dbias is not None:
        assert dbias.shape == (A.shape[0],)
    rc = lib.oracle_scan(L, N, nchan, _ptr(ch_b), _ptr(ch_d), _ptr(x), _ptr(delta), _ptr(z),
                         int(bool(delta_softplus)), disc, _ptr(dbias),
                         _ptr(Bm), _ptr(Cm), _ptr(A), _ptr(Dskip),
                         _ptr(h0), _ptr(y), _ptr(h_last),
                         int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_scan rejected its arguments")
    return y, h_last


def scan_bwd_f64(x, delta, A, Bm, Cm, Dskip, z, h0, gy, g_last, delta_softplus, ch_b, ch_d,
                 nthreads=None, delta_bias=None, discretization="mamba"):
    """Core backward call on float64 arrays (layouts as ``scan_f64``; gy [nchan, L],
    g_last [nchan, N] or None).  Returns a dict of per-channel results: dx, ddelta, dz
    [nchan, L] (dz None without a gate), dB_c, dC_c [nchan, L, N], dA_c, dh0 [nchan, N],
    dD_c [nchan]."""
    lib = _load()
    disc = DISCRETIZATIONS[discretization]
    x, delta, z, gy = _f64(x), _f64(delta), _f64(z), _f64(gy)
    Bm, Cm, A, Dskip, h0, g_last = _f64(Bm), _f64(Cm), _f64(A), _f64(Dskip), _f64(h0), _f64(g_last)
    dbias = _f64(delta_bias)
    nchan, L = x.shape
    N = A.shape[1]
    assert delta.shape == x.shape and gy.shape == x.shape and (z is None or z.shape == x.shape)
    ch_b = np.ascontiguousarray(ch_b, dtype=np.int64)
    ch_d = np.ascontiguousarray(ch_d, dtype=np.int64)
    out = {"dx": np.empty((nchan, L)), "ddelta": np.empty((nchan, L)),
           "dz": np.empty((nchan, L)) if z is not None else None,
           "dB_c": np.empty((nchan, L, N)), "dC_c": np.empty((nchan, L, N)),
           "dA_c": np.empty((nchan, N)), "dD_c": np.empty(nchan), "dh0": np.empty((nchan, N))}
    rc = lib.oracle_scan_bwd(L, N, nchan, _ptr(ch_b), _ptr(ch_d), _ptr(x), _ptr(delta), _ptr(z),
                             int(bool(delta_softplus)), disc, _ptr(dbias), _ptr(Bm), _ptr(Cm), _ptr(A), _ptr(Dskip),
                             _ptr(h0), _ptr(gy), _ptr(g_last), _ptr(out["dx"]), _ptr(out["ddelta"]),
                             _ptr(out["dz"]), _ptr(out["dB_c"]), _ptr(out["dC_c"]), _ptr(out["dA_c"]),
                             _ptr(out["dD_c"]), _ptr(out["dh0"]), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_scan_bwd rejected its arguments")
    return out


def scan_bwd(inp: dict, gy, g_last=None, nthreads=None):
    """Oracle of the scan's backward on storage-form inputs (a ``synth`` dict).

    gy: dLoss/dy [B, L, D] (float64, or anything numpy widens exactly);
    g_last: dLoss/dh_last [B, D, N] or None.  Returns float64 gradients with respect to
    every input: dx, ddelta, dz [B, L, D] (ddelta with respect to the raw input in
    softplus mode; dz None without a gate), dB, dC [B, L, N], dA [D, N], dD [D],
    dh0 [B, D, N], and ddelta_bias [D] when ``inp`` has a "delta_bias" (the sum of ddelta
    over batch rows and steps: the bias is added to every step's raw delta).  The
    discretisation is ``inp["discretization"]`` ("mamba" when absent).
    """
    dtype = inp["dtype"]
    x, delta, z = inp["x"], inp["delta"], inp["z"]
    Bsz, L, D = x.shape
    N = inp["A"].shape[1]
    cb, cd = np.meshgrid(np.arange(Bsz), np.arange(D), indexing="ij")
    cb, cd = cb.reshape(-1), cd.reshape(-1)

    def series(a, wide=True):
        if a is None:
            return None
        return _widen(a[cb, :, cd], dtype) if wide else np.asarray(a, np.float64)[cb, :, cd]

    h0 = inp.get("h0")
    h0c = None if h0 is None else np.asarray(h0, dtype=np.float64)[cb, cd, :]
    glc = None if g_last is None else np.asarray(g_last, dtype=np.float64)[cb, cd, :]
    r = scan_bwd_f64(series(x), series(delta), inp["A"], _widen(inp["B"], dtype),
                     _widen(inp["C"], dtype), inp["Dskip"], series(z), h0c,
                     series(gy, wide=False), glc, inp.get("delta_softplus", False), cb, cd, nthreads,
                     inp.get("delta_bias"), inp.get("discretization", "mamba"))
    back = lambda a: a.reshape(Bsz, D, L).transpose(0, 2, 1).copy()
    out = {"dx": back(r["dx"]), "ddelta": back(r["ddelta"]),
           "dz": None if r["dz"] is None else back(r["dz"]),
           "dB": r["dB_c"].reshape(Bsz, D, L, N).sum(axis=1),
           "dC": r["dC_c"].reshape(Bsz, D, L, N).sum(axis=1),
           "dA": r["dA_c"].reshape(Bsz, D, N).sum(axis=0),
           "dD": r["dD_c"].reshape(Bsz, D).sum(axis=0),
           "dh0": r["dh0"].reshape(Bsz, D, N)}
    if inp.get("delta_bias") is not None:
        out["ddelta_bias"] = out["ddelta"].sum(axis=(0, 1))
    return out


def _widen(a, dtype):
    if a is None:
        return None
    if dtype == "bf16":
        return (np.ascontiguousarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)) \
            .view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def scan(inp: dict, channels=None, nthreads=None):
    """Oracle of one selective-scan call on storage-form inputs (a ``synth`` dict).

    channels=None: every channel; returns y [B, L, D] and h_last [B, D, N] (float64).
    Optional keys of ``inp``: "discretization" ("mamba", "zoh", "bilinear") and
    "delta_bias" ([D] float32, added to delta before the softplus).
    channels=[(b, d), ...]: only those; returns y [nchan, L] and h_last [nchan, N].
    """
    dtype = inp["dtype"]
    x, delta, z = inp["x"], inp["delta"], inp["z"]
    Bsz, L, D = x.shape
    N = inp["A"].shape[1]
    if channels is None:
        cb, cd = np.meshgrid(np.arange(Bsz), np.arange(D), indexing="ij")
        cb, cd = cb.reshape(-1), cd.reshape(-1)
    else:
        ch = np.asarray(channels, dtype=np.int64).reshape(-1, 2)
        cb, cd = ch[:, 0], ch[:, 1]

    def series(a):
        if a is None:
            return None
        return _widen(a[cb, :, cd] if len(cb) else a[:0, :, 0], dtype)

    h0 = inp.get("h0")
    h0c = None if h0 is None else np.asarray(h0, dtype=np.float64)[cb, cd, :]
    y, h_last = scan_f64(series(x), series(delta), inp["A"], _widen(inp["B"], dtype),
                         _widen(inp["C"], dtype), inp["Dskip"], series(z), h0c,
                         inp.get("delta_softplus", False), cb, cd, nthreads,
                         inp.get("discretization", "mamba"), inp.get("delta_bias"))
    if channels is None:
        return y.reshape(Bsz, D, L).transpose(0, 2, 1).copy(), h_last.reshape(Bsz, D, N)
    return y, h_last


def state_update(h, step: dict, A, Dskip, dtype: str, channels=None, delta_softplus=False,
                 nthreads=None, discretization="mamba", delta_bias=None):
    """Oracle of one single-token state update (the scan body with L = 1).

    h: float64 state, [B, D, N] (channels=None) or [nchan, N] for the listed
    channels; it is returned updated (a new array) together with y
    ([B, D] or [nchan]).  step holds x, delta, z [B, D] and B, C [B, N] in
    storage form.
    """
    x = step["x"]
    Bsz, D = x.shape
    N = A.shape[1]
    if channels is None:
        cb, cd = np.meshgrid(np.arange(Bsz), np.arange(D), indexing="ij")
        cb, cd = cb.reshape(-1), cd.reshape(-1)
        h0 = np.asarray(h, dtype=np.float64).reshape(Bsz * D, N)
    else:
        ch = np.asarray(channels, dtype=np.int64).reshape(-1, 2)
        cb, cd = ch[:, 0], ch[:, 1]
        h0 = np.asarray(h, dtype=np.float64)

    def series(a):
        return None if a is None else _widen(a[cb, cd], dtype)[:, None]

    Bm = _widen(step["B"], dtype)[:, None, :]
    Cm = _widen(step["C"], dtype)[:, None, :]
    y, h_new = scan_f64(series(x), series(step["delta"]), A, Bm, Cm, Dskip, series(step.get("z")),
                        h0, delta_softplus, cb, cd, nthreads, discretization, delta_bias)
    if channels is None:
        return h_new.reshape(Bsz, D, N), y.reshape(Bsz, D)
    return h_new, y[:, 0]
