"""Seeded synthetic inputs for the selective scan and its single-token state update.

This module only draws random numbers and packs them into storage formats
(bf16 bit patterns, fp32).  It holds none of the scan's arithmetic, so both
the CPU oracle's tests and the GPU path's tests/bench can use it without
sharing any computation.

Recipe (shapes follow the "selective_scan(x, delta, A, B, C, D)" listing on
the managen.ai Mamba page, with B and C one vector of width N per token as in
the MambaBlock listing of the skillsdirectory "State Space Models Mamba" page):

* x ~ N(0, 1)                                    [B, L, D]
* delta log-uniform in [1e-3, 1e-1]              [B, L, D]
  (in softplus mode the stored tensor is u = log(expm1(delta)), so that
  softplus(u) = delta is log-uniform)
* z ~ N(0, 1)                                    [B, L, D]  (gate input)
* B, C ~ N(0, 1)                                 [B, L, N]
* A[d, n] = -(n + 1)        (the Mamba A_log = log(1..N) initialisation),
  or, with ``a_kind="random"``, -(n + 1) * exp(N(0, 0.5)) per (d, n) so
  that no structure across n holds
* Dskip = ones, or N(1, 0.1)                     [D]
* h0 ~ N(0, 1) when requested                    [B, D, N]  fp32
* delta bias ~ N(0, 0.5) when requested          [D]  fp32 (the bias of the map that
  produces delta; it scales the softplus step size by about e^bias)

Every [B, L, *] tensor is drawn in fixed blocks of ``BLOCK_ROWS`` rows of the
flattened (B*L) axis, each block from its own PCG64 stream keyed by
(seed, tensor id, block index).  Any slab of rows can therefore be regenerated
on its own, bit for bit, which is how million-token inputs are produced in
pieces.  Values are drawn in float32 and rounded to bf16 with
round-to-nearest-even when the storage dtype is bf16.
"""
from __future__ import annotations

import numpy as np

BLOCK_ROWS = 4096

_TENSOR_IDS = {"x": 1, "delta": 2, "z": 3, "B": 4, "C": 5, "A": 6, "D": 7, "h0": 8, "dbias": 9,
               "ssd_A": 10}

DELTA_MIN = 1e-3
DELTA_MAX = 1e-1


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return the uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    out = ((bits + rounding) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values ("bf16" bit patterns or "f32") to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def store(a32: np.ndarray, dtype: str) -> np.ndarray:
    """Put float32 values into storage form: uint16 bf16 bit patterns or float32."""
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def _rng(seed: int, tensor: str, block: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), _TENSOR_IDS[tensor], int(block)])


def _rows(seed: int, tensor: str, row0: int, row1: int, width: int, kind: str,
          softplus_input: bool = False) -> np.ndarray:
    """Float32 draws for rows [row0, row1) of a [rows, width] tensor, block-keyed."""
    out = np.empty((row1 - row0, width), dtype=np.float32)
    blk0 = row0 // BLOCK_ROWS
    blk1 = (row1 + BLOCK_ROWS - 1) // BLOCK_ROWS
    for blk in range(blk0, blk1):
        r_lo = blk * BLOCK_ROWS
        r_hi = r_lo + BLOCK_ROWS
        g = _rng(seed, tensor, blk)
        if kind == "normal":
            vals = g.standard_normal((BLOCK_ROWS, width), dtype=np.float32)
        elif kind == "delta":
            lo, hi = np.log(DELTA_MIN), np.log(DELTA_MAX)
            e = g.random((BLOCK_ROWS, width), dtype=np.float32)
            vals = np.exp(lo + (hi - lo) * e.astype(np.float64))
            if softplus_input:
                vals = np.log(np.expm1(vals))
            vals = vals.astype(np.float32)
        else:
            raise ValueError(kind)
        a, b = max(row0, r_lo), min(row1, r_hi)
        if a < b:
            out[a - row0:b - row0] = vals[a - r_lo:b - r_lo]
    return out


def token_rows(seed: int, tensor: str, row0: int, row1: int, width: int, dtype: str,
               softplus_input: bool = False) -> np.ndarray:
    """Rows [row0, row1) of the flattened (batch*seqlen) axis of x / delta / z / B / C."""
    kind = "delta" if tensor == "delta" else "normal"
    return store(_rows(seed, tensor, row0, row1, width, kind, softplus_input), dtype)


def make_A(seed: int, dim: int, dstate: int, a_kind: str = "mamba") -> np.ndarray:
    n = np.arange(1, dstate + 1, dtype=np.float32)
    A = -np.broadcast_to(n, (dim, dstate)).astype(np.float32).copy()
    if a_kind == "mamba":
        return A
    if a_kind == "random":
        g = _rng(seed, "A", 0)
        return (A * np.exp(0.5 * g.standard_normal((dim, dstate)))).astype(np.float32)
    raise ValueError(a_kind)


def make_D(seed: int, dim: int, d_kind: str = "ones") -> np.ndarray:
    if d_kind == "ones":
        return np.ones(dim, dtype=np.float32)
    if d_kind == "normal":
        g = _rng(seed, "D", 0)
        return (1.0 + 0.1 * g.standard_normal(dim)).astype(np.float32)
    raise ValueError(d_kind)


def make_delta_bias(seed: int, dim: int) -> np.ndarray:
    g = _rng(seed, "dbias", 0)
    return (0.5 * g.standard_normal(dim)).astype(np.float32)


def make_h0(seed: int, batch: int, dim: int, dstate: int) -> np.ndarray:
    g = _rng(seed, "h0", 0)
    return g.standard_normal((batch, dim, dstate), dtype=np.float32)


def scan_inputs(batch: int, seqlen: int, dim: int, dstate: int, dtype: str, seed: int,
                gate: bool = False, d_kind: str = "ones", a_kind: str = "mamba",
                softplus_input: bool = False, h0: bool = False) -> dict:
    """All inputs of one selective-scan call, in storage form.

    Returns a dict with x, delta, z (or None) of shape [B, L, D], B and C of
    shape [B, L, N] (uint16 bf16 bits or float32 per ``dtype``), A [D, N] and
    Dskip [D] float32, and h0 [B, D, N] float32 or None.
    """
    rows = batch * seqlen
    out = {
        "x": token_rows(seed, "x", 0, rows, dim, dtype).reshape(batch, seqlen, dim),
        "delta": token_rows(seed, "delta", 0, rows, dim, dtype, softplus_input).reshape(batch, seqlen, dim),
        "z": token_rows(seed, "z", 0, rows, dim, dtype).reshape(batch, seqlen, dim) if gate else None,
        "B": token_rows(seed, "B", 0, rows, dstate, dtype).reshape(batch, seqlen, dstate),
        "C": token_rows(seed, "C", 0, rows, dstate, dtype).reshape(batch, seqlen, dstate),
        "A": make_A(seed, dim, dstate, a_kind),
        "Dskip": make_D(seed, dim, d_kind),
        "h0": make_h0(seed, batch, dim, dstate) if h0 else None,
        "dtype": dtype,
        "delta_softplus": bool(softplus_input),
        "shape": (batch, seqlen, dim, dstate),
    }
    return out


def ssd_inputs(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int, dtype: str,
               seed: int, gate: bool = False, softplus_input: bool = False, h0: bool = False,
               delta_bias: bool = False, ngroups: int = 1) -> dict:
    """Inputs of one multi-head SSD (Mamba-2 layer) scan, in storage form.

    x, z [B, L, H, P] and B, C [B, L, N] ~ N(0, 1); delta [B, L, H] log-uniform in
    [1e-3, 1e-1] (one step per head; u = log(expm1(delta)) in softplus mode); A [H]
    float32 = -exp(U[log 1, log 16]) (one decay rate per head, the range Mamba-2
    initialises A in); Dskip [H] ~ N(1, 0.1); h0 [B, H, P, N] ~ N(0, 1) float32;
    delta_bias [H] ~ N(0, 0.5) (softplus mode) or 0.05 |N(0, 0.5)|.  ngroups > 1: B, C
    are [B, L, G, N] (one row per group of heads).
    """
    bc = (batch, seqlen, dstate) if ngroups == 1 else (batch, seqlen, ngroups, dstate)
    rows = batch * seqlen
    g = _rng(seed, "ssd_A", 0)
    A = (-np.exp(g.uniform(0.0, np.log(16.0), nheads))).astype(np.float32)
    bias = None
    if delta_bias:
        bias = make_delta_bias(seed, nheads)
        if not softplus_input:
            bias = (0.05 * np.abs(bias)).astype(np.float32)
    return {
        "x": token_rows(seed, "x", 0, rows, nheads * headdim, dtype).reshape(batch, seqlen, nheads, headdim),
        "delta": token_rows(seed, "delta", 0, rows, nheads, dtype, softplus_input).reshape(batch, seqlen, nheads),
        "z": (token_rows(seed, "z", 0, rows, nheads * headdim, dtype).reshape(batch, seqlen, nheads, headdim)
              if gate else None),
        "B": token_rows(seed, "B", 0, rows, ngroups * dstate, dtype).reshape(bc),
        "C": token_rows(seed, "C", 0, rows, ngroups * dstate, dtype).reshape(bc),
        "A": A,
        "Dskip": make_D(seed, nheads, "normal"),
        "h0": (_rng(seed, "h0", 0).standard_normal((batch, nheads, headdim, dstate), dtype=np.float32)
               if h0 else None),
        "delta_bias": bias,
        "dtype": dtype,
        "delta_softplus": bool(softplus_input),
        "shape": (batch, seqlen, nheads, headdim, dstate),
    }


# The five workloads: (name, batch, seqlen, dim, dstate, dtype, gate, d_kind)
CONFIGS = {
    "tiny_f32": dict(seed=0, name="tiny scan B1 L256 D64 N16 fp32", batch=1, seqlen=256, dim=64, dstate=16,
            dtype="f32", gate=False, d_kind="ones"),
    "mamba130m_layer": dict(seed=1, name="Mamba-130M-layer scan B8 L2048 D1536 N16 bf16 gated", batch=8, seqlen=2048,
            dim=1536, dstate=16, dtype="bf16", gate=True, d_kind="ones"),
    "mamba1p4b_layer": dict(seed=2, name="Mamba-1.4B-layer scan B4 L4096 D4096 N16 bf16 gated", batch=4, seqlen=4096,
            dim=4096, dstate=16, dtype="bf16", gate=True, d_kind="normal"),
    "million_token": dict(seed=3, name="million-token scan B1 L1048576 D1024 N16 bf16", batch=1, seqlen=1 << 20,
            dim=1024, dstate=16, dtype="bf16", gate=False, d_kind="normal"),
    "decode": dict(seed=4, name="decode state update h[256,4096,16] x 1024 steps bf16 gated", batch=256,
            seqlen=1024, dim=4096, dstate=16, dtype="bf16", gate=True, d_kind="normal"),
}


def config_inputs(name: str, seed: int | None = None, **overrides) -> dict:
    """Inputs of the named workload (its own seed unless ``seed`` is given)."""
    c = dict(CONFIGS[name])
    c.update(overrides)
    return scan_inputs(c["batch"], c["seqlen"], c["dim"], c["dstate"], c["dtype"],
                       c["seed"] if seed is None else seed, gate=c["gate"], d_kind=c["d_kind"],
                       a_kind=c.get("a_kind", "mamba"), softplus_input=c.get("softplus_input", False),
                       h0=c.get("h0", False))


def decode_step_inputs(seed: int, step: int, batch: int, dim: int, dstate: int, dtype: str,
                       gate: bool = True) -> dict:
    """Per-token inputs of decode step ``step``: x, delta, z [B, D] and B, C [B, N].

    Each step has its own PCG64 stream per tensor, keyed by (seed, tensor id,
    step), so any step is regenerated on its own.
    """
    def draw(tensor, width):
        g = np.random.default_rng([int(seed), _TENSOR_IDS[tensor], int(step), 0xDEC0])
        if tensor == "delta":
            lo, hi = np.log(DELTA_MIN), np.log(DELTA_MAX)
            e = g.random((batch, width), dtype=np.float32).astype(np.float64)
            return store(np.exp(lo + (hi - lo) * e).astype(np.float32), dtype)
        return store(g.standard_normal((batch, width), dtype=np.float32), dtype)

    return {"x": draw("x", dim), "delta": draw("delta", dim), "z": draw("z", dim) if gate else None,
            "B": draw("B", dstate), "C": draw("C", dstate)}
