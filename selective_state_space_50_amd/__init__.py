"""MI355X (gfx950) selective scan: thin Python binding of libssm.so.

The binding only marshals arguments: it checks tensor dtypes, devices and
contiguity, allocates outputs and the workspace with torch, and passes raw
device pointers plus torch's current HIP stream to the C ABI declared in
``include/ssm.h``.  Every step of the computation runs in the HIP kernels.
There is no CPU fallback: if the library is missing or fails to load, every
call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

__all__ = ["scan_fwd", "scan_fwd_save", "scan_save_sizes", "scan_bwd", "state_update", "scan_plan", "scan_workspace_bytes",
           "scan_bwd_workspace_bytes", "selective_scan", "conv1d_fwd", "conv1d_update", "lib",
           "SSMError", "LIB_PATH",
           "HEADER_PATH", "exported_api"]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssm.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "ssm.h")

SSM_OK, SSM_EINVAL, SSM_EUNSUPPORTED, SSM_EWORKSPACE, SSM_EHIP = range(5)
DTYPE_F32, DTYPE_BF16 = 0, 1
ABI_VERSION = 7     # SSM_ABI_VERSION of include/ssm.h


class SSMError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func} failed with status {status} ({_status_name(status)}): {detail}")


class ScanOpts(ctypes.Structure):
    _fields_ = [("chunk_len", ctypes.c_int64), ("states_per_lane", ctypes.c_int32),
                ("time_block", ctypes.c_int32), ("one_block_per_cu", ctypes.c_int32),
                ("a_structure", ctypes.c_int32)]


class Variant(ctypes.Structure):
    _fields_ = [("discretization", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("delta_bias", ctypes.c_void_p)]


DISCRETIZATIONS = {"mamba": 0, "zoh": 1, "bilinear": 2}


class ScanPlan(ctypes.Structure):
    _fields_ = [("chunk_len", ctypes.c_int64), ("n_chunks", ctypes.c_int64),
                ("states_per_lane", ctypes.c_int32), ("waves_per_block", ctypes.c_int32),
                ("time_block", ctypes.c_int32), ("specialised", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64), ("blocks", ctypes.c_uint64),
                ("lds_reserve", ctypes.c_uint64)]


_lib = None


def lib():
    """Load libssm.so (built in-tree by ``__graft_entry__.build()``); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libssm.so not found at {LIB_PATH}: build it first "
                          "(python -c 'import __graft_entry__ as g; g.build()')")
    # torch first: its HIP runtime is then the one libssm.so binds to (a process must not
    # load a second copy of the runtime, which would see no devices)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    I64, I32, P, SZ = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    L.ssm_abi_version.restype = I32
    L.ssm_abi_version.argtypes = []
    L.ssm_status_str.restype = ctypes.c_char_p
    L.ssm_status_str.argtypes = [I32]
    L.ssm_last_error.restype = ctypes.c_char_p
    L.ssm_last_error.argtypes = []
    L.ssm_scan_plan_get.restype = I32
    L.ssm_scan_plan_get.argtypes = [I64, I64, I64, I64, I32, ctypes.POINTER(ScanOpts),
                                    ctypes.POINTER(ScanPlan)]
    L.ssm_scan_workspace_bytes.restype = SZ
    L.ssm_scan_workspace_bytes.argtypes = [I64, I64, I64, I64, I32, ctypes.POINTER(ScanOpts)]
    L.ssm_scan_fwd.restype = I32
    L.ssm_scan_fwd.argtypes = [I64, I64, I64, I64, I32, P, P, P, P, P, P, P, P, P, P, I32,
                               ctypes.POINTER(Variant), ctypes.POINTER(ScanOpts), P, SZ, P]
    L.ssm_issue_probe.restype = I32
    L.ssm_issue_probe.argtypes = [I32, I64, I64, I64, P, P]
    L.ssm_noalloc_scratch_bytes.restype = SZ
    L.ssm_noalloc_scratch_bytes.argtypes = []
    L.ssm_scan_fwd_noalloc.restype = I32
    L.ssm_scan_fwd_noalloc.argtypes = [I64, I64, I64, I64, I32, P, P, P, P, P, P, P, P, P, P, I32,
                                       ctypes.POINTER(Variant), ctypes.POINTER(ScanOpts), P]
    L.ssm_state_update.restype = I32
    L.ssm_state_update.argtypes = [I64, I64, I64, I32, P, P, P, P, P, P, P, P, P, I32,
                                   ctypes.POINTER(Variant), P]
    L.ssm_scan_bwd_workspace_bytes.restype = SZ
    L.ssm_scan_bwd_workspace_bytes.argtypes = [I64, I64, I64, I64, I32, I32]
    L.ssm_scan_bwd.restype = I32
    L.ssm_scan_bwd.argtypes = [I64, I64, I64, I64, I32] + [P] * 18 + [I32, I32, P, P, P, P, SZ, P]
    L.ssm_scan_save_sizes.restype = I32
    L.ssm_scan_save_sizes.argtypes = [I64, I64, I64, I64, I32, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]
    L.ssm_scan_fwd_save.restype = I32
    L.ssm_scan_fwd_save.argtypes = [I64, I64, I64, I64, I32] + [P] * 10 + [I32, ctypes.POINTER(Variant), P, P, SZ, P]
    L.ssm_conv1d_fwd.restype = I32
    L.ssm_conv1d_fwd.argtypes = [I64, I64, I64, I64, I32, P, P, P, P, P, P, I32, P]
    L.ssm_ssd_fwd.restype = I32
    L.ssm_ssd_fwd.argtypes = [I64, I64, I64, I64, I64, I64, I32] + [P] * 11 + [I32, P]
    L.ssm_ssd_bwd_workspace_bytes.restype = SZ
    L.ssm_ssd_bwd_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, I32]
    L.ssm_ssd_bwd.restype = I32
    L.ssm_ssd_bwd.argtypes = [I64, I64, I64, I64, I64, I64, I32] + [P] * 20 + [I32, P, SZ, P]
    L.ssm_conv1d_update.restype = I32
    L.ssm_conv1d_update.argtypes = [I64, I64, I64, I32, P, P, P, P, P, I32, P]
    L.ssm_conv1d_bwd_workspace_bytes.restype = SZ
    L.ssm_conv1d_bwd_workspace_bytes.argtypes = [I64, I64, I64, I64, I32]
    L.ssm_conv1d_bwd.restype = I32
    L.ssm_conv1d_bwd.argtypes = [I64, I64, I64, I64, I32] + [P] * 9 + [I32, P, SZ, P]
    if L.ssm_abi_version() != ABI_VERSION:
        raise ImportError(f"libssm ABI version {L.ssm_abi_version()} != {ABI_VERSION}")
    _lib = L
    return L


def _status_name(status: int) -> str:
    try:
        return lib().ssm_status_str(status).decode()
    except Exception:  # pragma: no cover - used while building an error message
        return "?"


def _check(status: int, func: str):
    if status != SSM_OK:
        raise SSMError(status, func, lib().ssm_last_error().decode())


def exported_api():
    """Function names declared in include/ssm.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z_]+)\s*\(", text)))


def _opts(chunk_len=0, states_per_lane=0, time_block=0, one_block_per_cu=0, general_a=False):
    if not (chunk_len or states_per_lane or time_block or one_block_per_cu or general_a):
        return None
    return ScanOpts(int(chunk_len), int(states_per_lane), int(time_block), int(one_block_per_cu),
                    -1 if general_a else 0)


def _variant(discretization, delta_bias, dim, device):
    """The ssm_variant of a call (None for the default: Mamba, no delta bias)."""
    import torch
    if discretization not in DISCRETIZATIONS:
        raise ValueError(f"discretization {discretization!r} is not one of {sorted(DISCRETIZATIONS)}")
    _need(delta_bias, "delta_bias", (dim,), torch.float32, device)
    if discretization == "mamba" and delta_bias is None:
        return None
    return Variant(DISCRETIZATIONS[discretization], 0, _ptr(delta_bias))


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def scan_plan(batch, seqlen, dim, dstate, dtype="bf16", chunk_len=0, states_per_lane=0,
              time_block=0, one_block_per_cu=0) -> dict:
    """What ssm_scan_fwd will launch for this shape (host-only)."""
    code = DTYPE_BF16 if dtype in ("bf16", "bfloat16") else DTYPE_F32
    p = ScanPlan()
    o = _opts(chunk_len, states_per_lane, time_block, one_block_per_cu)
    _check(lib().ssm_scan_plan_get(batch, seqlen, dim, dstate, code,
                                   ctypes.byref(o) if o else None, ctypes.byref(p)),
           "ssm_scan_plan_get")
    return {k: getattr(p, k) for k, _ in ScanPlan._fields_}


def scan_workspace_bytes(batch, seqlen, dim, dstate, dtype="bf16", chunk_len=0,
                         states_per_lane=0, time_block=0, one_block_per_cu=0) -> int:
    code = DTYPE_BF16 if dtype in ("bf16", "bfloat16") else DTYPE_F32
    o = _opts(chunk_len, states_per_lane, time_block, one_block_per_cu)
    return int(lib().ssm_scan_workspace_bytes(batch, seqlen, dim, dstate, code,
                                              ctypes.byref(o) if o else None))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, shape, dtype, device):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def scan_fwd(x, delta, A, B, C, D=None, z=None, h0=None, *, delta_softplus=False,
             discretization="mamba", delta_bias=None,
             return_last_state=False, out=None, h_last=None, workspace=None, chunk_len=0,
             states_per_lane=0, time_block=0, one_block_per_cu=0, general_a=False, stream=None):
    """Selective scan y = S6(x, delta, A, B, C, D) [* silu(z)] on the GPU.

    x, delta, z: [B, L, D];  B, C: [B, L, N];  A: [D, N] fp32;  D: [D] fp32;
    h0: [B, D, N] fp32.  x/delta/z/B/C share one dtype (bfloat16 or float32).
    discretization: "mamba" (A_bar = exp(dt A), B_bar = dt B), "zoh" or "bilinear";
    delta_bias: [D] fp32 added to delta before the softplus.
    general_a: always one exp per state (never the structured-A path, ssm_scan_opts.a_structure).
    Returns y (same dtype as x), or (y, h_last) when return_last_state.
    """
    import torch
    if x.dim() != 3 or A.dim() != 2:
        raise ValueError("x must be [batch, seqlen, dim] and A [dim, dstate]")
    Bsz, L, Dm = x.shape
    N = A.shape[1]
    dev, dt = x.device, x.dtype
    if dev.type != "cuda":
        raise ValueError("scan_fwd runs on the GPU only; tensors must be on a cuda device")
    _need(x, "x", (Bsz, L, Dm), dt, dev)
    _need(delta, "delta", (Bsz, L, Dm), dt, dev)
    _need(z, "z", (Bsz, L, Dm), dt, dev)
    _need(B, "B", (Bsz, L, N), dt, dev)
    _need(C, "C", (Bsz, L, N), dt, dev)
    _need(A, "A", (Dm, N), torch.float32, dev)
    _need(D, "D", (Dm,), torch.float32, dev)
    _need(h0, "h0", (Bsz, Dm, N), torch.float32, dev)
    v = _variant(discretization, delta_bias, Dm, dev)
    code = _dtype_code(x)
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", (Bsz, L, Dm), dt, dev)
    if return_last_state and h_last is None:
        h_last = torch.empty((Bsz, Dm, N), dtype=torch.float32, device=dev)
    _need(h_last, "h_last", (Bsz, Dm, N), torch.float32, dev)
    o = _opts(chunk_len, states_per_lane, time_block, one_block_per_cu, general_a)
    ws_bytes = int(lib().ssm_scan_workspace_bytes(Bsz, L, Dm, N, code, ctypes.byref(o) if o else None))
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    st = lib().ssm_scan_fwd(Bsz, L, Dm, N, code, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                            _ptr(D), _ptr(z), _ptr(h0), _ptr(h_last), _ptr(out),
                            int(bool(delta_softplus)), ctypes.byref(v) if v else None,
                            ctypes.byref(o) if o else None,
                            _ptr(workspace) if ws_bytes else None, ws_bytes,
                            ctypes.c_void_p(s.cuda_stream))
    _check(st, "ssm_scan_fwd")
    return (out, h_last) if return_last_state else out


def scan_fwd_noalloc(x, delta, A, B, C, D=None, z=None, h0=None, *, delta_softplus=False,
                     discretization="mamba", delta_bias=None, out=None, h_last=None, chunk_len=0,
                     states_per_lane=0, general_a=False, stream=None):
    """scan_fwd through ssm_scan_fwd_noalloc: the library's fixed scratch array stands in for
    the workspace, so the call itself allocates no device memory when ``out`` (and
    ``h_last``, if wanted) are given.  Returns y, or (y, h_last) when h_last is given."""
    import torch
    if x.dim() != 3 or A.dim() != 2:
        raise ValueError("x must be [batch, seqlen, dim] and A [dim, dstate]")
    Bsz, L, Dm = x.shape
    N = A.shape[1]
    dev, dt = x.device, x.dtype
    if dev.type != "cuda":
        raise ValueError("scan_fwd_noalloc runs on the GPU only; tensors must be on a cuda device")
    for t, name, shape, tdt in ((x, "x", (Bsz, L, Dm), dt), (delta, "delta", (Bsz, L, Dm), dt),
                                (z, "z", (Bsz, L, Dm), dt), (B, "B", (Bsz, L, N), dt),
                                (C, "C", (Bsz, L, N), dt), (A, "A", (Dm, N), torch.float32),
                                (D, "D", (Dm,), torch.float32), (h0, "h0", (Bsz, Dm, N), torch.float32),
                                (h_last, "h_last", (Bsz, Dm, N), torch.float32)):
        _need(t, name, shape, tdt, dev)
    v = _variant(discretization, delta_bias, Dm, dev)
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", (Bsz, L, Dm), dt, dev)
    o = _opts(chunk_len, states_per_lane, 0, 0, general_a)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    st = lib().ssm_scan_fwd_noalloc(Bsz, L, Dm, N, _dtype_code(x), _ptr(x), _ptr(delta), _ptr(A), _ptr(B),
                                    _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(h_last), _ptr(out),
                                    int(bool(delta_softplus)), ctypes.byref(v) if v else None,
                                    ctypes.byref(o) if o else None, ctypes.c_void_p(s.cuda_stream))
    _check(st, "ssm_scan_fwd_noalloc")
    return (out, h_last) if h_last is not None else out


def issue_rates(workgroups=256, waves_per_workgroup=16, iters=4096, reps=5):
    """Measured VALU issue rates (lane operations per second) of an fp32 FMA, v_exp_f32 and
    v_rcp_f32 on the current GPU (ssm_issue_probe, timed with events; median of reps)."""
    import torch
    dev = torch.device("cuda", torch.cuda.current_device())
    sink = torch.empty(64 * waves_per_workgroup, dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream(dev)
    ops = workgroups * waves_per_workgroup * 64 * 8 * iters
    out = {}
    for op, name in ((0, "fma"), (1, "exp"), (2, "rcp")):
        times = []
        for r in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            _check(lib().ssm_issue_probe(op, workgroups, waves_per_workgroup, iters, _ptr(sink),
                                         ctypes.c_void_p(s.cuda_stream)), "ssm_issue_probe")
            e1.record(s)
            e1.synchronize()
            if r:
                times.append(e0.elapsed_time(e1))
        times.sort()
        out[name] = ops / (times[len(times) // 2] * 1e-3)
    return out


def state_update(h, x, delta, A, B, C, D=None, z=None, *, delta_softplus=False,
                 discretization="mamba", delta_bias=None, out=None, stream=None):
    """One recurrent step: updates h [B, D, N] fp32 in place and returns y [B, D].

    x, delta, z: [B, D];  B, C: [B, N];  A: [D, N] fp32;  D: [D] fp32;
    discretization and delta_bias as for scan_fwd.
    """
    import torch
    if h.dim() != 3:
        raise ValueError("h must be [batch, dim, dstate]")
    Bsz, Dm, N = h.shape
    dev, dt = x.device, x.dtype
    if dev.type != "cuda":
        raise ValueError("state_update runs on the GPU only; tensors must be on a cuda device")
    _need(h, "h", (Bsz, Dm, N), torch.float32, dev)
    _need(x, "x", (Bsz, Dm), dt, dev)
    _need(delta, "delta", (Bsz, Dm), dt, dev)
    _need(z, "z", (Bsz, Dm), dt, dev)
    _need(B, "B", (Bsz, N), dt, dev)
    _need(C, "C", (Bsz, N), dt, dev)
    _need(A, "A", (Dm, N), torch.float32, dev)
    _need(D, "D", (Dm,), torch.float32, dev)
    v = _variant(discretization, delta_bias, Dm, dev)
    code = _dtype_code(x)
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", (Bsz, Dm), dt, dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    st = lib().ssm_state_update(Bsz, Dm, N, code, _ptr(h), _ptr(x), _ptr(delta), _ptr(A), _ptr(B),
                                _ptr(C), _ptr(D), _ptr(z), _ptr(out), int(bool(delta_softplus)),
                                ctypes.byref(v) if v else None, ctypes.c_void_p(s.cuda_stream))
    _check(st, "ssm_state_update")
    return out


def scan_bwd_workspace_bytes(batch, seqlen, dim, dstate, dtype="bf16", saved_checkpoints=False) -> int:
    code = DTYPE_BF16 if dtype in ("bf16", "bfloat16") else DTYPE_F32
    return int(lib().ssm_scan_bwd_workspace_bytes(batch, seqlen, dim, dstate, code, int(bool(saved_checkpoints))))


def scan_save_sizes(batch, seqlen, dim, dstate, dtype="bf16"):
    """(workspace bytes, checkpoint bytes) of scan_fwd_save at this shape."""
    code = DTYPE_BF16 if dtype in ("bf16", "bfloat16") else DTYPE_F32
    ws, ck = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib().ssm_scan_save_sizes(batch, seqlen, dim, dstate, code, ctypes.byref(ws), ctypes.byref(ck)),
           "ssm_scan_save_sizes")
    return int(ws.value), int(ck.value)


def scan_fwd_save(x, delta, A, B, C, D=None, z=None, h0=None, *, delta_softplus=False,
                  discretization="mamba", delta_bias=None, return_last_state=False, out=None,
                  h_last=None, checkpoints=None, workspace=None, stream=None):
    """scan_fwd that also stores the state before every 8th step for scan_bwd (its
    ``checkpoints`` argument), on the backward's sequence chunking.  Arguments as
    scan_fwd (dstate 16 and dim a multiple of 64 only).  Returns (y, checkpoints), or
    (y, h_last, checkpoints) when return_last_state; checkpoints is a flat fp32 tensor
    [B, ceil(L/8), N, D]."""
    import torch
    if x.dim() != 3 or A.dim() != 2:
        raise ValueError("x must be [batch, seqlen, dim] and A [dim, dstate]")
    Bsz, L, Dm = x.shape
    N = A.shape[1]
    dev, dt = x.device, x.dtype
    if dev.type != "cuda":
        raise ValueError("scan_fwd_save runs on the GPU only; tensors must be on a cuda device")
    for t, name, shape, tdt in ((x, "x", (Bsz, L, Dm), dt), (delta, "delta", (Bsz, L, Dm), dt),
                                (z, "z", (Bsz, L, Dm), dt), (B, "B", (Bsz, L, N), dt), (C, "C", (Bsz, L, N), dt),
                                (A, "A", (Dm, N), torch.float32), (D, "D", (Dm,), torch.float32),
                                (h0, "h0", (Bsz, Dm, N), torch.float32)):
        _need(t, name, shape, tdt, dev)
    v = _variant(discretization, delta_bias, Dm, dev)
    code = _dtype_code(x)
    ws_bytes, ck_bytes = scan_save_sizes(Bsz, L, Dm, N, "bf16" if code == DTYPE_BF16 else "f32")
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", (Bsz, L, Dm), dt, dev)
    if return_last_state and h_last is None:
        h_last = torch.empty((Bsz, Dm, N), dtype=torch.float32, device=dev)
    _need(h_last, "h_last", (Bsz, Dm, N), torch.float32, dev)
    nck = (L + 7) // 8
    if checkpoints is None:
        checkpoints = torch.empty((Bsz, nck, N, Dm), dtype=torch.float32, device=dev)
    _need(checkpoints, "checkpoints", (Bsz, nck, N, Dm), torch.float32, dev)
    if not checkpoints.is_contiguous() or checkpoints.numel() * 4 != ck_bytes:
        raise ValueError(f"checkpoints must be a contiguous fp32 tensor of {ck_bytes} bytes")
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    st = lib().ssm_scan_fwd_save(Bsz, L, Dm, N, code, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                 _ptr(D), _ptr(z), _ptr(h0), _ptr(h_last), _ptr(out),
                                 int(bool(delta_softplus)), ctypes.byref(v) if v else None,
                                 _ptr(checkpoints), _ptr(workspace) if ws_bytes else None, ws_bytes,
                                 ctypes.c_void_p(s.cuda_stream))
    _check(st, "ssm_scan_fwd_save")
    return (out, h_last, checkpoints) if return_last_state else (out, checkpoints)


def scan_bwd(x, delta, A, B, C, D=None, z=None, h0=None, dy=None, dh_last=None, *,
             delta_softplus=False, discretization="mamba", delta_bias=None, need_dh0=True,
             checkpoints=None, workspace=None, stream=None):
    """Gradients of a loss through scan_fwd, given dy = dLoss/dy [B, L, D] (same dtype as
    x) and optionally dh_last = dLoss/dh_last [B, D, N] fp32.  discretization and
    delta_bias [D] fp32: as in scan_fwd.  checkpoints: what scan_fwd_save stored for these
    same inputs (the call then skips its own forward sweep), or None.

    Returns a dict: dx, ddelta, dz (None without z) in x's dtype [B, L, D]; dB, dC in
    x's dtype [B, L, N]; dA [D, N], dD [D] (None without D), ddelta_bias [D] (None
    without a bias) and dh0 [B, D, N] in fp32 (dh0 None when need_dh0 is false).
    """
    import torch
    if x.dim() != 3 or A.dim() != 2:
        raise ValueError("x must be [batch, seqlen, dim] and A [dim, dstate]")
    Bsz, L, Dm = x.shape
    N = A.shape[1]
    dev, dt = x.device, x.dtype
    if dev.type != "cuda":
        raise ValueError("scan_bwd runs on the GPU only; tensors must be on a cuda device")
    if dy is None:
        raise ValueError("dy is required")
    if discretization not in DISCRETIZATIONS:
        raise ValueError(f"discretization {discretization!r} is not one of {sorted(DISCRETIZATIONS)}")
    for t, name, shape, tdt in ((x, "x", (Bsz, L, Dm), dt), (delta, "delta", (Bsz, L, Dm), dt),
                                (z, "z", (Bsz, L, Dm), dt), (B, "B", (Bsz, L, N), dt),
                                (C, "C", (Bsz, L, N), dt), (A, "A", (Dm, N), torch.float32),
                                (D, "D", (Dm,), torch.float32), (h0, "h0", (Bsz, Dm, N), torch.float32),
                                (dy, "dy", (Bsz, L, Dm), dt), (dh_last, "dh_last", (Bsz, Dm, N), torch.float32),
                                (delta_bias, "delta_bias", (Dm,), torch.float32)):
        _need(t, name, shape, tdt, dev)
    if checkpoints is not None:
        _need(checkpoints, "checkpoints", (Bsz, (L + 7) // 8, N, Dm), torch.float32, dev)
    code = _dtype_code(x)
    out = {"dx": torch.empty_like(x), "ddelta": torch.empty_like(x),
           "dz": torch.empty_like(x) if z is not None else None,
           "dB": torch.empty((Bsz, L, N), dtype=dt, device=dev),
           "dC": torch.empty((Bsz, L, N), dtype=dt, device=dev),
           "dA": torch.empty((Dm, N), dtype=torch.float32, device=dev),
           "dD": torch.empty((Dm,), dtype=torch.float32, device=dev) if D is not None else None,
           "dh0": torch.empty((Bsz, Dm, N), dtype=torch.float32, device=dev) if need_dh0 else None,
           "ddelta_bias": torch.empty((Dm,), dtype=torch.float32, device=dev) if delta_bias is not None else None}
    ws_bytes = int(lib().ssm_scan_bwd_workspace_bytes(Bsz, L, Dm, N, code, int(checkpoints is not None)))
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    st = lib().ssm_scan_bwd(Bsz, L, Dm, N, code, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                            _ptr(D), _ptr(z), _ptr(h0), _ptr(dy), _ptr(dh_last), _ptr(out["dx"]),
                            _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]),
                            _ptr(out["dD"]), _ptr(out["dz"]), _ptr(out["dh0"]), int(bool(delta_softplus)),
                            DISCRETIZATIONS[discretization], _ptr(delta_bias), _ptr(out["ddelta_bias"]),
                            _ptr(checkpoints), _ptr(workspace) if ws_bytes else None, ws_bytes,
                            ctypes.c_void_p(s.cuda_stream))
    _check(st, "ssm_scan_bwd")
    return out


def selective_scan(x, delta, A, B, C, D=None, z=None, h0=None, delta_softplus=False, delta_bias=None,
                   discretization="mamba"):
    """Differentiable selective scan: y = scan_fwd(...) with a torch autograd backward
    through scan_bwd (gradients for every tensor argument, delta_bias included).  The
    forward stores the state checkpoints (scan_fwd_save) when the shape allows them
    (dstate 16, dim a multiple of 64), so that the backward skips its own forward
    sweep."""
    import torch

    class _Scan(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, delta, A, B, C, D, z, h0, delta_bias):
            ck = None
            if A.shape[1] == 16 and x.shape[2] % 64 == 0 and x.shape[1] > 0:
                y, ck = scan_fwd_save(x, delta, A, B, C, D, z, h0, delta_softplus=delta_softplus,
                                      discretization=discretization, delta_bias=delta_bias)
            else:
                y = scan_fwd(x, delta, A, B, C, D, z, h0, delta_softplus=delta_softplus,
                             discretization=discretization, delta_bias=delta_bias)
            ctx.save_for_backward(x, delta, A, B, C, D, z, h0, delta_bias, ck)
            return y

        @staticmethod
        def backward(ctx, gy):
            x, delta, A, B, C, D, z, h0, delta_bias, ck = ctx.saved_tensors
            g = scan_bwd(x, delta, A, B, C, D, z, h0, gy.contiguous(), delta_softplus=delta_softplus,
                         discretization=discretization, delta_bias=delta_bias, checkpoints=ck, need_dh0=h0 is not None and ctx.needs_input_grad[7])
            return (g["dx"], g["ddelta"], g["dA"], g["dB"], g["dC"], g["dD"], g["dz"], g["dh0"],
                    g["ddelta_bias"])

    return _Scan.apply(x, delta, A, B, C, D, z, h0, delta_bias)


def conv1d_fwd(x, w, bias=None, state=None, *, silu=True, return_state=False, out=None, stream=None):
    """Causal depthwise convolution along the sequence (+ SiLU): x [B, L, D] (bf16 or
    fp32), w [D, W] fp32 (W <= 4), bias [D] fp32, state [B, D, W-1] in x's dtype (the
    inputs before the sequence).  Returns y (and the final state when return_state)."""
    import torch
    if x.dim() != 3 or w.dim() != 2:
        raise ValueError("x must be [batch, seqlen, dim] and w [dim, width]")
    Bsz, L, Dm = x.shape
    W = w.shape[1]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("conv1d_fwd runs on the GPU only; tensors must be on a cuda device")
    _need(w, "w", (Dm, W), torch.float32, dev)
    _need(bias, "bias", (Dm,), torch.float32, dev)
    _need(state, "state", (Bsz, Dm, W - 1), x.dtype, dev)
    _need(x, "x", (Bsz, L, Dm), x.dtype, dev)
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", (Bsz, L, Dm), x.dtype, dev)
    st_out = torch.empty((Bsz, Dm, W - 1), dtype=x.dtype, device=dev) if return_state else None
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    _check(lib().ssm_conv1d_fwd(Bsz, L, Dm, W, _dtype_code(x), _ptr(x), _ptr(w), _ptr(bias), _ptr(state),
                                _ptr(out), _ptr(st_out), int(bool(silu)), ctypes.c_void_p(s.cuda_stream)),
           "ssm_conv1d_fwd")
    return (out, st_out) if return_state else out


def conv1d_bwd_workspace_bytes(batch, seqlen, dim, width, dtype="bf16") -> int:
    code = DTYPE_BF16 if dtype in ("bf16", "bfloat16") else DTYPE_F32
    return int(lib().ssm_conv1d_bwd_workspace_bytes(batch, seqlen, dim, width, code))


def conv1d_bwd(x, w, bias=None, state=None, dy=None, *, silu=True, need_dstate=None, workspace=None, stream=None):
    """Gradients of a loss through conv1d_fwd given dy = dLoss/dy [B, L, D] (x's dtype).
    Returns a dict: dx [B, L, D] (x's dtype), dw [D, W] fp32, dbias [D] fp32 (None without
    a bias) and dstate [B, D, W-1] (x's dtype; by default only when a state is given)."""
    import torch
    if x.dim() != 3 or w.dim() != 2:
        raise ValueError("x must be [batch, seqlen, dim] and w [dim, width]")
    Bsz, L, Dm = x.shape
    W = w.shape[1]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("conv1d_bwd runs on the GPU only; tensors must be on a cuda device")
    if dy is None:
        raise ValueError("dy is required")
    _need(w, "w", (Dm, W), torch.float32, dev)
    _need(bias, "bias", (Dm,), torch.float32, dev)
    _need(state, "state", (Bsz, Dm, W - 1), x.dtype, dev)
    _need(x, "x", (Bsz, L, Dm), x.dtype, dev)
    _need(dy, "dy", (Bsz, L, Dm), x.dtype, dev)
    if need_dstate is None:
        need_dstate = state is not None
    out = {"dx": torch.empty_like(x), "dw": torch.empty((Dm, W), dtype=torch.float32, device=dev),
           "dbias": torch.empty((Dm,), dtype=torch.float32, device=dev) if bias is not None else None,
           "dstate": torch.empty((Bsz, Dm, W - 1), dtype=x.dtype, device=dev) if need_dstate else None}
    code = _dtype_code(x)
    ws_bytes = int(lib().ssm_conv1d_bwd_workspace_bytes(Bsz, L, Dm, W, code))
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    _check(lib().ssm_conv1d_bwd(Bsz, L, Dm, W, code, _ptr(x), _ptr(w), _ptr(bias), _ptr(state), _ptr(dy),
                                _ptr(out["dx"]), _ptr(out["dw"]), _ptr(out["dbias"]), _ptr(out["dstate"]),
                                int(bool(silu)), _ptr(workspace) if ws_bytes else None, ws_bytes,
                                ctypes.c_void_p(s.cuda_stream)), "ssm_conv1d_bwd")
    return out


def causal_conv1d(x, w, bias=None, state=None, silu=True):
    """Differentiable causal depthwise convolution (+ SiLU): y = conv1d_fwd(...) with a
    torch autograd backward through conv1d_bwd (gradients for x, w, bias and state)."""
    import torch

    class _Conv(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, w, bias, state):
            y = conv1d_fwd(x, w, bias, state, silu=silu)
            ctx.save_for_backward(x, w, bias, state)
            return y

        @staticmethod
        def backward(ctx, gy):
            x, w, bias, state = ctx.saved_tensors
            g = conv1d_bwd(x, w, bias, state, gy.contiguous(), silu=silu,
                           need_dstate=state is not None and ctx.needs_input_grad[3])
            return g["dx"], g["dw"], g["dbias"], g["dstate"]

    return _Conv.apply(x, w, bias, state)


def conv1d_update(state, x, w, bias=None, *, silu=True, out=None, stream=None):
    """One token of conv1d_fwd: state [B, D, W-1] (x's dtype) updated in place, x [B, D];
    returns y [B, D]."""
    import torch
    if x.dim() != 2 or w.dim() != 2:
        raise ValueError("x must be [batch, dim] and w [dim, width]")
    Bsz, Dm = x.shape
    W = w.shape[1]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("conv1d_update runs on the GPU only; tensors must be on a cuda device")
    _need(w, "w", (Dm, W), torch.float32, dev)
    _need(bias, "bias", (Dm,), torch.float32, dev)
    _need(state, "state", (Bsz, Dm, W - 1), x.dtype, dev)
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", (Bsz, Dm), x.dtype, dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    _check(lib().ssm_conv1d_update(Bsz, Dm, W, _dtype_code(x), _ptr(state), _ptr(x), _ptr(w), _ptr(bias),
                                   _ptr(out), int(bool(silu)), ctypes.c_void_p(s.cuda_stream)),
           "ssm_conv1d_update")
    return out


def ssd_fwd(x, delta, A, B, C, D=None, z=None, h0=None, *, delta_softplus=False, delta_bias=None,
            return_last_state=False, out=None, h_last=None, stream=None):
    """Multi-head SSD scan (the Mamba-2 layer's state space model) on the GPU.

    x, z: [B, L, H, P];  delta: [B, L, H];  B, C: [B, L, N], or [B, L, G, N] for G groups
    of H / G consecutive heads each sharing one B and C row (all bf16, or all fp32);
    A, D, delta_bias: [H] fp32;  h0: [B, H, P, N] fp32.  P = 64, N = 128 in bf16 runs on the
    matrix cores; other P, N <= 256 and fp32 on the generic scan kernel.  Returns y
    [B, L, H, P] (x's dtype), or (y, h_last) when return_last_state.
    """
    import torch
    if x.dim() != 4 or A.dim() != 1:
        raise ValueError("x must be [batch, seqlen, nheads, headdim] and A [nheads]")
    Bsz, L, H, P = x.shape
    N = B.shape[-1]
    G = B.shape[2] if B.dim() == 4 else 1
    bc_shape = (Bsz, L, G, N) if B.dim() == 4 else (Bsz, L, N)
    dev, dt = x.device, x.dtype
    if dev.type != "cuda":
        raise ValueError("ssd_fwd runs on the GPU only; tensors must be on a cuda device")
    _need(delta, "delta", (Bsz, L, H), dt, dev)
    _need(z, "z", (Bsz, L, H, P), dt, dev)
    _need(B, "B", bc_shape, dt, dev)
    _need(C, "C", bc_shape, dt, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _need(D, "D", (H,), torch.float32, dev)
    _need(delta_bias, "delta_bias", (H,), torch.float32, dev)
    _need(h0, "h0", (Bsz, H, P, N), torch.float32, dev)
    code = _dtype_code(x)
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", (Bsz, L, H, P), dt, dev)
    if return_last_state and h_last is None:
        h_last = torch.empty((Bsz, H, P, N), dtype=torch.float32, device=dev)
    _need(h_last, "h_last", (Bsz, H, P, N), torch.float32, dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    st = lib().ssm_ssd_fwd(Bsz, L, H, P, N, G, code, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                           _ptr(z), _ptr(delta_bias), _ptr(h0), _ptr(h_last), _ptr(out),
                           int(bool(delta_softplus)), ctypes.c_void_p(s.cuda_stream))
    _check(st, "ssm_ssd_fwd")
    return (out, h_last) if return_last_state else out


def ssd_bwd_workspace_bytes(batch, seqlen, nheads, headdim, dstate, dtype="bf16") -> int:
    """Device workspace bytes of ssd_bwd for this shape (0: nothing to compute)."""
    code = DTYPE_BF16 if dtype in ("bf16", "bfloat16") else DTYPE_F32
    return int(lib().ssm_ssd_bwd_workspace_bytes(batch, seqlen, nheads, headdim, dstate, code))


def ssd_bwd(x, delta, A, B, C, D=None, z=None, h0=None, dy=None, dh_last=None, *, delta_softplus=False,
            delta_bias=None, workspace=None, stream=None):
    """Gradients of a loss through ssd_fwd (one B/C group: B, C [B, L, N]), given dy =
    dLoss/dy [B, L, H, P] (x's dtype) and optionally dh_last = dLoss/dh_last [B, H, P, N] fp32.

    Returns a dict: dx, dz (None without z) [B, L, H, P] and ddelta [B, L, H] and dB, dC
    [B, L, N] in x's dtype; dA, dD (None without D), ddelta_bias (None without a bias) [H] and
    dh0 [B, H, P, N] in fp32.
    """
    import torch
    if x.dim() != 4 or A.dim() != 1:
        raise ValueError("x must be [batch, seqlen, nheads, headdim] and A [nheads]")
    if B.dim() != 3:
        raise ValueError("ssd_bwd takes one B/C group: B and C [batch, seqlen, dstate]")
    Bsz, L, H, P = x.shape
    N = B.shape[-1]
    dev, dt = x.device, x.dtype
    if dev.type != "cuda":
        raise ValueError("ssd_bwd runs on the GPU only; tensors must be on a cuda device")
    if dy is None:
        raise ValueError("dy is required")
    for t, name, shape, tdt in ((delta, "delta", (Bsz, L, H), dt), (z, "z", (Bsz, L, H, P), dt),
                                (B, "B", (Bsz, L, N), dt), (C, "C", (Bsz, L, N), dt), (A, "A", (H,), torch.float32),
                                (D, "D", (H,), torch.float32), (delta_bias, "delta_bias", (H,), torch.float32),
                                (h0, "h0", (Bsz, H, P, N), torch.float32), (dy, "dy", (Bsz, L, H, P), dt),
                                (dh_last, "dh_last", (Bsz, H, P, N), torch.float32)):
        _need(t, name, shape, tdt, dev)
    code = _dtype_code(x)
    f32 = torch.float32
    out = {"dx": torch.empty_like(x), "ddelta": torch.empty((Bsz, L, H), dtype=dt, device=dev),
           "dz": torch.empty_like(x) if z is not None else None,
           "dB": torch.empty((Bsz, L, N), dtype=dt, device=dev), "dC": torch.empty((Bsz, L, N), dtype=dt, device=dev),
           "dA": torch.empty((H,), dtype=f32, device=dev),
           "dD": torch.empty((H,), dtype=f32, device=dev) if D is not None else None,
           "ddelta_bias": torch.empty((H,), dtype=f32, device=dev) if delta_bias is not None else None,
           "dh0": torch.empty((Bsz, H, P, N), dtype=f32, device=dev)}
    ws_bytes = int(lib().ssm_ssd_bwd_workspace_bytes(Bsz, L, H, P, N, code))
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    st = lib().ssm_ssd_bwd(Bsz, L, H, P, N, 1, code, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                           _ptr(z), _ptr(delta_bias), _ptr(h0), _ptr(dy), _ptr(dh_last), _ptr(out["dx"]),
                           _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]),
                           _ptr(out["dz"]), _ptr(out["ddelta_bias"]), _ptr(out["dh0"]), int(bool(delta_softplus)),
                           _ptr(workspace) if ws_bytes else None, ws_bytes, ctypes.c_void_p(s.cuda_stream))
    _check(st, "ssm_ssd_bwd")
    return out
