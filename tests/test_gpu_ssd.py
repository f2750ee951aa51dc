"""GPU parity of the multi-head SSD scan (ssm_ssd_fwd, the Mamba-2 layer's state space
model on the matrix cores) against the fp64 oracle (MI355X only)."""
import json

import numpy as np
import pytest

import synth
from oracle import ssd_oracle
from tests.gpu_util import assert_close, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ssm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_50_amd as m
    m.lib()
    return m


def _dev(inp):
    import torch
    t = {k: to_dev(inp[k], "bf16") for k in ("x", "delta", "z", "B", "C")}
    for k in ("A", "Dskip", "delta_bias", "h0"):
        t[k] = None if inp.get(k) is None else torch.from_numpy(inp[k]).cuda()
    return t


def _run(ssm, inp):
    import torch
    t = _dev(inp)
    y, h = ssm.ssd_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["Dskip"], t["z"], t["h0"],
                       delta_softplus=inp["delta_softplus"], delta_bias=t["delta_bias"], return_last_state=True)
    torch.cuda.synchronize()
    return y, h


CASES = [
    # B, L, H, gate, h0, softplus, bias
    (1, 64, 1, False, False, False, False),
    (1, 1, 2, False, True, False, False),
    (2, 100, 3, True, True, False, False),
    (2, 300, 4, True, True, True, True),
    (1, 1000, 2, False, False, True, False),
    (3, 129, 5, True, False, False, True),
    (1, 4100, 1, True, True, True, False),
]


@pytest.mark.parametrize("Bsz,L,H,gate,h0,sp,bias", CASES)
def test_ssd_parity(ssm, Bsz, L, H, gate, h0, sp, bias):
    inp = synth.ssd_inputs(Bsz, L, H, 64, 128, "bf16", seed=900 + L + H, gate=gate, softplus_input=sp,
                           h0=h0, delta_bias=bias)
    y, h = _run(ssm, inp)
    yr, hr = ssd_oracle.ssd_storage(inp)
    st = assert_close(to_host(y), yr, "bf16")
    assert_close(to_host(h), hr, "f32", "h_last")
    print(f"[parity] ssd {Bsz}x{L}x{H}: {json.dumps(st)}", flush=True)


@pytest.mark.timeout(600)
def test_ssd_layer_shape_sampled(ssm):
    """B4 L4096 H64 (Mamba-2 layer of d_inner 4096), bf16, gated: every output is finite,
    and 68 (batch row, head) pairs (every row x heads 0, 4, ..., 60 and 63) match the
    oracle over the whole sequence, y and the final state."""
    import torch
    inp = synth.ssd_inputs(4, 4096, 64, 64, 128, "bf16", seed=7, gate=True)
    y, h = _run(ssm, inp)
    assert bool(torch.isfinite(y.float()).all())
    heads = list(range(0, 64, 4)) + [63]
    yr, hr = ssd_oracle.ssd_storage(inp, batches=[0, 1, 2, 3], heads=heads)
    st = assert_close(to_host(y[:, :, heads]), yr, "bf16")
    sth = assert_close(to_host(h[:, heads]), hr, "f32", "h_last")
    print(f"[parity] ssd layer, {4 * len(heads)} (b, h) pairs: {json.dumps(st)} {json.dumps(sth)}", flush=True)


def test_ssd_split_and_resume(ssm):
    """Two calls, the second started from the first one's final state, equal one call."""
    import torch
    inp = synth.ssd_inputs(2, 200, 3, 64, 128, "bf16", seed=11, gate=True, h0=True)
    t = _dev(inp)
    y, h = ssm.ssd_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["Dskip"], t["z"], t["h0"],
                       return_last_state=True)
    T = 77
    sl = lambda a: a[:, :T].contiguous()
    sr = lambda a: a[:, T:].contiguous()
    y1, h1 = ssm.ssd_fwd(sl(t["x"]), sl(t["delta"]), t["A"], sl(t["B"]), sl(t["C"]), t["Dskip"], sl(t["z"]),
                         t["h0"], return_last_state=True)
    y2, h2 = ssm.ssd_fwd(sr(t["x"]), sr(t["delta"]), t["A"], sr(t["B"]), sr(t["C"]), t["Dskip"], sr(t["z"]),
                         h1, return_last_state=True)
    torch.cuda.synchronize()
    assert_close(to_host(torch.cat([y1, y2], dim=1)), to_host(y), "bf16")
    assert_close(to_host(h2), to_host(h), "f32", "h_last")


def test_ssd_empty_and_errors(ssm):
    import torch
    inp = synth.ssd_inputs(2, 0, 3, 64, 128, "bf16", seed=12, h0=True)
    t = _dev(inp)
    y, h = ssm.ssd_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], None, None, t["h0"], return_last_state=True)
    torch.cuda.synchronize()
    assert y.numel() == 0 and torch.equal(h, t["h0"])
    x = torch.zeros(1, 8, 2, 32, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ssm.SSMError) as e:   # more than 256 states
        ssm.ssd_fwd(x, torch.zeros(1, 8, 2, dtype=torch.bfloat16, device="cuda"), torch.zeros(2, device="cuda"),
                    torch.zeros(1, 8, 300, dtype=torch.bfloat16, device="cuda"),
                    torch.zeros(1, 8, 300, dtype=torch.bfloat16, device="cuda"))
    assert e.value.status == ssm.SSM_EUNSUPPORTED


GENERIC = [
    # B, L, H, P, N, dtype, gate, h0, softplus, bias
    (2, 100, 3, 32, 64, "bf16", True, True, False, False),
    (1, 77, 2, 64, 128, "f32", True, True, True, True),
    (2, 50, 4, 16, 16, "bf16", False, True, False, True),
    (1, 40, 2, 128, 256, "f32", True, False, False, False),
    (2, 30, 3, 10, 7, "f32", True, True, True, False),
    (1, 65, 5, 64, 64, "bf16", True, False, False, False),
]


@pytest.mark.parametrize("Bsz,L,H,P,N,dt,gate,h0,sp,bias", GENERIC)
def test_ssd_generic_shapes(ssm, Bsz, L, H, P, N, dt, gate, h0, sp, bias):
    """Head dims and state sizes other than 64 / 128, and fp32: the generic scan kernel over
    the H * P channels with one step size, decay, D and bias per head; every output against
    the oracle."""
    inp = synth.ssd_inputs(Bsz, L, H, P, N, dt, seed=700 + L + P + N, gate=gate, softplus_input=sp, h0=h0,
                           delta_bias=bias)
    import torch
    t = {k: to_dev(inp[k], dt) for k in ("x", "delta", "z", "B", "C")}
    for k in ("A", "Dskip", "delta_bias", "h0"):
        t[k] = None if inp.get(k) is None else torch.from_numpy(inp[k]).cuda()
    y, h = ssm.ssd_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["Dskip"], t["z"], t["h0"],
                       delta_softplus=inp["delta_softplus"], delta_bias=t["delta_bias"], return_last_state=True)
    torch.cuda.synchronize()
    yr, hr = ssd_oracle.ssd_storage(inp)
    st = assert_close(to_host(y), yr, dt)
    assert_close(to_host(h), hr, "f32", "h_last")
    print(f"[parity] ssd generic {Bsz}x{L}x{H} P={P} N={N} {dt}: {json.dumps(st)}", flush=True)


def test_ssd_determinism(ssm):
    import torch
    inp = synth.ssd_inputs(2, 333, 4, 64, 128, "bf16", seed=13, gate=True, h0=True)
    y1, h1 = _run(ssm, inp)
    y2, h2 = _run(ssm, inp)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_ssd_degenerate_steps_and_decays(ssm):
    """A head with a = 0 (no decay), delta = 0 on whole steps and on one head (state held),
    and a large step, against the oracle."""
    inp = synth.ssd_inputs(2, 200, 4, 64, 128, "bf16", seed=63, gate=True, h0=True)
    d = synth.to_f64(inp["delta"], "bf16").copy()
    d[:, 50:70, :] = 0.0
    d[:, :, 3] = 0.0
    d[:, 120, 1] = 20.0
    inp["delta"] = synth.store(d.astype(np.float32), "bf16")
    A = inp["A"].copy()
    A[2] = 0.0
    inp["A"] = A
    y, h = _run(ssm, inp)
    yr, hr = ssd_oracle.ssd_storage(inp)
    st = assert_close(to_host(y), yr, "bf16")
    assert_close(to_host(h), hr, "f32", "h_last")
    print(f"[parity] ssd degenerate: {json.dumps(st)}", flush=True)


GROUPED = [
    # B, L, H, G, P, N, dtype, gate, h0, softplus, bias   (P = 64, N = 128, bf16: matrix cores)
    (2, 300, 4, 2, 64, 128, "bf16", True, True, False, False),
    (1, 200, 6, 3, 64, 128, "bf16", False, True, True, True),
    (2, 130, 8, 8, 64, 128, "bf16", True, False, False, False),
    (2, 100, 4, 2, 32, 64, "bf16", True, True, False, False),      # generic: 64 channels per group
    (1, 77, 4, 4, 64, 16, "f32", True, True, True, True),
    (2, 60, 8, 2, 16, 32, "f32", False, True, False, False),
]


@pytest.mark.parametrize("Bsz,L,H,G,P,N,dt,gate,h0,sp,bias", GROUPED)
def test_ssd_bc_groups(ssm, Bsz, L, H, G, P, N, dt, gate, h0, sp, bias):
    """B, C [B, L, G, N]: the heads of group g = h // (H / G) read group g's rows.  Every
    output against the oracle (which runs each group's heads with that group's B and C)."""
    import torch
    inp = synth.ssd_inputs(Bsz, L, H, P, N, dt, seed=1300 + L + G, gate=gate, softplus_input=sp, h0=h0,
                           delta_bias=bias, ngroups=G)
    t = {k: to_dev(inp[k], dt) for k in ("x", "delta", "z", "B", "C")}
    for k in ("A", "Dskip", "delta_bias", "h0"):
        t[k] = None if inp.get(k) is None else torch.from_numpy(inp[k]).cuda()
    y, h = ssm.ssd_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["Dskip"], t["z"], t["h0"],
                       delta_softplus=inp["delta_softplus"], delta_bias=t["delta_bias"], return_last_state=True)
    torch.cuda.synchronize()
    yr, hr = ssd_oracle.ssd_storage(inp)
    st = assert_close(to_host(y), yr, dt)
    assert_close(to_host(h), hr, "f32", "h_last")
    print(f"[parity] ssd {G} groups {Bsz}x{L}x{H} P={P} N={N} {dt}: {json.dumps(st)}", flush=True)


def test_ssd_bc_groups_errors(ssm):
    import torch
    bf = torch.bfloat16
    x = torch.zeros(1, 8, 4, 32, dtype=bf, device="cuda")
    d = torch.zeros(1, 8, 4, dtype=bf, device="cuda")
    A = torch.zeros(4, device="cuda")
    with pytest.raises(ssm.SSMError) as e:   # 3 groups do not divide 4 heads
        bc = torch.zeros(1, 8, 3, 64, dtype=bf, device="cuda")
        ssm.ssd_fwd(x, d, A, bc, bc)
    assert e.value.status == ssm.SSM_EINVAL
    with pytest.raises(ssm.SSMError) as e:   # generic kernel: a group of 32 channels
        bc = torch.zeros(1, 8, 4, 64, dtype=bf, device="cuda")
        ssm.ssd_fwd(x, d, A, bc, bc)
    assert e.value.status == ssm.SSM_EUNSUPPORTED


@pytest.mark.timeout(600)
def test_ssd_layer_shape_with_groups_sampled(ssm):
    """B4 L4096 H64 with 8 groups of 8 heads (matrix cores): 20 (batch row, head) pairs that
    cover every group, over the whole sequence."""
    import torch
    inp = synth.ssd_inputs(4, 4096, 64, 64, 128, "bf16", seed=17, gate=True, ngroups=8)
    y, h = _run(ssm, inp)
    assert bool(torch.isfinite(y.float()).all())
    heads = [0, 7, 9, 18, 27, 36, 45, 54, 63, 62]
    yr, hr = ssd_oracle.ssd_storage(inp, batches=[0, 3], heads=heads)
    st = assert_close(to_host(y[[0, 3]][:, :, heads]), yr, "bf16")
    assert_close(to_host(h[[0, 3]][:, heads]), hr, "f32", "h_last")
    print(f"[parity] ssd layer, 8 groups: {json.dumps(st)}", flush=True)


SSD_BWD = [
    # B, L, H, P, N, dtype, gate, h0, dh_last, softplus, bias
    (2, 40, 3, 8, 16, "f32", True, True, True, False, False),
    (1, 70, 4, 16, 32, "bf16", True, False, True, True, True),
    (2, 33, 2, 64, 128, "bf16", True, True, True, True, True),
    (1, 20, 5, 7, 20, "f32", False, True, False, False, True),
]


@pytest.mark.parametrize("Bsz,L,H,P,N,dt,gate,h0,dhl,sp,bias", SSD_BWD)
def test_ssd_backward_matches_oracle(ssm, Bsz, L, H, P, N, dt, gate, h0, dhl, sp, bias):
    """ssm_ssd_bwd (the scan backward on the per-channel expansion, tied gradients summed per
    head) against the SSD backward oracle, on every output."""
    import torch
    from tests.gpu_util import assert_close_grad
    seed = 700 + L + H + P + N
    inp = synth.ssd_inputs(Bsz, L, H, P, N, dt, seed=seed, gate=gate, softplus_input=sp, h0=h0, delta_bias=bias)
    r = np.random.default_rng(seed + 1)
    gy = synth.store(r.standard_normal((Bsz, L, H, P)).astype(np.float32), dt)
    gl = r.standard_normal((Bsz, H, P, N)).astype(np.float32) if dhl else None
    t = {k: to_dev(inp[k], dt) if inp.get(k) is not None else None for k in ("x", "delta", "z", "B", "C")}
    f = {k: None if inp.get(k) is None else torch.from_numpy(np.asarray(inp[k], dtype=np.float32)).cuda()
         for k in ("A", "Dskip", "delta_bias", "h0")}
    g = ssm.ssd_bwd(t["x"], t["delta"], f["A"], t["B"], t["C"], f["Dskip"], t["z"], f["h0"], to_dev(gy, dt),
                    None if gl is None else torch.from_numpy(gl).cuda(), delta_softplus=sp,
                    delta_bias=f["delta_bias"])
    torch.cuda.synchronize()
    ref = ssd_oracle.ssd_bwd_storage(inp, gy, gl)
    worst = {}
    for k in ("dx", "ddelta", "dz", "dB", "dC"):
        if ref[k] is None:
            assert g[k] is None, k
            continue
        worst[k] = assert_close_grad(to_host(g[k]), ref[k], dt, f"ssd bwd {k}")
    for k in ("dA", "dD", "dh0", "ddelta_bias"):
        if ref[k] is None:
            assert g[k] is None, k
            continue
        worst[k] = assert_close_grad(to_host(g[k]), ref[k], "f32", f"ssd bwd {k}")
    print(f"[parity] ssd backward {Bsz}x{L}x{H}x{P} N={N} {dt}: " +
          ", ".join(f"{k} {v:.3f}" for k, v in worst.items()), flush=True)


def test_ssd_backward_deterministic_and_edges(ssm):
    """Two calls give bit-identical gradients; no steps gives zero parameter gradients and
    dh0 = dh_last; several B/C groups are SSM_EUNSUPPORTED."""
    import torch
    inp = synth.ssd_inputs(1, 50, 2, 16, 32, "bf16", seed=9, gate=True, h0=True)
    t = {k: to_dev(inp[k], "bf16") for k in ("x", "delta", "z", "B", "C")}
    A = torch.from_numpy(inp["A"]).cuda()
    Dk = torch.from_numpy(inp["Dskip"]).cuda()
    h0 = torch.from_numpy(inp["h0"]).cuda()
    gy = torch.randn(t["x"].shape, device="cuda").to(torch.bfloat16)
    a = ssm.ssd_bwd(t["x"], t["delta"], A, t["B"], t["C"], Dk, t["z"], h0, gy)
    b = ssm.ssd_bwd(t["x"], t["delta"], A, t["B"], t["C"], Dk, t["z"], h0, gy)
    torch.cuda.synchronize()
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k
    x0 = t["x"][:, :0].contiguous()
    hl = torch.randn(h0.shape, device="cuda")
    e = ssm.ssd_bwd(x0, t["delta"][:, :0].contiguous(), A, t["B"][:, :0].contiguous(), t["C"][:, :0].contiguous(),
                    Dk, None, None, x0, hl)
    torch.cuda.synchronize()
    assert torch.equal(e["dh0"], hl) and float(e["dA"].abs().sum()) == 0.0 and float(e["dD"].abs().sum()) == 0.0
    L_ = t["x"].shape[1]
    Bg = torch.zeros((1, L_, 2, 32), device="cuda", dtype=torch.bfloat16)
    outs = [torch.empty_like(t["x"]), torch.empty((1, L_, 2), device="cuda", dtype=torch.bfloat16),
            torch.empty(2, device="cuda"), torch.empty((1, L_, 2, 32), device="cuda", dtype=torch.bfloat16),
            torch.empty((1, L_, 2, 32), device="cuda", dtype=torch.bfloat16)]
    P_ = ssm._ptr
    st = ssm.lib().ssm_ssd_bwd(1, L_, 2, 16, 32, 2, 1, P_(t["x"]), P_(t["delta"]), P_(A), P_(Bg), P_(Bg), None, None,
                               None, None, P_(gy), None, *[P_(o) for o in outs], None, None, None, None, 0, None, 0,
                               None)
    assert st == ssm.SSM_EUNSUPPORTED   # two B/C groups
