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
    and sampled (batch row, head) pairs match the oracle over the whole sequence."""
    import torch
    inp = synth.ssd_inputs(4, 4096, 64, 64, 128, "bf16", seed=7, gate=True)
    y, h = _run(ssm, inp)
    assert bool(torch.isfinite(y.float()).all())
    for b, hh in ((0, 0), (3, 63), (1, 37)):
        yr, hr = ssd_oracle.ssd_storage(inp, batches=[b], heads=[hh])
        st = assert_close(to_host(y[b:b + 1, :, hh:hh + 1]), yr, "bf16")
        assert_close(to_host(h[b:b + 1, hh:hh + 1]), hr, "f32", "h_last")
        print(f"[parity] ssd layer b={b} h={hh}: {json.dumps(st)}", flush=True)


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
    with pytest.raises(ssm.SSMError) as e:
        ssm.ssd_fwd(x, torch.zeros(1, 8, 2, dtype=torch.bfloat16, device="cuda"), torch.zeros(2, device="cuda"),
                    torch.zeros(1, 8, 128, dtype=torch.bfloat16, device="cuda"),
                    torch.zeros(1, 8, 128, dtype=torch.bfloat16, device="cuda"))
    assert e.value.status == ssm.SSM_EUNSUPPORTED


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
