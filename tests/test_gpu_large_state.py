"""GPU parity of the scan and the single-token update with more than 16 states per channel
(the generic kernel with 16 states per lane in up to 16 waves; the update with up to 64
lanes per channel) against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import assert_close, device_inputs, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ssm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_50_amd as m
    m.lib()
    return m


LARGE = [
    # B, L, D, N, dtype, gate, h0, softplus, A kind, discretisation
    (1, 40, 64, 17, "f32", True, True, False, "random", "mamba"),
    (2, 100, 70, 32, "bf16", True, False, False, "mamba", "mamba"),
    (1, 65, 128, 64, "f32", False, True, True, "random", "zoh"),
    (2, 50, 130, 100, "bf16", True, True, False, "random", "bilinear"),
    (1, 33, 64, 128, "f32", True, True, False, "mamba", "mamba"),
    (1, 20, 96, 256, "f32", True, True, False, "random", "mamba"),
    (2, 9, 5, 200, "bf16", False, True, False, "random", "zoh"),
    (1, 12, 70, 255, "f32", True, True, False, "random", "mamba"),
]


@pytest.mark.parametrize("Bsz,L,D,N,dt,gate,h0,sp,ak,disc", LARGE)
def test_scan_more_than_16_states(ssm, Bsz, L, D, N, dt, gate, h0, sp, ak, disc):
    import torch
    inp = synth.scan_inputs(Bsz, L, D, N, dt, seed=500 + L + N, gate=gate, d_kind="normal", a_kind=ak,
                            softplus_input=sp, h0=h0)
    inp["discretization"] = disc
    plan = ssm.scan_plan(Bsz, L, D, N, dt)
    assert plan["specialised"] == 0 and plan["states_per_lane"] == 16 and plan["n_chunks"] == 1
    t = device_inputs(inp)
    y, h = ssm.scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"],
                        delta_softplus=sp, discretization=disc, return_last_state=True)
    torch.cuda.synchronize()
    yr, hr = oracle.scan(inp)
    st = assert_close(to_host(y), yr, dt)
    assert_close(to_host(h), hr, "f32", "h_last")
    print(f"[parity] {N} states {Bsz}x{L}x{D} {dt} {disc}: worst ratio {st['worst_ratio']:.3f}", flush=True)


@pytest.mark.parametrize("N,chunk", [(64, 30), (256, 7)])
def test_scan_more_than_16_states_chunked(ssm, N, chunk):
    """A requested chunk length: chunk carries of the 16-states-per-lane kernel, their
    combine, then every chunk from its carried-in state."""
    import torch
    inp = synth.scan_inputs(2, 100, 64, N, "f32", seed=600 + N, gate=True, d_kind="normal", a_kind="random",
                            h0=True)
    t = device_inputs(inp)
    y, h = ssm.scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"],
                        return_last_state=True, chunk_len=chunk)
    torch.cuda.synchronize()
    yr, hr = oracle.scan(inp)
    assert_close(to_host(y), yr, "f32")
    assert_close(to_host(h), hr, "f32", "h_last")


@pytest.mark.parametrize("Bsz,D,N,dt", [(2, 70, 32, "f32"), (3, 64, 64, "bf16"), (1, 33, 256, "f32"),
                                        (2, 128, 100, "bf16"), (2, 40, 130, "f32"), (1, 65, 255, "bf16"),
                                        (2, 10, 37, "f32")])
def test_state_update_more_than_16_states(ssm, Bsz, D, N, dt):
    import torch
    A = synth.make_A(7, D, N, "random")
    Dk = synth.make_D(7, D, "normal")
    h = torch.from_numpy(synth.make_h0(7, Bsz, D, N)).cuda()
    h_ref = synth.make_h0(7, Bsz, D, N).astype(np.float64)
    At, Dt = torch.from_numpy(A).cuda(), torch.from_numpy(Dk).cuda()
    for s in range(6):
        step = synth.decode_step_inputs(7, s, Bsz, D, N, dt)
        t = {k: to_dev(step[k], dt) for k in ("x", "delta", "z", "B", "C")}
        y = ssm.state_update(h, t["x"], t["delta"], At, t["B"], t["C"], Dt, t["z"])
        torch.cuda.synchronize()
        h_ref, y_ref = oracle.state_update(h_ref, step, A, Dk, dt)
        assert_close(to_host(y), y_ref, dt)
        assert_close(to_host(h), h_ref, "f32", "h")


def test_scan_more_than_16_states_with_delta_bias(ssm):
    """A per-channel step-size bias (before the softplus) with 48 states, all three maps."""
    import torch
    for disc in ("mamba", "zoh", "bilinear"):
        inp = synth.scan_inputs(2, 60, 70, 48, "f32", seed=650, gate=True, d_kind="normal", a_kind="random",
                                softplus_input=True, h0=True)
        inp["discretization"] = disc
        inp["delta_bias"] = synth.make_delta_bias(650, 70)
        t = device_inputs(inp)
        y, h = ssm.scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"],
                            delta_softplus=True, discretization=disc,
                            delta_bias=torch.from_numpy(inp["delta_bias"]).cuda(), return_last_state=True)
        torch.cuda.synchronize()
        yr, hr = oracle.scan(inp)
        assert_close(to_host(y), yr, "f32", f"y {disc}")
        assert_close(to_host(h), hr, "f32", f"h_last {disc}")


def test_more_than_256_states_rejected(ssm):
    import torch
    x = torch.zeros((1, 4, 64), device="cuda")
    with pytest.raises(ssm.SSMError) as e:
        ssm.scan_fwd(x, x, torch.zeros((64, 257), device="cuda"), torch.zeros((1, 4, 257), device="cuda"),
                     torch.zeros((1, 4, 257), device="cuda"))
    assert e.value.status == ssm.SSM_EUNSUPPORTED
