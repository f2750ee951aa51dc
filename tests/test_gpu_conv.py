"""GPU parity of ssm_conv1d_fwd / ssm_conv1d_update against the fp64 convolution oracle."""
import numpy as np
import pytest

import synth
from oracle.conv_oracle import conv1d, conv1d_update
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


def _inputs(Bsz, L, D, W, dt, seed):
    r = np.random.default_rng(seed)
    x = synth.store(r.standard_normal((Bsz, L, D)).astype(np.float32), dt)
    st = synth.store(r.standard_normal((Bsz, D, W - 1)).astype(np.float32), dt)
    w = (r.standard_normal((D, W)) * 0.5).astype(np.float32)
    bias = (r.standard_normal(D) * 0.1).astype(np.float32)
    return x, st, w, bias


CASES = [
    # B, L, D, W, dtype, bias, state_in, silu
    (1, 1, 4, 4, "f32", False, False, True),
    (2, 37, 64, 4, "bf16", True, True, True),
    (3, 100, 130, 3, "f32", True, False, True),
    (2, 5, 12, 2, "bf16", False, True, False),
    (1, 70, 256, 1, "bf16", True, False, True),
    (2, 33, 64, 4, "f32", True, True, False),
    (1, 2, 8, 4, "bf16", True, True, True),
    (2, 1000, 1536, 4, "bf16", True, True, True),
]


@pytest.mark.parametrize("Bsz,L,D,W,dt,use_bias,use_state,silu", CASES)
def test_conv_parity(ssm, Bsz, L, D, W, dt, use_bias, use_state, silu):
    import torch
    x, st, w, bias = _inputs(Bsz, L, D, W, dt, seed=L + D + W)
    y, so = ssm.conv1d_fwd(to_dev(x, dt), torch.from_numpy(w).cuda(),
                           torch.from_numpy(bias).cuda() if use_bias else None,
                           to_dev(st, dt) if use_state else None, silu=silu, return_state=True)
    torch.cuda.synchronize()
    yr, sr = conv1d(synth.to_f64(x, dt), w, bias if use_bias else None,
                    synth.to_f64(st, dt) if use_state else None, silu)
    assert_close(to_host(y), yr, dt, "conv y")
    assert np.array_equal(to_host(so), sr), "state_out is the last inputs, bit for bit"


def test_conv_empty_sequence_passes_state(ssm):
    import torch
    x, st, w, _ = _inputs(2, 0, 8, 4, "bf16", seed=1)
    y, so = ssm.conv1d_fwd(to_dev(x, "bf16"), torch.from_numpy(w).cuda(), None, to_dev(st, "bf16"),
                           return_state=True)
    torch.cuda.synchronize()
    assert y.numel() == 0 and np.array_equal(to_host(so), synth.to_f64(st, "bf16"))


@pytest.mark.parametrize("dt,W", [("bf16", 4), ("f32", 3), ("bf16", 1)])
def test_updates_equal_forward(ssm, dt, W):
    import torch
    Bsz, L, D = 3, 20, 96
    x, st, w, bias = _inputs(Bsz, L, D, W, dt, seed=5)
    wt, bt = torch.from_numpy(w).cuda(), torch.from_numpy(bias).cuda()
    xd = to_dev(x, dt)
    y, so = ssm.conv1d_fwd(xd, wt, bt, to_dev(st, dt), return_state=True)
    state = to_dev(st, dt).clone()
    ys = [ssm.conv1d_update(state, xd[:, t].contiguous(), wt, bt) for t in range(L)]
    torch.cuda.synchronize()
    assert torch.equal(torch.stack(ys, dim=1), y)
    assert torch.equal(state, so)
    yr, sr = conv1d(synth.to_f64(x, dt), w, bias, synth.to_f64(st, dt))
    assert_close(to_host(y), yr, dt, "conv y")


def test_conv_errors(ssm):
    import torch
    x = torch.zeros((1, 4, 8), device="cuda")
    with pytest.raises(ssm.SSMError) as e:
        ssm.conv1d_fwd(x, torch.zeros((8, 5), device="cuda"))
    assert e.value.status == ssm.SSM_EUNSUPPORTED
    with pytest.raises(ssm.SSMError) as e:
        ssm.conv1d_fwd(x, torch.zeros((8, 4), device="cuda"), out=x)   # y overlaps x
    assert e.value.status == ssm.SSM_EINVAL


@pytest.mark.timeout(600)
def test_conv_headline_shape_full(ssm):
    """x [4, 4096, 4096] bf16, width 4, bias, SiLU (the layer shape the bench times), no
    carried state: every output against the fp64 oracle."""
    import torch
    x, _, w, bias = _inputs(4, 4096, 4096, 4, "bf16", seed=4096)
    y = ssm.conv1d_fwd(to_dev(x, "bf16"), torch.from_numpy(w).cuda(), torch.from_numpy(bias).cuda())
    torch.cuda.synchronize()
    yr, _ = conv1d(synth.to_f64(x, "bf16"), w, bias, None, True)
    st = assert_close(to_host(y), yr, "bf16", "conv y (headline shape)")
    print(f"[parity] conv1d headline shape: {st}", flush=True)


# ---- backward ---------------------------------------------------------------------

from oracle.conv_oracle import conv1d_bwd  # noqa: E402
from tests.gpu_util import assert_close_grad  # noqa: E402

BWD_CASES = [
    # B, L, D, W, dtype, bias, state_in, silu   (tiles of 64 steps; D % 4 != 0 takes one channel per thread)
    (1, 1, 4, 4, "f32", True, True, True),
    (2, 64, 64, 4, "bf16", True, False, True),
    (2, 130, 96, 4, "f32", True, True, True),
    (1, 3, 8, 4, "bf16", False, True, True),        # shorter than the filter
    (3, 200, 130, 3, "f32", True, True, False),
    (2, 65, 12, 2, "bf16", False, False, True),
    (1, 100, 256, 1, "f32", True, False, True),
    (2, 1000, 1536, 4, "bf16", True, True, True),
]


def _bwd_run(ssm, x, st, w, bias, dy, dt, use_bias, use_state, silu):
    import torch
    g = ssm.conv1d_bwd(to_dev(x, dt), torch.from_numpy(w).cuda(), torch.from_numpy(bias).cuda() if use_bias else None,
                       to_dev(st, dt) if use_state else None, to_dev(dy, dt), silu=silu, need_dstate=True)
    torch.cuda.synchronize()
    return {k: None if v is None else to_host(v) for k, v in g.items()}


@pytest.mark.parametrize("Bsz,L,D,W,dt,use_bias,use_state,silu", BWD_CASES)
def test_conv_bwd_parity(ssm, Bsz, L, D, W, dt, use_bias, use_state, silu):
    x, st, w, bias = _inputs(Bsz, L, D, W, dt, seed=7 * L + D + W)
    dy = synth.store(np.random.default_rng(L + 1).standard_normal((Bsz, L, D)).astype(np.float32), dt)
    g = _bwd_run(ssm, x, st, w, bias, dy, dt, use_bias, use_state, silu)
    r = conv1d_bwd(synth.to_f64(x, dt), w, bias if use_bias else None, synth.to_f64(st, dt) if use_state else None,
                   synth.to_f64(dy, dt), silu)
    worst = {"dx": assert_close_grad(g["dx"], r["dx"], dt, "conv dx"),
             "dw": assert_close_grad(g["dw"], r["dw"], "f32", "conv dw")}
    if use_bias:
        worst["dbias"] = assert_close_grad(g["dbias"], r["dbias"], "f32", "conv dbias")
    else:
        assert g["dbias"] is None
    if W > 1:
        worst["dstate"] = assert_close_grad(g["dstate"], r["dstate"], dt, "conv dstate")
    print(f"[parity] conv1d backward {Bsz}x{L}x{D} W={W} {dt}: " + ", ".join(f"{k} {v:.3f}" for k, v in worst.items()),
          flush=True)


def test_conv_bwd_empty_sequence(ssm):
    import torch
    x = torch.zeros((2, 0, 8), dtype=torch.bfloat16, device="cuda")
    w = torch.ones((8, 4), device="cuda")
    g = ssm.conv1d_bwd(x, w, torch.ones(8, device="cuda"), None, x, need_dstate=True)
    torch.cuda.synchronize()
    assert float(g["dw"].abs().sum()) == 0.0 and float(g["dbias"].abs().sum()) == 0.0
    assert float(g["dstate"].float().abs().sum()) == 0.0
    # no rows: dw and dbias are written as zeros
    x0 = torch.zeros((0, 6, 8), dtype=torch.bfloat16, device="cuda")
    g = ssm.conv1d_bwd(x0, w, torch.ones(8, device="cuda"), None, x0)
    torch.cuda.synchronize()
    assert float(g["dw"].abs().sum()) == 0.0 and float(g["dbias"].abs().sum()) == 0.0


@pytest.mark.timeout(600)
def test_conv_bwd_headline_shape_full(ssm):
    """x [4, 4096, 4096] bf16, width 4, bias, SiLU: every element of dx, and dw, dbias,
    against the fp64 oracle."""
    x, _, w, bias = _inputs(4, 4096, 4096, 4, "bf16", seed=4097)
    dy = synth.store(np.random.default_rng(4098).standard_normal((4, 4096, 4096), dtype=np.float32), "bf16")
    g = _bwd_run(ssm, x, None, w, bias, dy, "bf16", True, False, True)
    r = conv1d_bwd(synth.to_f64(x, "bf16"), w, bias, None, synth.to_f64(dy, "bf16"), True)
    worst = {"dx": assert_close_grad(g["dx"], r["dx"], "bf16", "headline conv dx"),
             "dw": assert_close_grad(g["dw"], r["dw"], "f32", "headline conv dw"),
             "dbias": assert_close_grad(g["dbias"], r["dbias"], "f32", "headline conv dbias")}
    print("[parity] conv1d backward headline shape: " + ", ".join(f"{k} {v:.3f}" for k, v in worst.items()), flush=True)


def test_causal_conv1d_autograd(ssm):
    import torch
    x, st, w, bias = _inputs(2, 150, 64, 4, "f32", seed=5)
    dy = np.random.default_rng(6).standard_normal((2, 150, 64)).astype(np.float32)
    leaves = {"x": torch.from_numpy(x).cuda(), "w": torch.from_numpy(w).cuda(), "bias": torch.from_numpy(bias).cuda(),
              "state": torch.from_numpy(st).cuda()}
    leaves = {k: v.clone().requires_grad_(True) for k, v in leaves.items()}
    y = ssm.causal_conv1d(leaves["x"], leaves["w"], leaves["bias"], leaves["state"], silu=True)
    (y * torch.from_numpy(dy).cuda()).sum().backward()
    r = conv1d_bwd(x, w, bias, st, dy, True)
    for k, rk in (("x", "dx"), ("w", "dw"), ("bias", "dbias"), ("state", "dstate")):
        assert_close_grad(to_host(leaves[k].grad), r[rk], "f32", f"autograd conv {k}")
