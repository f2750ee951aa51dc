"""The C-ABI library on the CPU: it loads, exports what include/ssm.h declares,
and its host layer rejects bad arguments without launching anything."""
import ctypes
import os
import subprocess

import pytest

import selective_state_space_50_amd as ssm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "selective_state_space_50_amd", "csrc")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssm.LIB_PATH):
        pytest.skip("libssm.so not built")
    return ssm.lib()


def test_exports_every_declared_symbol(lib):
    names = ssm.exported_api()
    assert {"ssm_scan_fwd", "ssm_state_update", "ssm_scan_workspace_bytes", "ssm_scan_plan_get",
            "ssm_status_str", "ssm_last_error", "ssm_abi_version"} <= set(names)
    raw = ctypes.CDLL(ssm.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_version_and_status_text(lib):
    assert lib.ssm_abi_version() == 7
    assert lib.ssm_status_str(0) == b"ok"
    assert lib.ssm_status_str(3) == b"workspace too small"


def test_plans(lib):
    p2 = ssm.scan_plan(4, 4096, 4096, 16, "bf16")
    # one 64-channel block per CU: two compute waves per SIMD with 2 states per lane
    assert p2["n_chunks"] == 1 and p2["states_per_lane"] == 2 and p2["waves_per_block"] == 13
    p8 = ssm.scan_plan(8, 4096, 4096, 16, "bf16")
    assert p8["states_per_lane"] == 4 and p8["waves_per_block"] == 8
    assert p2["blocks"] == 4 * 64 and p2["specialised"] == 1
    assert ssm.scan_plan(2, 100, 130, 16, "bf16")["specialised"] == 0
    assert ssm.scan_plan(2, 100, 128, 12, "bf16")["specialised"] == 0
    assert p2["workspace_bytes"] == 4 * 4096 * 16 * 2 * 4   # packed B/C rows
    p3 = ssm.scan_plan(1, 1 << 20, 1024, 16, "bf16")
    assert p3["n_chunks"] > 1 and p3["workspace_bytes"] > 0
    assert ssm.scan_workspace_bytes(1, 1 << 20, 1024, 16, "bf16") == p3["workspace_bytes"]
    assert ssm.scan_plan(2, 100, 64, 16, "f32", chunk_len=30)["n_chunks"] == 4


G4 = 1 << 32   # fake device addresses 4 GiB apart; never dereferenced


def _scan_status(lib, *, B=1, L=8, D=64, N=16, dtype=1, x=G4, y=2 * G4, ws=None,
                 ws_bytes=0, opts=None, softplus=0, variant=None):
    base = 1 << 40
    V = ctypes.c_void_p
    return lib.ssm_scan_fwd(B, L, D, N, dtype, V(base + x), V(base + 3 * G4), V(base + 4 * G4),
                            V(base + 5 * G4), V(base + 6 * G4), None, None, None, None,
                            V(base + y) if y is not None else None, softplus,
                            ctypes.byref(variant) if variant else None,
                            ctypes.byref(opts) if opts else None, ws, ws_bytes, None)


def test_validation_rejects_before_launch(lib):
    assert _scan_status(lib, dtype=5) == 1
    assert _scan_status(lib, N=257) == 2
    assert _scan_status(lib, N=0) == 1
    assert _scan_status(lib, B=-1) == 1
    assert _scan_status(lib, y=None) == 1
    assert b"NULL" in lib.ssm_last_error()
    assert _scan_status(lib, x=G4 + 2) == 1
    assert b"aligned" in lib.ssm_last_error()
    assert _scan_status(lib, y=G4 + 16) == 1
    assert b"overlaps" in lib.ssm_last_error()
    assert _scan_status(lib, softplus=3) == 1
    assert _scan_status(lib, L=4096, opts=ssm.ScanOpts(128, 0, 0, 0, 0)) == 3
    assert _scan_status(lib, L=16, D=64) == 3        # packed B/C rows need a workspace
    assert _scan_status(lib, opts=ssm.ScanOpts(0, 3, 0, 0, 0)) == 1
    assert _scan_status(lib, opts=ssm.ScanOpts(0, 0, 0, 0, 7)) == 1
    # discretisation variants: bad enum, nonzero reserved word, misaligned delta bias
    assert _scan_status(lib, variant=ssm.Variant(3, 0, None)) == 1
    assert _scan_status(lib, variant=ssm.Variant(1, 1, None)) == 1
    assert _scan_status(lib, variant=ssm.Variant(2, 0, (1 << 40) + 7 * G4 + 4)) == 1
    assert b"delta_bias" in lib.ssm_last_error()
    V = ctypes.c_void_p
    assert lib.ssm_state_update(4, 64, 16, 1, None, V(1 << 40), V(1 << 41), V(1 << 42), V(1 << 43),
                                V(1 << 44), None, None, V(1 << 45), 0, None, None) == 1
    assert lib.ssm_state_update(4, 64, 16, 1, V(1 << 39), V(1 << 40), V(1 << 41), V(1 << 42),
                                V(1 << 43), V(1 << 44), None, None, V(1 << 45), 0,
                                ctypes.byref(ssm.Variant(7, 0, None)), None) == 1


def test_binding_refuses_cpu_tensors(lib):
    import torch
    x = torch.zeros(1, 4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ssm.scan_fwd(x, x, torch.zeros(8, 4), torch.zeros(1, 4, 4, dtype=torch.bfloat16),
                     torch.zeros(1, 4, 4, dtype=torch.bfloat16))


def test_product_path_never_touches_the_oracle():
    """The package and its sources name no oracle module."""
    pkg = os.path.join(ROOT, "selective_state_space_50_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "liboracle" not in text, f


def test_host_checks_under_sanitizers(tmp_path):
    exe = tmp_path / "check_host"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "host", "check_host.cpp"), os.path.join(CSRC, "ssm_host.cpp"),
           "-o", str(exe)]
    subprocess.run(cmd, check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok: 0 failure(s)" in r.stdout


def test_ssm_log_prints_the_plan():
    """SSM_LOG=1: every call says on stderr what it launches (the launch itself fails here,
    without a GPU, after the line is printed); unset, nothing is printed."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import tests.test_abi_host as t, selective_state_space_50_amd as ssm; "
            "print(t._scan_status(ssm.lib(), D=65, N=8))")
    env = {k: v for k, v in os.environ.items() if k not in ("SSM_LOG", "SSM_SYNC")}
    on = subprocess.run([sys.executable, "-c", code], env={**env, "SSM_LOG": "1"}, cwd=root,
                        capture_output=True, text=True, timeout=300)
    assert "[ssm] scan B=1 L=8 D=65 N=8 dtype=1 disc=0: generic kernel" in on.stderr, on.stderr[-2000:]
    off = subprocess.run([sys.executable, "-c", code], env=env, cwd=root, capture_output=True, text=True,
                         timeout=300)
    assert "[ssm]" not in off.stderr
