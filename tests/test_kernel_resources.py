"""Occupancy budgets of the specialised scan kernel, read from the compiler's kernel
metadata (the sources are compiled to gfx950 assembly here; no GPU needed).

The planner runs four states per lane (G = 4) when a launch has more than one
workgroup per CU, counting on two workgroups sharing each CU: that needs at most half
of the CU's 160 KiB of LDS and, with 2 x 8 waves on 4 SIMDs, at most 128 VGPRs per
lane.  With two states per lane (13 waves, one workgroup per CU) the limits are the
whole LDS and again 128 VGPRs (four waves on the busiest SIMD)."""
import os
import re
import shutil
import subprocess

import pytest

from selective_state_space_50_amd import build_lib

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _kernels(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    flags = [f for f in build_lib.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [HIPCC, *flags, "--cuda-device-only", "-S", "-I", build_lib.INCLUDE, "-I", build_lib.CSRC,
           os.path.join(build_lib.CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    text = out.read_text()
    meta = text[text.index("amdhsa.kernels:"):]
    res = {}
    for entry in re.split(r"\n  - ", meta)[1:]:
        f = dict(re.findall(r"^\s+\.(name|group_segment_fixed_size|vgpr_count|vgpr_spill_count):\s+(\S+)",
                            entry, re.M))
        if "name" in f:
            res[f["name"]] = {k: int(v) for k, v in f.items() if k != "name"}
    return res


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="no hipcc")
@pytest.mark.parametrize("src,disc", [("scan_fast.hip", 0), ("scan_fast_zoh.hip", 1)])
def test_scan_kernel_occupancy_budgets(tmp_path, src, disc):
    ks = _kernels(src, tmp_path)
    # scan_fast_kernel<DISC, T, G, HAS_Z, CARRY, CKPT>: the forward (CARRY = CKPT = false)
    pat = re.compile(r"scan_fast_kernelILi%dE([tf])Li([24])ELb([01])ELb0ELb0E" % disc)
    seen = 0
    for name, r in ks.items():
        m = pat.search(name)
        if not m:
            continue
        seen += 1
        g = int(m.group(2))
        lds_cap = 80 * 1024 if g == 4 else 160 * 1024
        assert r["group_segment_fixed_size"] <= lds_cap, (name, r)
        assert r["vgpr_count"] <= 128, (name, r)
        assert r.get("vgpr_spill_count", 0) == 0, (name, r)
    assert seen == 8, sorted(ks)


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="no hipcc")
def test_ssd_kernel_register_budget(tmp_path):
    """The matrix-core SSD kernel runs 16 waves per workgroup (four per SIMD), so at most 128
    VGPRs per lane; none of its instantiations may spill vector registers to scratch (a
    runtime B/C row stride once did, and cost 14% of the launch)."""
    ks = _kernels("ssd.hip", tmp_path)
    seen = 0
    for name, r in ks.items():
        if "ssd_kernel" not in name:
            continue
        seen += 1
        assert r["vgpr_count"] <= 128, (name, r)
        assert r.get("vgpr_spill_count", 0) == 0, (name, r)
    assert seen == 4, sorted(ks)


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="no hipcc")
def test_backward_sweep_register_budget(tmp_path):
    """The reverse sweep runs 8 waves per workgroup, one workgroup per CU (two waves per SIMD,
    at most 256 VGPRs); no instantiation, for any discretisation, may spill to scratch."""
    ks = _kernels("scan_bwd.hip", tmp_path)
    seen = 0
    for name, r in ks.items():
        if "scan_bwd_kernel" not in name:
            continue
        seen += 1
        assert r["vgpr_count"] <= 256, (name, r)
        assert r.get("vgpr_spill_count", 0) == 0, (name, r)
    assert seen == 12, sorted(ks)
