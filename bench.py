#!/usr/bin/env python3
"""Throughput of the MI355X selective scan: one JSON line on stdout.

Headline workload (a "step"): one selective scan of the Mamba-1.4B-layer
shape B=4, L=4096, D=4096, N=16, bf16 inputs/outputs, fp32 state,
z-gated, with the inputs already resident in HBM.  metric = state updates
per second (B*L*D*N per step).

Also reported in the same line:
  roofline      -- the scan kernel against its binding roofline (VALU issue
                   slots; the HBM fraction is given beside it), from HIP events
                   around every timed launch;
  cpu_baseline  -- the fp64 C oracle on this same input, on the host cores;
  secondary     -- the decode state update (1024 steps of h[256,4096,16]) and
                   the million-token chunked scan (B1 L1048576 D1024 N16).

Options: --gpus N (only 1 is supported), --steps K, --warmup W,
--no-cpu-baseline, --no-secondary, --profile-run (short run for rocprofv3),
--copy-calibration MiB (also run a plain torch copy of that size, for
counter calibration).
"""
from __future__ import annotations

import argparse
import hashlib
import math
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFS = 2500.0   # dense bf16 matrix-core peak
# VALU issue slots per second with packed FP32 off: 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz
VALU_PEAK_TSLOTS = 256 * 4 * 16 * 2.4e9 / 1e12


def slot_model(x_exp, x_rcp):
    """Algorithmic VALU issue slots, with a v_exp_f32 costing x_exp and a v_rcp_f32 x_rcp FMA
    slots (both measured by ssm_issue_probe at run time).

    per state update, Mamba form, general A: mul (delta*A), exp, mul (delta*x*B), fma (state),
        fma (readout) = 4 + x_exp; the structured-A path (what A = -(n+1) takes): half an exp
        and half a mul per update (one per lane and step, two states), one mul by E, and the
        three others = 4 + x_exp / 2, plus E staged once per (t, d): mul + exp;
    per (b, t, d): delta*x, D*x fma, gate (mul, exp, add, rcp, mul, mul) = 6 + x_exp + x_rcp
        (ungated: 2);
    zero-order hold: mul, exp, fma ((e - 1) / A), mul (x*B), mul (by the factor), fma, fma
        = 6 + x_exp (the series branch and its select are accuracy work, not counted);
    bilinear: fma (1 - delta*A/2), rcp, mul (delta*x*B), fma (2h + .), fma (r * . - h), fma
        (readout) = 5 + x_rcp;
    backward: checkpoint pass (mul, exp, mul, fma), recompute (the same + readout fma), adjoint
        (fma, mul, mul, fma, mul, mul + fma for the A term, mul + fma for dA, mul = 10) and the
        sums of the dB, dC terms over channels (2) = 19 + 2 x_exp."""
    return {"update": 4.0 + x_exp, "update_structured": 4.0 + x_exp / 2.0, "e_stage": 1.0 + x_exp,
            "token_gated": 6.0 + x_exp + x_rcp, "token": 2.0,
            "zoh": 6.0 + x_exp, "bilinear": 5.0 + x_rcp, "bwd": 19.0 + 2.0 * x_exp}


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_50_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".cpp", ".h")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def time_calls(torch, fn, n):
    """n calls of fn queued back to back, each between two events on the current stream,
    and one synchronisation at the end (a synchronisation after every call lets the GPU
    idle between calls, and a call that starts on an idle GPU runs slower).  Returns the
    per-call times in ms, sorted."""
    ev = []
    for _ in range(n):
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        fn()
        b_.record()
        ev.append((a_, b_))
    torch.cuda.synchronize()
    return sorted(a_.elapsed_time(b_) for a_, b_ in ev)


def settle_calls(torch, fn, ms=50.0):
    """Untimed calls of fn for about ms of GPU time (at least two): the GPU runs a workload
    slower for its first ~25 ms after the host work between workloads."""
    fn()
    torch.cuda.synchronize()
    a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a_.record()
    fn()
    b_.record()
    torch.cuda.synchronize()
    n = max(1, int(ms / max(a_.elapsed_time(b_), 1e-3)))
    for _ in range(n):
        fn()
    torch.cuda.synchronize()


def load_traffic(name, src_hash):
    """HBM bytes per launch measured by rocprofv3 counters (profiles/counters.json),
    only while the kernel sources are unchanged since they were taken."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(name)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def scan_bytes(B, L, D, N, esz, gated):
    tok = B * L * D * esz
    return tok * (3 + (1 if gated else 0)) + 2 * B * L * N * esz + D * N * 4 + D * 4


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle", type=int, default=100, metavar="LAUNCHES",
                    help="untimed flushed scan launches before the warmup steps: the first ~50 launches "
                         "of a fresh process run up to 15%% slower while the GPU settles")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--profile-run", action="store_true",
                    help="few steps, no CPU baseline, no secondary (for rocprofv3)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB")
    ap.add_argument("--secondary-only", action="store_true")
    ap.add_argument("--profile-decode", type=int, default=0, metavar="STEPS",
                    help="only run this many decode steps of h[256,4096,16] (for rocprofv3)")
    ap.add_argument("--profile-conv", type=int, default=0, metavar="CALLS",
                    help="only run this many conv1d calls at the headline shape (for rocprofv3)")
    ap.add_argument("--profile-bwd", type=int, default=0, metavar="CALLS",
                    help="only run this many backward calls at the headline shape (for rocprofv3)")
    ap.add_argument("--profile-ssd", type=int, default=0, metavar="CALLS",
                    help="only run this many SSD (Mamba-2 layer) scans (for rocprofv3)")
    ap.add_argument("--profile-ssd-bwd", type=int, default=0, metavar="CALLS",
                    help="only run this many SSD backward calls (for rocprofv3)")
    ap.add_argument("--profile-long", type=int, default=0, metavar="CALLS",
                    help="only run this many million-token scans (B1 L1048576 D1024 N16 bf16; for rocprofv3)")
    ap.add_argument("--profile-decode-graph", type=int, default=0, metavar="REPLAYS",
                    help="only replay the 1024-step decode graph this many times (for rocprofv3)")
    ap.add_argument("--profile-variant", choices=("zoh", "bilinear"), default=None,
                    help="with --profile-run: time this discretisation instead of the Mamba one")
    ap.add_argument("--profile-general", action="store_true",
                    help="with --profile-run: time the general-A path (one exp per state update)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU (every kernel works on one device's share); run with --gpus 1",
                          "requested_gpus": args.gpus}), flush=True)
        sys.exit(2)
    if args.profile_run:
        args.no_cpu_baseline = True
        args.no_secondary = True

    import numpy as np
    import torch

    import selective_state_space_50_amd as ssm
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    ssm.lib()
    src_hash = kernel_source_hash()

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copy calibration: {args.copy_calibration} MiB copied 3 times")

    if args.profile_decode:
        profile_decode(torch, ssm, synth, dev, args.profile_decode)
        log(f"decode profile run: {args.profile_decode} steps")
        return
    if args.profile_long:
        x, dl, A, Bm, Cm, Dk, y, ws = _long_inputs(torch, ssm, synth, dev)
        for _ in range(args.profile_long):
            ssm.scan_fwd(x, dl, A, Bm, Cm, Dk, out=y, workspace=ws)
        torch.cuda.synchronize()
        log(f"million-token profile run: {args.profile_long} calls")
        return
    if args.profile_decode_graph:
        run = _decode_graph(torch, ssm, synth, dev)
        for _ in range(args.profile_decode_graph):
            run()
        torch.cuda.synchronize()
        log(f"decode graph profile run: {args.profile_decode_graph} replays of 1024 steps")
        return
    if args.profile_bwd:
        c = synth.CONFIGS["mamba1p4b_layer"]
        gen = torch.Generator(device=dev)
        gen.manual_seed(4)
        bf = torch.bfloat16
        Bsz, L, D, N = c["batch"], c["seqlen"], c["dim"], c["dstate"]
        x, dl, z, gy = (_randn((Bsz, L, D), gen, dev, bf) if k != "dl" else _delta((Bsz, L, D), gen, dev, bf)
                        for k in ("x", "dl", "z", "gy"))
        Bm, Cm = _randn((Bsz, L, N), gen, dev, bf), _randn((Bsz, L, N), gen, dev, bf)
        A = torch.from_numpy(synth.make_A(2, D, N)).to(dev)
        Dk = torch.from_numpy(synth.make_D(2, D, "normal")).to(dev)
        ws = torch.empty(ssm.scan_bwd_workspace_bytes(Bsz, L, D, N, "bf16"), dtype=torch.uint8, device=dev)
        for _ in range(args.profile_bwd):
            ssm.scan_bwd(x, dl, A, Bm, Cm, Dk, z, None, gy, workspace=ws, need_dh0=False)
        torch.cuda.synchronize()
        log(f"backward profile run: {args.profile_bwd} calls")
        return
    if args.profile_ssd:
        t = _ssd_inputs(torch, dev)
        for _ in range(args.profile_ssd):
            ssm.ssd_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], out=t["y"])
        torch.cuda.synchronize()
        log(f"ssd profile run: {args.profile_ssd} calls")
        return
    if args.profile_ssd_bwd:
        t = _ssd_inputs(torch, dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(6)
        gys = _randn(tuple(t["x"].shape), gen, dev, torch.bfloat16)
        sws = torch.empty(ssm.ssd_bwd_workspace_bytes(*t["x"].shape, t["B"].shape[-1], "bf16"), dtype=torch.uint8,
                          device=dev)
        for _ in range(args.profile_ssd_bwd):
            ssm.ssd_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], None, gys, workspace=sws)
        torch.cuda.synchronize()
        log(f"ssd backward profile run: {args.profile_ssd_bwd} calls")
        return
    if args.profile_conv:
        x, w, bias = _conv_inputs(torch, synth, dev)
        for _ in range(args.profile_conv):
            ssm.conv1d_fwd(x, w, bias)
        torch.cuda.synchronize()
        log(f"conv1d profile run: {args.profile_conv} calls")
        return

    result = {}
    cfg = synth.CONFIGS["mamba1p4b_layer"]
    B, L, D, N = cfg["batch"], cfg["seqlen"], cfg["dim"], cfg["dstate"]
    updates = B * L * D * N
    if not args.secondary_only:
        t0 = time.time()
        inp = synth.config_inputs("mamba1p4b_layer")
        log(f"generated {cfg['name']} inputs in {time.time() - t0:.1f}s")

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

        x, dl, z, Bm, Cm = (up(inp[k]) for k in ("x", "delta", "z", "B", "C"))
        A = torch.from_numpy(inp["A"]).to(dev)
        Dk = torch.from_numpy(inp["Dskip"]).to(dev)
        y = torch.empty_like(x)
        plan = ssm.scan_plan(B, L, D, N, "bf16")
        ws = None
        if plan["workspace_bytes"]:
            ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device=dev)

        disc = args.profile_variant if args.profile_run and args.profile_variant else "mamba"

        def step(general=False):
            ssm.scan_fwd(x, dl, A, Bm, Cm, Dk, z, out=y, workspace=ws, discretization=disc, general_a=general)

        # Issue rates of this GPU (fp32 FMA, v_exp_f32, v_rcp_f32): a transcendental costs
        # fma_rate / its rate issue slots in the slot model of the roofline.
        rates = ssm.issue_rates()
        x_exp = rates["fma"] / rates["exp"]
        x_rcp = rates["fma"] / rates["rcp"]
        log(f"issue rates: fma {rates['fma']:.3e}, exp {rates['exp']:.3e}, rcp {rates['rcp']:.3e} lane-ops/s "
            f"-> exp {x_exp:.2f}, rcp {x_rcp:.2f} FMA slots")
        # Each timed launch follows an untimed 1 GiB write that evicts the L2s and the 256 MB
        # Infinity Cache, so every launch reads its inputs from HBM.
        flush = None if args.profile_run else torch.empty(1 << 30, dtype=torch.uint8, device=dev)

        def timed(n, general=False, flushed=True, read_flush=False):
            ms = []
            for _ in range(n):
                if flushed and flush is not None:
                    if read_flush:
                        flush.view(torch.int64).amax()   # evicts by reading: leaves no dirty lines
                    else:
                        flush.fill_(1)
                a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a_.record()
                step(general)
                b_.record()
                ms.append((a_, b_))
            torch.cuda.synchronize()
            return sorted(a_.elapsed_time(b_) for a_, b_ in ms)

        # Settle: a fresh process's first ~50 flushed launches run up to 15% slower than the
        # ones after them (285 -> 267 -> 252 us in successive groups of 25 on one MI355X, flat
        # from there over 400 launches), so the timed launches follow that many untimed ones
        # under the same flushed protocol, then the warmup steps.  (A profiling run settles too,
        # on the path it profiles, so that its trace's later dispatches are the settled ones.)
        for _ in range(args.settle):
            if flush is not None:
                flush.fill_(1)
            step(args.profile_run and args.profile_general)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        steps = args.steps
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        kms = timed(steps, general=args.profile_run and args.profile_general)
        elapsed = time.perf_counter() - t_start
        k_med = kms[len(kms) // 2]
        k_min = kms[0]
        k_avg = sum(kms) / len(kms)
        ms_per_step = k_med
        value = updates / (k_med * 1e-3)
        alg_bytes = scan_bytes(B, L, D, N, 2, True)
        # algorithmic VALU slots: the structured-A path (what runs on this A = -(n+1)) takes one
        # exp per lane and step for two states and one multiply for the other, plus E staged
        # once per (t, d); the general path one exp per state update
        spu_struct = 4.0 + x_exp / 2.0
        spu_general = 4.0 + x_exp
        per_td = 6.0 + x_exp + x_rcp            # delta*x, D*x, the gate (mul, exp, add, rcp, mul, mul)
        alg_slots = updates * spu_struct + B * L * D * (per_td + 1.0 + x_exp)
        alg_slots_general = updates * spu_general + B * L * D * per_td
        hbm_gbs = alg_bytes / (k_med * 1e-3) / 1e9
        alu_tslots = alg_slots / (k_med * 1e-3) / 1e12
        traffic = load_traffic("scan_B4_L4096_D4096_N16_bf16_gated", src_hash)
        roofline = {"bound": "alu", "achieved": round(alu_tslots, 3), "peak": round(VALU_PEAK_TSLOTS, 3),
                    "unit": "Tslot/s", "frac": round(alu_tslots / VALU_PEAK_TSLOTS, 4),
                    "traffic": traffic,
                    "kernel": "scan_fast_kernel<mamba, bf16, G=%d, gated> + bc_pack" % plan["states_per_lane"],
                    "path": "structured A (one exp per lane and step)",
                    "kernel_ms_median": round(k_med, 5), "kernel_ms_min": round(k_min, 5),
                    "kernel_ms_avg": round(k_avg, 5),
                    "alg_slots_per_launch": alg_slots, "alg_bytes_per_launch": alg_bytes,
                    "slot_model": {"exp_slots_measured": round(x_exp, 3), "rcp_slots_measured": round(x_rcp, 3),
                                   "slots_per_update": round(spu_struct, 3),
                                   "slots_per_token_channel": round(per_td + 1.0 + x_exp, 3),
                                   "issue_rates_lane_ops_per_s": {k: float("%.4g" % v) for k, v in rates.items()}},
                    "hbm": {"achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(hbm_gbs / HBM_PEAK_GBS, 4)}}
        log(f"scan (flushed): {k_med * 1e3:.1f} us/launch median ({k_min * 1e3:.1f} min), {value:.3e} updates/s, "
            f"HBM {hbm_gbs:.0f} GB/s ({hbm_gbs / HBM_PEAK_GBS:.1%}), VALU {alu_tslots / VALU_PEAK_TSLOTS:.1%}")
        result.update({
            "metric": "state-updates/s (B*L*D*N), scan B4 L4096 D4096 N16",
            "value": value, "unit": "state-updates/s", "n_gpus": 1, "steps": steps,
            "warmup": args.warmup, "settle_launches": args.settle,
            "ms_per_step": ms_per_step, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "dtype_note": "the arithmetic and the state are fp32; x, delta, z, B, C and y are stored as bf16",
            "timing": "median of the timed launches, each between two events on the launch stream and each "
                      "after an untimed 1 GiB write (L2 and Infinity Cache evicted); value = B*L*D*N / median; "
                      "before the warmup steps, settle_launches untimed launches under the same protocol",
            "data": "synthetic (seeded generator: x,z,B,C ~ N(0,1), delta log-uniform [1e-3,1e-1], "
                    "A=-(n+1), D ~ N(1,0.1))",
            "config": {"workload": cfg["name"], "batch": B, "seqlen": L, "dim": D, "dstate": N,
                       "io_dtype": "bf16", "state_dtype": "f32", "gate": True, "plan": plan},
            "hbm_frac": round(hbm_gbs / HBM_PEAK_GBS, 4),
            "roofline": roofline,
            "source_hash": src_hash,
        })
        if not args.profile_run:
            # the general path (one exp per state: what a trained, unstructured A takes), and the
            # warm figure: launches back to back, nothing evicted in between
            gms = timed(steps, general=True)
            g_med = gms[len(gms) // 2]
            wms = timed(steps, flushed=False)
            w_med = wms[len(wms) // 2]
            rms = timed(steps, read_flush=True)
            r_med = rms[len(rms) // 2]
            dst = torch.empty_like(flush)
            cp = []
            for _ in range(5):
                a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a_.record()
                dst.copy_(flush)
                b_.record()
                torch.cuda.synchronize()
                cp.append(a_.elapsed_time(b_))
            copy_gbs = 2 * (1 << 30) / (min(cp) * 1e-3) / 1e9
            result_extra = {
                "general_a_path": {
                    "kernel_ms_median": round(g_med, 5), "state_updates_per_s": updates / (g_med * 1e-3),
                    "roofline": {"bound": "alu", "achieved": round(alg_slots_general / (g_med * 1e-3) / 1e12, 3),
                                 "peak": round(VALU_PEAK_TSLOTS, 3), "unit": "Tslot/s",
                                 "frac": round(alg_slots_general / (g_med * 1e-3) / 1e12 / VALU_PEAK_TSLOTS, 4),
                                 "slots_per_update": round(spu_general, 3),
                                 "hbm_frac": round(alg_bytes / (g_med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
                    "note": "ssm_scan_opts.a_structure = -1: one exp per state update, the path any A without "
                            "the structure takes; same flushed protocol"},
                "warm": {"kernel_ms_median": round(w_med, 5), "state_updates_per_s": updates / (w_med * 1e-3),
                         "note": "launches back to back, no eviction in between"},
                "read_flushed": {"kernel_ms_median": round(r_med, 5), "state_updates_per_s": updates / (r_med * 1e-3),
                                 "note": "each launch after an untimed 1 GiB read instead of the write: caches "
                                         "evicted without leaving dirty lines to write back"},
                "copy_probe": {"GB/s": round(copy_gbs, 1), "note": "1 GiB device-to-device copy, read + write bytes"}}
            log(f"general path (flushed): {g_med * 1e3:.1f} us median; warm: {w_med * 1e3:.1f} us median; "
                f"read-flushed: {r_med * 1e3:.1f} us median; "
                f"copy probe {copy_gbs:.0f} GB/s")
            del flush, dst
        else:
            result_extra = {}
        result.update(result_extra)
        del x, dl, z, Bm, Cm, y

        if not args.no_cpu_baseline:
            import oracle
            cores = oracle.default_threads()
            w = lambda a: synth.to_f64(a, "bf16")
            t0 = time.time()
            ch_b = np.repeat(np.arange(B), D)
            ch_d = np.tile(np.arange(D), B)
            xs = w(inp["x"]).transpose(0, 2, 1).reshape(B * D, L)
            ds = w(inp["delta"]).transpose(0, 2, 1).reshape(B * D, L)
            zs = w(inp["z"]).transpose(0, 2, 1).reshape(B * D, L)
            Bw, Cw = w(inp["B"]), w(inp["C"])
            log(f"oracle inputs widened in {time.time() - t0:.1f}s; timing the oracle on {cores} threads")
            t0 = time.perf_counter()
            oracle.scan_f64(xs, ds, inp["A"], Bw, Cw, inp["Dskip"], zs, None, False, ch_b, ch_d,
                            nthreads=cores)
            t_cpu = time.perf_counter() - t0
            result["cpu_baseline"] = {
                "value": updates / t_cpu, "unit": "state-updates/s", "cores": cores, "kind": "oracle",
                "sample": f"the whole headline input (all {B * D} channels x {L} steps, "
                          f"{updates:.3e} updates), fp64 C oracle, {t_cpu:.2f} s wall",
                "cpu": platform.processor() or platform.machine()}
            log(f"oracle: {t_cpu:.2f}s on {cores} threads -> {updates / t_cpu:.3e} updates/s")
            del xs, ds, zs

    if not args.no_secondary:
        if args.secondary_only:
            rates = ssm.issue_rates()
        sm = slot_model(rates["fma"] / rates["exp"], rates["fma"] / rates["rcp"])
        result["secondary"] = secondary(torch, ssm, synth, dev, log, src_hash, sm)

    print(json.dumps(result), flush=True)


def _host(t):
    """A (sampled) device tensor as float64 on the host (bf16 and fp32 values are exact)."""
    import numpy as np
    return t.float().cpu().numpy().astype(np.float64)


def _cpu_entry(seconds, work, unit, sample, cores):
    return {"value": work / seconds, "unit": unit, "cores": cores, "kind": "oracle", "seconds": round(seconds, 3),
            "sample": sample}


def _timed(fn):
    t0 = time.perf_counter()
    fn()
    return time.perf_counter() - t0


def _randn(shape, gen, dev, dtype):
    import torch
    return torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).to(dtype)


def _delta(shape, gen, dev, dtype):
    import math
    import torch
    u = torch.rand(shape, generator=gen, device=dev, dtype=torch.float32)
    lo, hi = math.log(1e-3), math.log(1e-1)
    return torch.exp(lo + (hi - lo) * u).to(dtype)


def _conv_inputs(torch, synth, dev):
    """Headline-shape input of the convolution: x [4, 4096, 4096] bf16, width-4 filter."""
    c = synth.CONFIGS["mamba1p4b_layer"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    x = _randn((c["batch"], c["seqlen"], c["dim"]), gen, dev, torch.bfloat16)
    w = torch.randn((c["dim"], 4), generator=gen, device=dev) * 0.5
    bias = torch.randn((c["dim"],), generator=gen, device=dev) * 0.1
    return x, w, bias


SSD_SHAPE = dict(batch=4, seqlen=4096, nheads=64, headdim=64, dstate=128)


def _ssd_inputs(torch, dev):
    """Mamba-2 layer SSD scan input: x, z [4, 4096, 64, 64] bf16, delta [4, 4096, 64],
    B, C [4, 4096, 128], A [64] = -exp(U[0, log 16]), D [64] ~ N(1, 0.1)."""
    c = SSD_SHAPE
    Bsz, L, H, P, N = c["batch"], c["seqlen"], c["nheads"], c["headdim"], c["dstate"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(9)
    bf = torch.bfloat16
    t = {"x": _randn((Bsz, L, H, P), gen, dev, bf), "z": _randn((Bsz, L, H, P), gen, dev, bf),
         "delta": _delta((Bsz, L, H), gen, dev, bf), "B": _randn((Bsz, L, N), gen, dev, bf),
         "C": _randn((Bsz, L, N), gen, dev, bf),
         "A": -torch.exp(torch.rand((H,), generator=gen, device=dev) * math.log(16.0)),
         "D": 1.0 + 0.1 * torch.randn((H,), generator=gen, device=dev)}
    t["y"] = torch.empty_like(t["x"])
    return t


def ssd_alg(c, Q=64):
    """Algorithmic work of one SSD scan call: HBM bytes (x, z, y once each, delta, B, C, A,
    D) and matrix-core flops of the chunked form with chunk Q: per chunk and head, the
    masked C B^T (lower triangle incl. diagonal, Q(Q+1)/2 entries of length N), its product
    with x, the carried state's readout C S^T and the state update (Q*N*P each)."""
    Bsz, L, H, P, N = c["batch"], c["seqlen"], c["nheads"], c["headdim"], c["dstate"]
    byts = 3 * Bsz * L * H * P * 2 + Bsz * L * H * 2 + 2 * Bsz * L * N * 2 + 2 * H * 4
    tri = Q * (Q + 1) // 2
    per_chunk = 2 * tri * N + 2 * tri * P + 2 * Q * N * P + 2 * Q * N * P
    flops = Bsz * H * ((L + Q - 1) // Q) * per_chunk
    return byts, flops


def profile_decode(torch, ssm, synth, dev, steps):
    """A few decode steps on the decode workload's state (h [256, 4096, 16] fp32)."""
    c = synth.CONFIGS["decode"]
    Bsz, D, N = c["batch"], c["dim"], c["dstate"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)
    bf = torch.bfloat16
    A = torch.from_numpy(synth.make_A(4, D, N)).to(dev)
    Dk = torch.from_numpy(synth.make_D(4, D, "normal")).to(dev)
    h = torch.zeros((Bsz, D, N), device=dev)
    y = torch.empty((Bsz, D), dtype=bf, device=dev)
    for s in range(steps):
        x, dl, z = _randn((Bsz, D), gen, dev, bf), _delta((Bsz, D), gen, dev, bf), _randn((Bsz, D), gen, dev, bf)
        Bm, Cm = _randn((Bsz, N), gen, dev, bf), _randn((Bsz, N), gen, dev, bf)
        ssm.state_update(h, x, dl, A, Bm, Cm, Dk, z, out=y)
    torch.cuda.synchronize()


def _long_inputs(torch, ssm, synth, dev):
    """The million-token layer's input (B1 L1048576 D1024 N16 bf16), drawn on the GPU."""
    c = synth.CONFIGS["million_token"]
    Bsz, L, D, N = c["batch"], c["seqlen"], c["dim"], c["dstate"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    bf = torch.bfloat16
    x, dl = _randn((Bsz, L, D), gen, dev, bf), _delta((Bsz, L, D), gen, dev, bf)
    Bm, Cm = _randn((Bsz, L, N), gen, dev, bf), _randn((Bsz, L, N), gen, dev, bf)
    A = torch.from_numpy(synth.make_A(3, D, N)).to(dev)
    Dk = torch.from_numpy(synth.make_D(3, D, "normal")).to(dev)
    ws = torch.empty(max(ssm.scan_plan(Bsz, L, D, N, "bf16")["workspace_bytes"], 1), dtype=torch.uint8, device=dev)
    return x, dl, A, Bm, Cm, Dk, torch.empty_like(x), ws


def _decode_graph(torch, ssm, synth, dev):
    """A HIP graph of the decode workload's 1024 gated steps on h [256, 4096, 16] fp32 from
    zero; returns a function that zeroes h and replays it."""
    c = synth.CONFIGS["decode"]
    Bsz, D, N, S = c["batch"], c["dim"], c["dstate"], c["seqlen"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)
    bf = torch.bfloat16
    A = torch.from_numpy(synth.make_A(4, D, N)).to(dev)
    Dk = torch.from_numpy(synth.make_D(4, D, "normal")).to(dev)
    xs, ds, zs = _randn((S, Bsz, D), gen, dev, bf), _delta((S, Bsz, D), gen, dev, bf), _randn((S, Bsz, D), gen, dev, bf)
    Bs, Cs = _randn((S, Bsz, N), gen, dev, bf), _randn((S, Bsz, N), gen, dev, bf)
    h = torch.zeros((Bsz, D, N), device=dev)
    y = torch.empty((Bsz, D), dtype=bf, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ssm.state_update(h, xs[0], ds[0], A, Bs[0], Cs[0], Dk, zs[0], out=y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s in range(S):
            ssm.state_update(h, xs[s], ds[s], A, Bs[s], Cs[s], Dk, zs[s], out=y)
    keep = (xs, ds, zs, Bs, Cs, A, Dk, y)

    def run():
        h.zero_()
        graph.replay()
        return keep
    return run


def secondary(torch, ssm, synth, dev, log, src_hash, sm):
    """Decode (1024 steps) and the million-token chunked scan.  Inputs drawn on the
    GPU with torch's seeded generator, same distributions as the headline input."""
    out = {}
    deferred = []   # (entry, oracle call, work, unit, sample, threads), timed at the end
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)
    bf = torch.bfloat16
    # --- decode: h[256, 4096, 16] fp32, 1024 gated steps from zero ---
    c = synth.CONFIGS["decode"]
    Bsz, D, N, S = c["batch"], c["dim"], c["dstate"], c["seqlen"]
    A = torch.from_numpy(synth.make_A(4, D, N)).to(dev)
    Dk = torch.from_numpy(synth.make_D(4, D, "normal")).to(dev)
    xs = _randn((S, Bsz, D), gen, dev, bf)
    ds = _delta((S, Bsz, D), gen, dev, bf)
    zs = _randn((S, Bsz, D), gen, dev, bf)
    Bs = _randn((S, Bsz, N), gen, dev, bf)
    Cs = _randn((S, Bsz, N), gen, dev, bf)
    h = torch.zeros((Bsz, D, N), device=dev)
    y = torch.empty((Bsz, D), dtype=bf, device=dev)

    def run_decode():
        h.zero_()
        for s in range(S):
            ssm.state_update(h, xs[s], ds[s], A, Bs[s], Cs[s], Dk, zs[s], out=y)

    run_decode()
    torch.cuda.synchronize()
    # Eager launches from Python are host-bound here (the binding's checks take longer
    # than a step), so the step is timed from a HIP graph of the whole 1024-step loop,
    # the way a serving loop would replay it.  The eager time is reported beside it.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    h.zero_()
    torch.cuda.synchronize()
    e0.record()
    run_decode_steps = lambda: [ssm.state_update(h, xs[s], ds[s], A, Bs[s], Cs[s], Dk, zs[s], out=y)
                                for s in range(S)]
    run_decode_steps()
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ssm.state_update(h, xs[0], ds[0], A, Bs[0], Cs[0], Dk, zs[0], out=y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_decode_steps()
    reps = []
    for _ in range(5):   # (the first replays also settle the GPU after the host work before them)
        h.zero_()
        torch.cuda.synchronize()
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        reps.append(e0.elapsed_time(e1))
    tot_ms = min(reps)
    k_avg = tot_ms / S
    del graph
    step_bytes = Bsz * D * N * 8 + Bsz * D * 2 * 4 + 2 * Bsz * N * 2 + D * N * 4 + D * 4
    out["decode"] = {
        "workload": c["name"], "tokens_per_s": Bsz * S / (tot_ms * 1e-3),
        "state_updates_per_s": Bsz * D * N * S / (tot_ms * 1e-3), "ms_total": tot_ms,
        "roofline": {"bound": "hbm", "achieved": round(step_bytes / (k_avg * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(step_bytes / (k_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic("state_update_B256_D4096_N16_bf16_gated", src_hash),
                     "kernel_us_avg": round(k_avg * 1e3, 2), "alg_bytes_per_launch": step_bytes},
        "timing": "HIP graph of the 1024-step loop, best of 5 replays; per-step = replay / 1024",
        "eager_ms_total": round(eager_ms, 2),
        "note": "h (67 MB) fits the 256 MB Infinity Cache, so steps after the first can beat HBM",
    }
    log(f"decode: {tot_ms:.2f} ms for {S} steps from a graph ({k_avg * 1e3:.1f} us/step); "
        f"eager from Python {eager_ms:.2f} ms")
    import numpy as np
    import oracle
    from oracle import conv_oracle, ssd_oracle
    cores = oracle.default_threads()
    # oracle beside it: every batch row, every 64th channel, the first 128 steps (L steps
    # of the update from zero = one scan over those L tokens)
    Ss, dsel = 1024, torch.arange(0, D, 64, device=dev)
    ser = lambda t: _host(t[:Ss][:, :, dsel].permute(1, 2, 0)).reshape(Bsz * len(dsel), Ss)
    cb = np.repeat(np.arange(Bsz), len(dsel))
    cd = np.tile(np.arange(len(dsel)), Bsz)
    # (host copies now; every oracle timing runs after the last GPU measurement, so that
    # the GPU does not idle between them)
    a_ = (ser(xs), ser(ds), _host(A[dsel]), _host(Bs[:Ss].permute(1, 0, 2)), _host(Cs[:Ss].permute(1, 0, 2)),
          _host(Dk[dsel]), ser(zs), None, False, cb, cd, cores)
    deferred.append((out["decode"], lambda a_=a_: oracle.scan_f64(*a_), Bsz * len(dsel) * Ss * N, "state-updates/s",
                     f"{Bsz * len(dsel)} channels (every 64th) x all {Ss} steps, fp64 C oracle", cores))
    del xs, ds, zs, Bs, Cs, h
    torch.cuda.empty_cache()
    # --- the other discretisations at the headline shape ---
    c = synth.CONFIGS["mamba1p4b_layer"]
    Bsz, L, D, N = c["batch"], c["seqlen"], c["dim"], c["dstate"]
    x, dl, z = (_randn((Bsz, L, D), gen, dev, bf) if k != "dl" else _delta((Bsz, L, D), gen, dev, bf)
                for k in ("x", "dl", "z"))
    Bm = _randn((Bsz, L, N), gen, dev, bf)
    Cm = _randn((Bsz, L, N), gen, dev, bf)
    A = torch.from_numpy(synth.make_A(2, D, N)).to(dev)
    Dk = torch.from_numpy(synth.make_D(2, D, "normal")).to(dev)
    y = torch.empty_like(x)
    ws = torch.empty(max(ssm.scan_plan(Bsz, L, D, N, "bf16")["workspace_bytes"], 1), dtype=torch.uint8,
                     device=dev)
    out["variants"] = {}
    for disc in ("zoh", "bilinear"):
        settle_calls(torch, lambda disc=disc: ssm.scan_fwd(x, dl, A, Bm, Cm, Dk, z, out=y, workspace=ws,
                                                           discretization=disc))
        vt = time_calls(torch, lambda disc=disc: ssm.scan_fwd(x, dl, A, Bm, Cm, Dk, z, out=y, workspace=ws,
                                                              discretization=disc), 10)
        ms = vt[len(vt) // 2]
        upd = Bsz * L * D * N
        slots = upd * sm[disc] + Bsz * L * D * sm["token_gated"]
        ts = slots / (ms * 1e-3) / 1e12
        out["variants"][disc] = {
            "workload": c["name"] + f", {disc} discretisation",
            "ms_median": round(ms, 4), "state_updates_per_s": upd / (ms * 1e-3),
            "roofline": {"bound": "alu", "achieved": round(ts, 3), "peak": round(VALU_PEAK_TSLOTS, 3),
                         "unit": "Tslot/s", "frac": round(ts / VALU_PEAK_TSLOTS, 4),
                         "alg_slots_per_launch": slots},
            "timing": "median of 10 launches queued back to back, each between two events (B/C pre-pass included)",
        }
        log(f"{disc}: {ms * 1e3:.1f} us/launch, {upd / (ms * 1e-3):.3e} updates/s, "
            f"VALU {ts / VALU_PEAK_TSLOTS:.1%}")
        # oracle beside it: 256 channels of every batch row over the whole sequence
        dsel = torch.arange(0, D, 4, device=dev)
        ser = lambda t: _host(t[:, :, dsel].permute(0, 2, 1)).reshape(Bsz * len(dsel), L)
        cb = np.repeat(np.arange(Bsz), len(dsel))
        cd = np.tile(np.arange(len(dsel)), Bsz)
        a_ = (ser(x), ser(dl), _host(A[dsel]), _host(Bm), _host(Cm), _host(Dk[dsel]), ser(z), None, False,
              cb, cd, cores, disc)
        deferred.append((out["variants"][disc], lambda a_=a_: oracle.scan_f64(*a_), Bsz * len(dsel) * L * N,
                         "state-updates/s", f"{Bsz * len(dsel)} channels (every 4th) x {L} steps, fp64 C oracle", cores))
    del x, dl, z, Bm, Cm, y, ws
    torch.cuda.empty_cache()
    # --- multi-head SSD scan (Mamba-2 layer) on the matrix cores ---
    t = _ssd_inputs(torch, dev)
    settle_calls(torch, lambda: ssm.ssd_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], out=t["y"]))
    st = time_calls(torch, lambda: ssm.ssd_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                                               out=t["y"]), 10)
    ms = st[len(st) // 2]
    byts, flops = ssd_alg(SSD_SHAPE)
    gbs = byts / (ms * 1e-3) / 1e9
    tfs = flops / (ms * 1e-3) / 1e12
    c = SSD_SHAPE
    out["ssd"] = {
        "workload": "Mamba-2 layer SSD scan B4 L4096 H64 P64 N128 bf16 gated",
        "ms_median": round(ms, 4),
        "state_updates_per_s": c["batch"] * c["seqlen"] * c["nheads"] * c["headdim"] * c["dstate"] / (ms * 1e-3),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic("ssd_B4_L4096_H64_P64_N128_bf16_gated", src_hash),
                     "alg_bytes_per_launch": byts},
        "mfma": {"achieved": round(tfs, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                 "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4), "alg_flops_per_launch": flops,
                 "note": "algorithmic flops of the chunked form (chunk 64); the kernel issues about 1.7x "
                         "that (split-bf16 operands, full diagonal tiles)"},
        "timing": "median of 10 launches queued back to back, each between two events",
    }
    log(f"ssd: {ms * 1e3:.1f} us/launch, HBM {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%}), "
        f"MFMA {tfs:.0f} TFLOP/s ({tfs / MFMA_BF16_PEAK_TFS:.1%})")
    # oracle beside it: one (batch row, head) over the whole sequence (numpy, fp64)
    a_ = (_host(t["x"][:1, :, :8]), _host(t["delta"][:1, :, :8]), _host(t["A"][:8]), _host(t["B"][:1]),
          _host(t["C"][:1]), _host(t["D"][:8]), _host(t["z"][:1, :, :8]))
    deferred.append((out["ssd"], lambda a_=a_: ssd_oracle.ssd(*a_), 8 * c["seqlen"] * c["headdim"] * c["dstate"],
                     "state-updates/s", "8 heads of one batch row x 4096 steps, fp64 numpy oracle (one thread)", 1))
    # --- its backward (ssm_ssd_bwd: the scan backward on the per-channel expansion) ---
    gys = _randn(tuple(t["x"].shape), gen, dev, bf)
    sws = torch.empty(ssm.ssd_bwd_workspace_bytes(*t["x"].shape, c["dstate"], "bf16"), dtype=torch.uint8, device=dev)

    def ssd_b():
        ssm.ssd_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], None, gys, workspace=sws)

    settle_calls(torch, ssd_b)
    sbt = time_calls(torch, ssd_b, 3)
    sbms = sbt[len(sbt) // 2]
    upd = c["batch"] * c["seqlen"] * c["nheads"] * c["headdim"] * c["dstate"]
    out["ssd_backward"] = {
        "workload": "Mamba-2 layer SSD scan B4 L4096 H64 P64 N128 bf16 gated, backward (dx, ddelta, dA, dB, dC, dD, dz)",
        "ms_median": round(sbms, 3), "state_updates_per_s": upd / (sbms * 1e-3),
        "timing": "median of 3 calls queued back to back, each between two events",
        "workspace_bytes": sws.numel(),
        "note": "the scan backward over the 4096 channels of the per-channel expansion (fp32), 8 groups of "
                "16 states summed in the sweep kernel, then the per-head sums",
    }
    log(f"ssd backward: {sbms:.2f} ms/call ({upd / (sbms * 1e-3):.3e} state-updates/s)")
    a_ = tuple(None if v is None else _host(v) for v in (t["x"][:1, :, :2], t["delta"][:1, :, :2], t["A"][:2],
                                                       t["B"][:1], t["C"][:1], t["D"][:2], t["z"][:1, :, :2]))
    gy_ = _host(gys[:1, :, :2])
    deferred.append((out["ssd_backward"],
                     lambda a_=a_, gy_=gy_: ssd_oracle.ssd_bwd(*a_, None, False, None, gy_, None),
                     2 * c["seqlen"] * c["headdim"] * c["dstate"], "state-updates/s",
                     "2 heads of one batch row x 4096 steps, fp64 numpy oracle (one thread)", 1))
    del t, gys, sws
    torch.cuda.empty_cache()
    # --- causal conv1d + SiLU at the headline shape (HBM-bound) ---
    x, w, bias = _conv_inputs(torch, synth, dev)
    yc = torch.empty_like(x)
    settle_calls(torch, lambda: ssm.conv1d_fwd(x, w, bias, out=yc))
    # 20 launches back to back between two events (a single launch would also time the
    # host's launch latency, longer than this kernel's gaps), 5 repetitions
    ct = []
    for _ in range(5):
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        for _ in range(20):
            ssm.conv1d_fwd(x, w, bias, out=yc)
        b_.record()
        torch.cuda.synchronize()
        ct.append(a_.elapsed_time(b_) / 20)
    ct.sort()
    conv_bytes = 2 * x.numel() * 2 + w.numel() * 4 + bias.numel() * 4
    conv_gbs = conv_bytes / (ct[len(ct) // 2] * 1e-3) / 1e9
    out["conv1d"] = {
        "workload": "causal depthwise conv1d width 4 + SiLU, x [4, 4096, 4096] bf16",
        "kernel_us_median": round(ct[len(ct) // 2] * 1e3, 2),
        "timing": "median over 5 repetitions of 20 back-to-back launches between two events",
        "roofline": {"bound": "hbm", "achieved": round(conv_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(conv_gbs / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic("conv1d_B4_L4096_D4096_W4_bf16", src_hash),
                     "alg_bytes_per_launch": conv_bytes},
    }
    log(f"conv1d: {ct[len(ct) // 2] * 1e3:.1f} us median, {conv_gbs:.0f} GB/s ({conv_gbs / HBM_PEAK_GBS:.1%} of HBM)")
    out["conv1d"]["elements_per_s"] = x.numel() / (ct[len(ct) // 2] * 1e-3)
    # oracle beside it: every 2nd channel of the whole input (numpy, fp64)
    dsel = torch.arange(0, x.shape[2], 2, device=dev)
    a_ = (_host(x[:, :, dsel]), _host(w[dsel]), _host(bias[dsel]))
    deferred.append((out["conv1d"], lambda a_=a_: conv_oracle.conv1d(*a_), x.shape[0] * x.shape[1] * len(dsel),
                     "elements/s", f"every 2nd channel ({len(dsel)}) x 4 x 4096 steps, fp64 numpy oracle (one thread)", 1))
    # --- its backward (dx, dw, dbias) at the same shape ---
    gyc = _randn(tuple(x.shape), gen, dev, bf)
    cws = torch.empty(ssm.conv1d_bwd_workspace_bytes(*x.shape, w.shape[1], "bf16"), dtype=torch.uint8, device=dev)
    settle_calls(torch, lambda: ssm.conv1d_bwd(x, w, bias, None, gyc, workspace=cws))
    ct = []
    for _ in range(5):
        a_e, b_e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_e.record()
        for _ in range(10):
            ssm.conv1d_bwd(x, w, bias, None, gyc, workspace=cws)
        b_e.record()
        torch.cuda.synchronize()
        ct.append(a_e.elapsed_time(b_e) / 10)
    ct.sort()
    # algorithmic bytes: x and dy read, dx written (the per-tile sums are the kernel's own)
    cb_bytes = 3 * x.numel() * 2 + w.numel() * 4 * 2 + bias.numel() * 4 * 2
    cb_gbs = cb_bytes / (ct[len(ct) // 2] * 1e-3) / 1e9
    out["conv1d_backward"] = {
        "workload": "causal depthwise conv1d width 4 + SiLU backward (dx, dw, dbias), x [4, 4096, 4096] bf16",
        "us_median": round(ct[len(ct) // 2] * 1e3, 2),
        "timing": "median over 5 repetitions of 10 back-to-back calls (both launches) between two events",
        "roofline": {"bound": "hbm", "achieved": round(cb_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(cb_gbs / HBM_PEAK_GBS, 4), "alg_bytes_per_launch": cb_bytes},
        "elements_per_s": x.numel() / (ct[len(ct) // 2] * 1e-3),
    }
    log(f"conv1d backward: {ct[len(ct) // 2] * 1e3:.1f} us median, {cb_gbs:.0f} GB/s ({cb_gbs / HBM_PEAK_GBS:.1%} of HBM)")
    # oracle beside it: every 8th channel of the whole input (numpy, fp64)
    dsel = torch.arange(0, x.shape[2], 8, device=dev)
    a_ = (_host(x[:, :, dsel]), _host(w[dsel]), _host(bias[dsel]), None, _host(gyc[:, :, dsel]))
    deferred.append((out["conv1d_backward"], lambda a_=a_: conv_oracle.conv1d_bwd(*a_), x.shape[0] * x.shape[1] * len(dsel),
                     "elements/s", f"every 8th channel ({len(dsel)}) x 4 x 4096 steps, fp64 numpy oracle (one thread)", 1))
    del x, yc, gyc, cws
    # --- backward pass at the headline shape ---
    c = synth.CONFIGS["mamba1p4b_layer"]
    Bsz, L, D, N = c["batch"], c["seqlen"], c["dim"], c["dstate"]
    x, dl, z, gy = (_randn((Bsz, L, D), gen, dev, bf) if k != "dl" else _delta((Bsz, L, D), gen, dev, bf)
                    for k in ("x", "dl", "z", "gy"))
    Bm = _randn((Bsz, L, N), gen, dev, bf)
    Cm = _randn((Bsz, L, N), gen, dev, bf)
    A = torch.from_numpy(synth.make_A(2, D, N)).to(dev)
    Dk = torch.from_numpy(synth.make_D(2, D, "normal")).to(dev)
    ws = torch.empty(ssm.scan_bwd_workspace_bytes(Bsz, L, D, N, "bf16"), dtype=torch.uint8, device=dev)
    settle_calls(torch, lambda: ssm.scan_bwd(x, dl, A, Bm, Cm, Dk, z, None, gy, workspace=ws, need_dh0=False))
    bt = time_calls(torch, lambda: ssm.scan_bwd(x, dl, A, Bm, Cm, Dk, z, None, gy, workspace=ws, need_dh0=False), 5)
    ms = bt[len(bt) // 2]
    upd = Bsz * L * D * N
    bwd_ts = upd * sm["bwd"] / (ms * 1e-3) / 1e12
    out["backward"] = {
        "workload": c["name"] + " backward (dx, ddelta, dz, dB, dC, dA, dD)",
        "ms_median": round(ms, 4), "ms_min": round(bt[0], 4),
        "state_updates_per_s": upd / (ms * 1e-3),
        "roofline": {"bound": "alu", "achieved": round(bwd_ts, 3), "peak": round(VALU_PEAK_TSLOTS, 3),
                     "unit": "Tslot/s", "frac": round(bwd_ts / VALU_PEAK_TSLOTS, 4),
                     "alg_slots_per_launch": upd * sm["bwd"]},
        "timing": "median of 5 calls queued back to back (checkpoint pass, reverse sweep, reductions), each between two events",
        "note": "forward sweep with state checkpoints every 8 steps, then the reverse sweep with recompute",
        "workspace_bytes": ws.numel(),
        "workspace_bytes_given_saved_checkpoints": ssm.scan_bwd_workspace_bytes(Bsz, L, D, N, "bf16", True),
        "checkpoint_bytes": ssm.scan_save_sizes(Bsz, L, D, N, "bf16")[1],
    }
    log(f"backward: {ms:.3f} ms median ({upd / (ms * 1e-3):.3e} state-updates/s, VALU {bwd_ts / VALU_PEAK_TSLOTS:.1%})")
    # the same backward under the other discretisations (their derivatives cost more VALU
    # work per state update than Mamba's; timed, not priced against the roofline)
    out["backward"]["variants"] = {}
    for disc in ("zoh", "bilinear"):
        settle_calls(torch, lambda disc=disc: ssm.scan_bwd(x, dl, A, Bm, Cm, Dk, z, None, gy, workspace=ws,
                                                           need_dh0=False, discretization=disc))
        vt = time_calls(torch, lambda disc=disc: ssm.scan_bwd(x, dl, A, Bm, Cm, Dk, z, None, gy, workspace=ws,
                                                              need_dh0=False, discretization=disc), 5)
        vms = vt[len(vt) // 2]
        out["backward"]["variants"][disc] = {"ms_median": round(vms, 4), "state_updates_per_s": upd / (vms * 1e-3)}
        log(f"backward, {disc}: {vms:.3f} ms median ({upd / (vms * 1e-3):.3e} state-updates/s)")
    # a training step's scan: the forward that saves the checkpoints, then the backward
    # given them (it skips its own forward sweep), against the forward + the backward alone
    y = torch.empty_like(x)
    fws_b, ck_b = ssm.scan_save_sizes(Bsz, L, D, N, "bf16")
    fws = torch.empty(max(fws_b, 1), dtype=torch.uint8, device=dev)
    ck = torch.empty((Bsz, (L + 7) // 8, N, D), dtype=torch.float32, device=dev)
    pws = torch.empty(max(ssm.scan_plan(Bsz, L, D, N, "bf16")["workspace_bytes"], 1), dtype=torch.uint8, device=dev)
    bws = torch.empty(ssm.scan_bwd_workspace_bytes(Bsz, L, D, N, "bf16", saved_checkpoints=True), dtype=torch.uint8,
                      device=dev)

    def fwd_plain():
        ssm.scan_fwd(x, dl, A, Bm, Cm, Dk, z, out=y, workspace=pws)

    def fwd_save():
        ssm.scan_fwd_save(x, dl, A, Bm, Cm, Dk, z, out=y, checkpoints=ck, workspace=fws)

    def bwd_full():
        ssm.scan_bwd(x, dl, A, Bm, Cm, Dk, z, None, gy, workspace=ws, need_dh0=False)

    def bwd_saved():
        ssm.scan_bwd(x, dl, A, Bm, Cm, Dk, z, None, gy, workspace=bws, need_dh0=False, checkpoints=ck)

    def med(fns):
        settle_calls(torch, lambda: [f() for f in fns])
        tt = time_calls(torch, lambda: [f() for f in fns], 5)
        return tt[len(tt) // 2]

    t_save, t_bsaved = med([fwd_save]), med([bwd_saved])
    t_pair_saved, t_pair_plain = med([fwd_save, bwd_saved]), med([fwd_plain, bwd_full])
    out["backward"]["training_step"] = {
        "workload": c["name"] + " forward + backward (all gradients)",
        "ms_forward_saving_checkpoints": round(t_save, 4), "ms_backward_from_checkpoints": round(t_bsaved, 4),
        "ms_step_with_saved_checkpoints": round(t_pair_saved, 4),
        "ms_step_recomputing_checkpoints": round(t_pair_plain, 4),
        "checkpoint_bytes": ck_b,
        "timing": "medians of 5 queued back to back, each call or pair between two events",
    }
    log(f"training step: forward saving checkpoints {t_save:.3f} ms + backward from them {t_bsaved:.3f} ms; "
        f"pair {t_pair_saved:.3f} ms against {t_pair_plain:.3f} ms for forward + recomputing backward")
    del y, fws, ck, pws, bws
    # oracle beside it: 64 channels of every batch row over the whole sequence
    dsel = torch.arange(0, D, 32, device=dev)   # (the oracle keeps per-channel dB, dC: [channels, L, N] each)
    ser = lambda t: _host(t[:, :, dsel].permute(0, 2, 1)).reshape(Bsz * len(dsel), L)
    cb = np.repeat(np.arange(Bsz), len(dsel))
    cd = np.tile(np.arange(len(dsel)), Bsz)
    a_ = (ser(x), ser(dl), _host(A[dsel]), _host(Bm), _host(Cm), _host(Dk[dsel]), ser(z), None, ser(gy),
          None, False, cb, cd, cores)
    deferred.append((out["backward"], lambda a_=a_: oracle.scan_bwd_f64(*a_), Bsz * len(dsel) * L * N, "state-updates/s",
                     f"{Bsz * len(dsel)} channels (every 32nd) x {L} steps, fp64 C oracle", cores))
    del x, dl, z, gy, Bm, Cm, ws
    torch.cuda.empty_cache()
    # --- million-token scan (chunk carries) ---
    c = synth.CONFIGS["million_token"]
    Bsz, L, D, N = c["batch"], c["seqlen"], c["dim"], c["dstate"]
    x = _randn((Bsz, L, D), gen, dev, bf)
    dl = _delta((Bsz, L, D), gen, dev, bf)
    Bm = _randn((Bsz, L, N), gen, dev, bf)
    Cm = _randn((Bsz, L, N), gen, dev, bf)
    A = torch.from_numpy(synth.make_A(3, D, N)).to(dev)
    Dk = torch.from_numpy(synth.make_D(3, D, "normal")).to(dev)
    plan = ssm.scan_plan(Bsz, L, D, N, "bf16")
    ws = torch.empty(max(plan["workspace_bytes"], 1), dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    settle_calls(torch, lambda: ssm.scan_fwd(x, dl, A, Bm, Cm, Dk, out=y, workspace=ws))
    reps = 5
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        ev[i][0].record()
        ssm.scan_fwd(x, dl, A, Bm, Cm, Dk, out=y, workspace=ws)
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / reps
    upd = Bsz * L * D * N
    byts = scan_bytes(Bsz, L, D, N, 2, False)
    slots = upd * sm["update_structured"] + Bsz * L * D * (sm["token"] + sm["e_stage"])
    out["long_sequence"] = {
        "workload": c["name"], "state_updates_per_s": upd / (ms * 1e-3), "ms_per_call": ms,
        "plan": plan, "hbm_frac": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "alu_frac_single_pass_work": round(slots / (ms * 1e-3) / 1e12 / VALU_PEAK_TSLOTS, 4),
        "roofline": {"bound": "alu", "achieved": round(slots / (ms * 1e-3) / 1e12, 3),
                     "peak": round(VALU_PEAK_TSLOTS, 3), "unit": "Tslot/s",
                     "frac": round(slots / (ms * 1e-3) / 1e12 / VALU_PEAK_TSLOTS, 4),
                     "traffic": load_traffic("long_B1_L1048576_D1024_N16_bf16", src_hash),
                     "alg_slots_per_call": slots, "alg_bytes_per_call": byts,
                     "note": "slots of one pass over the sequence (structured path); the call also rescans "
                             "the 4096-step prefixes of 15 chunks"},
        "workspace_bytes": plan["workspace_bytes"],
        "note": "all launches of one call inside the events: B/C pre-pass, every chunk scanned from its own "
                "start, the carry combine (a parallel scan over chunks), the 4096-step prefix of every later "
                "chunk rescanned from its carried-in state, and the continuation launch (whose workgroups exit "
                "at once: no chunk's carried-in state survives its prefix on this input)",
    }
    log(f"long sequence: {ms:.2f} ms/call, {upd / (ms * 1e-3):.3e} updates/s, plan {plan}")
    # oracle beside it: 16 channels over the whole million steps
    dsel = torch.arange(0, D, 64, device=dev)
    ser = lambda t: _host(t[:, :, dsel].permute(0, 2, 1)).reshape(Bsz * len(dsel), L)
    cb = np.repeat(np.arange(Bsz), len(dsel))
    cd = np.tile(np.arange(len(dsel)), Bsz)
    a_ = (ser(x), ser(dl), _host(A[dsel]), _host(Bm), _host(Cm), _host(Dk[dsel]), None, None, False, cb, cd, cores)
    deferred.append((out["long_sequence"], lambda a_=a_: oracle.scan_f64(*a_), Bsz * len(dsel) * L * N,
                     "state-updates/s", f"{len(dsel)} channels x {L} steps, fp64 C oracle", cores))
    del y, ws
    torch.cuda.empty_cache()
    # --- the million-token backward (chunked: checkpoints from the chunk carries, adjoint
    # carries, one reverse sweep per chunk) ---
    gy = _randn((Bsz, L, D), gen, dev, bf)
    wsb = torch.empty(ssm.scan_bwd_workspace_bytes(Bsz, L, D, N, "bf16"), dtype=torch.uint8, device=dev)
    settle_calls(torch, lambda: ssm.scan_bwd(x, dl, A, Bm, Cm, Dk, None, None, gy, workspace=wsb, need_dh0=False))
    bt = time_calls(torch, lambda: ssm.scan_bwd(x, dl, A, Bm, Cm, Dk, None, None, gy, workspace=wsb,
                                                need_dh0=False), 3)
    ms = bt[len(bt) // 2]
    bwd_ts = upd * sm["bwd"] / (ms * 1e-3) / 1e12
    out["long_sequence_backward"] = {
        "workload": c["name"] + " backward (dx, ddelta, dB, dC, dA, dD)",
        "ms_median": round(ms, 3), "state_updates_per_s": upd / (ms * 1e-3),
        "roofline": {"bound": "alu", "achieved": round(bwd_ts, 3), "peak": round(VALU_PEAK_TSLOTS, 3),
                     "unit": "Tslot/s", "frac": round(bwd_ts / VALU_PEAK_TSLOTS, 4),
                     "alg_slots_per_launch": upd * sm["bwd"]},
        "timing": "median of 3 calls queued back to back, each between two events",
        "note": "chunks of the forward planner (16 x 65536 steps): chunked checkpoint pass, adjoint carries and "
                "their combine, reverse sweep per chunk; the carry passes are not counted as algorithmic work",
        "workspace_bytes": wsb.numel(),
        "checkpoint_bytes": ssm.scan_save_sizes(Bsz, L, D, N, "bf16")[1],
    }
    log(f"long-sequence backward: {ms:.2f} ms/call ({upd / (ms * 1e-3):.3e} state-updates/s, "
        f"VALU {bwd_ts / VALU_PEAK_TSLOTS:.1%})")
    # oracle beside it: 2 channels over the whole million steps (its per-channel dB, dC are
    # [channels, L, N] each)
    dsel = torch.arange(0, D, 512, device=dev)
    ser = lambda t: _host(t[:, :, dsel].permute(0, 2, 1)).reshape(Bsz * len(dsel), L)
    cb = np.repeat(np.arange(Bsz), len(dsel))
    cd = np.tile(np.arange(len(dsel)), Bsz)
    a_ = (ser(x), ser(dl), _host(A[dsel]), _host(Bm), _host(Cm), _host(Dk[dsel]), None, None, ser(gy),
          None, False, cb, cd, cores)
    deferred.append((out["long_sequence_backward"], lambda a_=a_: oracle.scan_bwd_f64(*a_), Bsz * len(dsel) * L * N,
                     "state-updates/s", f"{len(dsel)} channels x {L} steps, fp64 C oracle", cores))
    del x, dl, gy, Bm, Cm, wsb
    torch.cuda.empty_cache()
    # the oracle beside each measurement, on its bounded sample, after the last GPU timing
    for entry, fn, work, unit, sample, nthr in deferred:
        entry["cpu_baseline"] = _cpu_entry(_timed(fn), work, unit, sample, nthr)
    log("oracle baselines of the secondary measurements: " +
        ", ".join(f"{e['cpu_baseline']['value']:.3e} {e['cpu_baseline']['unit']}" for e, *_ in deferred))
    return out


if __name__ == "__main__":
    main()
