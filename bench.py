#!/usr/bin/env python3
"""Benchmark of the fused attention forward pass on one MI355X.

One step = one ``fa_fwd`` call over the whole workload (every query row of
every head: Q-tile load, K/V loop with scores, online softmax and P V, and the
normalised store), with Q, K, V already resident in HBM.  The default
workload is B=2, H=16, Nq=Nk=8192, d=128 (non-causal, BF16), one of the
sequence lengths at which the 60 %-of-peak goal is stated.

Prints ONE JSON line: throughput (TFLOP/s, 4*B*H*Nq*Nk*d per call), a
``roofline`` object for the kernel (achieved TFLOP/s from HIP events on the
launch stream vs the MI355X dense-BF16 MFMA peak), a ``cpu_baseline`` object
(the fp64 oracle timed on a bounded sample of the same workload on this
host's cores; ``all_rows`` says whether the sample is the whole workload),
``also`` (the 16K workload timed the same way, after the main one), ``clock``
(the shader clock sampled by a child process during a sustained run after
the timed region) and ``parity_ok``.  The oracle's rows double as a parity
check against the forward's gates; if any check fails the line is still
printed and the process exits with status 3.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import fa06_inputs as fi  # noqa: E402

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X published dense BF16 matrix peak
MFMA_FP8_PEAK_TFLOPS = 5000.0    # MI355X published dense FP8 matrix peak
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "b2_h16_n8192"
# HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE
# (one run each) on the default workload, each scaled by what the same counter
# reads for a plain copy kernel of known size (read x2.000, write x1.000).
# Reported only while the library's build string is the one measured; any
# other kernel build reports null.  (The string last changed for the 4-wave
# kernels at head sizes 64 and 128, the causal kernel, the head-size-64
# bias kernel and the key split; the 8-wave kernel that the default workload
# runs compiles to the same machine code as when it was measured.)
MEASURED_TRAFFIC = {
    "kernel": "gfx950 fa_fwd v19: BR=128 (4 waves x 32 rows; 256 = 8 waves for head size 128 without bias and 64 "
              "without mask or bias on grids of >= 256 workgroups incl. key-split ranges without mask, causal from "
              "8192 rows; 8 waves as two key groups of 4 on 128 rows, merged in LDS, where 128-row workgroups give "
              "each CU one), plain tiles (below the diagonal with the causal mask; with a bias not at head size "
              "64, (192, 128) causal only with a bias) in fixed MFMA segments (32 at head sizes 128 and 256, 40 at "
              "(192, 128), 16 at 64 and at 128 with a bias, 20 at (192, 128) with a bias), BC=64 (32 with bias), "
              "3-stage K/V pipeline (S two tiles ahead of P V, softmax in between, its exponent, exponential and "
              "row sum a segment apart), direct-to-LDS, S^T=K.Q^T on mfma_f32_32x32x16_bf16 (K fragments read two "
              "k steps ahead at head size 128, one at (192, 128) without mask or bias; three waves per SIMD and a "
              "two-FMA exponent at head size 64 with a bias), V^T via ds_read_b64_tr_b16; O divided by the sum of "
              "the bf16 P taken on mfma_f32_16x16x32_bf16 with a 0/1 mask (bf16 dot products at head size 256 with "
              "a bias and (192, 128) without mask or bias); no tile max unless exp2 exceeds 2^16; causal tile "
              "skipping; fp32 additive bias; key split with LSE merge",
    "workload": "b2_h16_n8192",
    "bytes": 269.8e6,
    "profile": "profiles/fa_fwd_kernel__b2_h16_n8192__hbm_bytes.txt",
}


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=25)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=fi.WORKLOAD_ORDER)
    p.add_argument("--cpu-seconds", type=float, default=20.0,
                   help="target wall time of the oracle sample (CPU baseline)")
    p.add_argument("--causal", action="store_true",
                   help="causal mask (key j hidden from query i when j > i + Nk - Nq); throughput counts "
                        "only the visible (query, key) pairs")
    p.add_argument("--bias", choices=["none", "alibi", "keys"], default="none",
                   help="fp32 additive bias: 'alibi' = -2^-(h+1)*|i + Nk - Nq - j| materialised as "
                        "[1, H, Nq, Nk] (read from HBM every call), 'keys' = one random value per "
                        "(b, h, key), broadcast over the rows ([B, H, 1, Nk]).  Without a bias the "
                        "oracle sample is timed; with one it is skipped")
    p.add_argument("--bwd", action="store_true",
                   help="time the backward pass (fa_bwd_dv: dQ, dK, dV from dO, with O and LSE from one "
                        "forward call) instead of the forward; FLOP = five matrix products, 2*(3d + 2d_v) per "
                        "visible pair (2.5x the forward's when d_v = d; the kernels' recomputation of S and dP "
                        "in the dQ pass is not counted)")
    p.add_argument("--mxfp8", action="store_true",
                   help="time the MXFP8 forward (fa_fwd_mxfp8) on the workload's Q, K, V quantized once by the "
                        "library's GPU encoders (not timed); peak = dense FP8 MFMA")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--also", default=None,
                   help="comma-separated further workloads timed after the main one and reported under "
                        "'also' (default: the 16K workload and the 5090 benchmark shape when the main one is "
                        "the default plain forward; 'none' for none)")
    p.add_argument("--no-clock", action="store_true",
                   help="skip the sustained run that samples the shader clock")
    p.add_argument("--splitkv", type=int, default=None, metavar="N",
                   help="time the key-split forward (fa_fwd_splitkv, split kernel + merge kernel) with N key "
                        "ranges (0: the library's choice)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="instead of attention, run a plain copy kernel (256 MiB read + 256 MiB "
                        "written per launch) to calibrate the HBM byte counters")
    return p.parse_args()


def calibrate_copy(args):
    """Plain streaming kernel of known size, for scaling FETCH_SIZE/WRITE_SIZE."""
    import torch
    n = 64 << 20  # fp32 elements: 256 MiB each way
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(args.warmup):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        torch.neg(x, out=y)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    print(json.dumps({"calibration": "copy kernel (torch.neg, fp32)", "bytes_read": 4 * n,
                      "bytes_written": 4 * n, "kernel_ms": round(ms, 4),
                      "GB_per_s": round(8 * n / ms / 1e6, 1), "steps": args.steps}), flush=True)


def visible_pairs(Nq: int, Nk: int, causal: bool) -> int:
    """(query, key) pairs one head computes: Nq*Nk, or the causal count."""
    if not causal:
        return Nq * Nk
    off = Nk - Nq
    i = np.arange(Nq, dtype=np.int64)
    return int(np.clip(i + off + 1, 0, Nk).sum())


# Shader-clock sampler, run as a child process (it never touches HIP): reads
# the GFX clock and socket power through amdsmi every ~20 ms until its stdin
# closes, then prints one JSON object with the samples.
CLOCK_SAMPLER = r"""
import json, sys, threading, time
out = {"sclk_mhz": [], "power_w": [], "error": None}
try:
    import amdsmi
    amdsmi.amdsmi_init()
    h = amdsmi.amdsmi_get_processor_handles()[0]
except Exception as e:  # no amdsmi or no device: report why
    out["error"] = repr(e)
    h = None
stop = threading.Event()
threading.Thread(target=lambda: (sys.stdin.read(), stop.set()), daemon=True).start()
print("ready", flush=True)
while h is not None and not stop.is_set():
    try:
        out["sclk_mhz"].append(amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.SYS)["clk"])
    except Exception as e:
        out["error"] = repr(e)
    try:
        m = amdsmi.amdsmi_get_gpu_metrics_info(h)
        p = m.get("current_socket_power", m.get("average_socket_power"))
        if isinstance(p, (int, float)):
            out["power_w"].append(p)
    except Exception:
        pass
    time.sleep(0.02)
print(json.dumps(out), flush=True)
"""


def sustained_clock(step, seconds=1.5):
    """Runs `step` back to back for about `seconds` while a child process
    samples the shader clock; returns the median and range of the samples."""
    import subprocess

    import torch
    child = subprocess.Popen([sys.executable, "-c", CLOCK_SAMPLER], stdin=subprocess.PIPE,
                             stdout=subprocess.PIPE, text=True)
    try:
        if child.stdout.readline().strip() != "ready":
            return {"error": "sampler did not start"}
        t_end = time.perf_counter() + seconds
        calls = 0
        while time.perf_counter() < t_end:
            for _ in range(8):
                step()
            calls += 8
            torch.cuda.synchronize()
        child.stdin.close()
        res = json.loads(child.stdout.readline() or "{}")
    finally:
        child.wait(timeout=30)
    clk = sorted(res.get("sclk_mhz") or [])
    pw = sorted(res.get("power_w") or [])
    if not clk:
        return {"error": res.get("error") or "no samples", "calls": calls}
    # skip the first quarter of the samples: the clock settles after the load starts
    tail = clk[len(clk) // 4:] if len(clk) >= 8 else clk
    return {"sclk_mhz_median": float(np.median(tail)), "sclk_mhz_min": clk[0], "sclk_mhz_max": clk[-1],
            "samples": len(clk), "socket_power_w_median": float(np.median(pw)) if pw else None,
            "seconds": seconds, "calls": calls, "source": "amdsmi GFX clock, child process"}


def time_calls(step, stream, steps, warmup):
    """HIP events on the launch stream around `steps` back-to-back calls after
    `warmup` untimed ones; returns ms per call."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def metric_name(args, w, bias_kind):
    """The metric text for the flags actually used; without flags it is the
    headline metric (forward, bf16, d=128, non-causal)."""
    dtype = "mxfp8" if args.mxfp8 else "bf16"
    hd = f"d={w.d}" if w.d == w.d_v else f"d={w.d}, d_v={w.d_v}"
    mask = "causal" if args.causal else "non-causal"
    extra = "" if bias_kind == "none" else f", bias {bias_kind}"
    split = "" if args.splitkv is None else ", key split"
    peak = "FP8" if args.mxfp8 else ""
    return (("bwd" if args.bwd else "fwd") + f" attention TFLOP/s ({dtype}, {hd}, {mask}{extra}{split}) and % of "
            f"MI355X {peak + ' ' if peak else ''}MFMA peak")


def cpu_baseline(Q, K, V, w, target_s, o_gpu=None, lse_gpu=None, causal=False):
    import oracle
    import torch
    per_row_flop = 2 * w.Nk * (w.d + w.d_v)
    total_rows = w.B * w.H * w.Nq
    rng = np.random.default_rng(w.seed + 17)
    # calibrate on a small sample, then size the timed sample to ~target_s
    n0 = 512
    rows0 = np.sort(rng.choice(total_rows, size=n0, replace=False)).astype(np.int64)

    def run(rows):
        if causal:
            return oracle.attention_masked(Q, K, V, w.scale, causal=True, rows=rows)
        return oracle.attention_rows(Q, K, V, w.scale, rows)

    def flops(rows):
        if not causal:
            return len(rows) * per_row_flop
        i = rows % w.Nq
        return int(np.clip(i + (w.Nk - w.Nq) + 1, 0, w.Nk).sum()) * 2 * (w.d + w.d_v)

    t0 = time.perf_counter()
    run(rows0)
    dt0 = time.perf_counter() - t0
    n = int(min(total_rows, max(n0, n0 * target_s / max(dt0, 1e-6))))
    rows = np.sort(rng.choice(total_rows, size=n, replace=False)).astype(np.int64)
    t0 = time.perf_counter()
    Oo, Lo = run(rows)
    dt = time.perf_counter() - t0
    res = {
        "value": flops(rows) / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": f"{n} of {total_rows} query rows of {w.name}{' causal' if causal else ''} "
                  f"(all their visible keys), fp64, {dt:.1f} s",
        "rows": n,
        "rows_total": total_rows,
        "all_rows": n == total_rows,
    }
    parity = None
    if o_gpu is not None:
        idx = torch.from_numpy(rows).to(o_gpu.device)
        og = o_gpu.view(-1, w.d_v)[idx].float().cpu().numpy().astype(np.float64)
        lg = lse_gpu.view(-1)[idx].cpu().numpy().astype(np.float64)
        dO = np.abs(og - Oo)
        parity = {"rows": n, "max_abs_dO": float(dO.max()), "mean_abs_dO": float(dO.mean()),
                  "max_abs_dLSE": float(np.abs(lg - Lo).max())}
    return res, parity


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the forward pass shards "
              "over (batch, head, q-tile) with no communication, so multi-GPU runs are not part "
              "of this benchmark.", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args)
        return
    import torch
    import flashattention_forward_06_amd as fa

    w = fi.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    Q, K, V = fi.make_workload(w)

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = up(Q), up(K), up(V)
    o = torch.empty((w.B, w.H, w.Nq, w.d_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    fa.load_library()
    bias = None
    if args.bias == "alibi":
        i = torch.arange(w.Nq, device=dev, dtype=torch.int64)[:, None] + (w.Nk - w.Nq)
        j = torch.arange(w.Nk, device=dev, dtype=torch.int64)[None, :]
        slopes = 2.0 ** -(torch.arange(w.H, device=dev, dtype=torch.float32) + 1)
        bias = (-slopes[:, None, None] * (i - j).abs().to(torch.float32)[None])[None].contiguous()
        sb, sh, sq = 0, w.Nq * w.Nk, w.Nk
    elif args.bias == "keys":
        g = torch.Generator(device=dev).manual_seed(w.seed)
        bias = torch.randn((w.B, w.H, 1, w.Nk), generator=g, device=dev, dtype=torch.float32)
        sb, sh, sq = w.H * w.Nk, w.Nk, 0
    if bias is not None and (w.Nk % 4 or bias.data_ptr() % 16):
        raise SystemExit("bias rows must be 16-byte aligned (Nk a multiple of 4)")
    if args.splitkv is not None:
        if args.mxfp8 or args.bwd:
            raise SystemExit("--splitkv is a forward option of the bf16 path")
        ws_bytes, n_used = fa.splitkv_workspace_bytes(w.B, w.H, w.Nq, w.Nk, w.d_v, args.splitkv)
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        call = fa.fa_fwd_splitkv_raw
        call_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                     w.B, w.H, w.Nq, w.Nk, w.d, w.d_v, w.scale, int(args.causal),
                     None if bias is None else bias.data_ptr(), *((sb, sh, sq) if bias is not None else (0, 0, 0)),
                     args.splitkv, ws.data_ptr(), ws_bytes, sptr)
    elif w.d_v != w.d:
        call = fa.fa_fwd_dv_raw
        call_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                     w.B, w.H, w.Nq, w.Nk, w.d, w.d_v, w.scale, int(args.causal),
                     None if bias is None else bias.data_ptr(), *((sb, sh, sq) if bias is not None else (0, 0, 0)),
                     sptr)
    elif args.causal or bias is not None:
        call = fa.fa_fwd_masked_raw
        call_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                     w.B, w.H, w.Nq, w.Nk, w.d, w.scale, int(args.causal),
                     None if bias is None else bias.data_ptr(), *((sb, sh, sq) if bias is not None else (0, 0, 0)),
                     sptr)
    else:
        call = fa.fa_fwd_raw
        call_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                     w.B, w.H, w.Nq, w.Nk, w.d, w.scale, sptr)
    flop = 2 * w.B * w.H * (w.d + w.d_v) * visible_pairs(w.Nq, w.Nk, args.causal)
    if args.mxfp8:
        if bias is not None or args.bwd or w.d != 128 or w.d_v != 128:
            raise SystemExit("--mxfp8 takes no bias, no --bwd and head size 128 only")
        q8, qs, k8, ks, vt8, vs, _ = fa.mxfp8_inputs(q, k, v)
        torch.cuda.synchronize()
        call = lambda *a: fa.load_library().fa_fwd_mxfp8(*a)
        call_args = (q8.data_ptr(), qs.data_ptr(), k8.data_ptr(), ks.data_ptr(), vt8.data_ptr(), vs.data_ptr(),
                     o.data_ptr(), lse.data_ptr(), w.B, w.H, w.Nq, w.Nk, w.d, vt8.shape[3],
                     ctypes.c_float(w.scale), int(args.causal), sptr)
    if args.bwd:
        if (w.d, w.d_v) not in ((64, 64), (128, 128), (256, 256), (192, 128)) or args.splitkv is not None:
            raise SystemExit("--bwd takes (d, d_v) = (64, 64), (128, 128), (256, 256) or (192, 128) and no --splitkv")
        dO = fi.make_qkv(w.B, w.H, w.Nq, 1, w.d_v, seed=w.seed + 5000)[0]
        g = up(dO)
        rc = call(*call_args)  # forward once: O and LSE
        if rc != 0:
            raise fa.FaError(rc, fa.fa_status_string(rc))
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dv = torch.empty_like(v)
        delta = torch.empty_like(lse)
        call = fa.fa_bwd_dv_raw
        call_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), g.data_ptr(), lse.data_ptr(),
                     dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                     w.B, w.H, w.Nq, w.Nk, w.d, w.d_v, w.scale, int(args.causal),
                     None if bias is None else bias.data_ptr(), *((sb, sh, sq) if bias is not None else (0, 0, 0)),
                     sptr)
        # the conventional five products: S and dK, dQ over d; dP and dV over d_v
        flop = 2 * w.B * w.H * (3 * w.d + 2 * w.d_v) * visible_pairs(w.Nq, w.Nk, args.causal)

    def step():
        rc = call(*call_args)
        if rc != 0:
            raise fa.FaError(rc, fa.fa_status_string(rc))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1) / args.steps

    # per-call durations, after the timed region: one event pair around each call
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in pairs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    per_call = sorted(e0.elapsed_time(e1) for e0, e1 in pairs)

    ms_per_step = wall * 1e3 / args.steps
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (ev_ms * 1e-3) / 1e12
    peak = MFMA_FP8_PEAK_TFLOPS if args.mxfp8 else MFMA_BF16_PEAK_TFLOPS
    # HBM bytes per launch taken from the committed counter profile (not
    # measured in this run); null when the kernel or workload differs
    traffic = (MEASURED_TRAFFIC["bytes"]
               if (fa.fa_build_info() == MEASURED_TRAFFIC["kernel"] and not args.causal and not args.bwd
                   and not args.mxfp8 and bias is None and args.splitkv is None
                   and w.name == MEASURED_TRAFFIC["workload"]) else None)
    roof = {
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "traffic": traffic,
        "traffic_source": ("rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE, " + MEASURED_TRAFFIC["profile"]
                           if traffic is not None else "not measured for this kernel build and workload"),
        "kernel_ms": round(ev_ms, 4),
        "per_call_ms": {"median": round(float(np.median(per_call)), 4), "min": round(per_call[0], 4),
                        "max": round(per_call[-1], 4), "calls": len(per_call)},
    }
    out = {
        "metric": metric_name(args, w, args.bias),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8 (e4m3 + e8m0)" if args.mxfp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name + ("+causal" if args.causal else "") +
                   ("" if bias is None else f"+bias_{args.bias}") + ("+bwd" if args.bwd else "") +
                   ("+mxfp8" if args.mxfp8 else "") +
                   ("" if args.splitkv is None else f"+splitkv{n_used}"), "B": w.B, "H": w.H,
                   "Nq": w.Nq, "Nk": w.Nk, "d": w.d, "d_v": w.d_v, "causal": bool(args.causal), "bias": args.bias,
                   "flop_per_step": flop, "scale": w.scale, "seed": w.seed,
                   "pct_of_peak": round(100 * value / (MFMA_FP8_PEAK_TFLOPS if args.mxfp8 else MFMA_BF16_PEAK_TFLOPS), 2),
                   "kernel": (fa.fa_bwd_build_info() if args.bwd else
                              fa.fa_mxfp8_build_info() if args.mxfp8 else fa.fa_build_info())},
        "roofline": roof,
        "cpu_baseline": None,
        "env": {"device": torch.cuda.get_device_name(dev),
                "arch": getattr(torch.cuda.get_device_properties(dev), "gcnArchName", None),
                "cus": torch.cuda.get_device_properties(dev).multi_processor_count,
                "torch": torch.__version__, "hip": torch.version.hip},
    }
    if bias is not None:
        out["bias_bytes"] = bias.numel() * 4
    if args.bwd:
        out["roofline"]["note"] = "whole backward call (delta + dK/dV + dQ kernels); per-kernel split in profiles/"
    if args.splitkv is not None:
        out["roofline"]["note"] = f"whole key-split call: split kernel ({n_used} key ranges) + merge kernel"
    plain = not (args.causal or args.bwd or args.mxfp8 or bias is not None or args.splitkv is not None)
    if not args.no_clock:
        out["clock"] = sustained_clock(step)
    also = args.also
    if also is None:
        also = "b1_h16_n16384_koffset,rtx5090_q4096_kv8192" if plain and w.name == DEFAULT_WORKLOAD else "none"
    failures = []
    if also != "none":
        if not plain:
            raise SystemExit("--also times the plain forward only")
        out["also"] = {}
        for name in also.split(","):
            wa = fi.WORKLOADS[name]
            Qa, Ka, Va = fi.make_workload(wa)
            qa, ka, va = up(Qa), up(Ka), up(Va)
            oa = torch.empty((wa.B, wa.H, wa.Nq, wa.d_v), dtype=torch.bfloat16, device=dev)
            la = torch.empty((wa.B, wa.H, wa.Nq), dtype=torch.float32, device=dev)
            a_args = (qa.data_ptr(), ka.data_ptr(), va.data_ptr(), oa.data_ptr(), la.data_ptr(),
                      wa.B, wa.H, wa.Nq, wa.Nk, wa.d, wa.d_v, wa.scale, 0, None, 0, 0, 0, sptr)

            def step_a():
                rc = fa.fa_fwd_dv_raw(*a_args)
                if rc != 0:
                    raise fa.FaError(rc, fa.fa_status_string(rc))

            # the clock has dropped during the previous workload's host-side
            # parity check: warm up for ~40 ms of calls however short a call is
            est = time_calls(step_a, stream, 5, 1)
            ms = time_calls(step_a, stream, args.steps, max(args.warmup, int(40.0 / max(est, 1e-3))))
            fl = wa.flops
            rec = {"TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 2), "frac": round(fl / (ms * 1e-3) / 1e12 / peak, 4),
                   "kernel_ms": round(ms, 4), "steps": args.steps, "warmup": args.warmup, "flop_per_step": fl}
            rows = fi.sample_rows(wa.B, wa.H, wa.Nq, 256, seed=wa.seed)
            import oracle
            Or, Lr = oracle.attention_rows(Qa, Ka, Va, wa.scale, rows)
            idx = torch.from_numpy(rows).to(dev)
            og = oa.view(-1, wa.d_v)[idx].float().cpu().numpy().astype(np.float64)
            lg = la.view(-1)[idx].cpu().numpy().astype(np.float64)
            rec["parity_sampled"] = gate({"rows": len(rows), "max_abs_dO": float(np.abs(og - Or).max()),
                                          "mean_abs_dO": float(np.abs(og - Or).mean()),
                                          "max_abs_dLSE": float(np.abs(lg - Lr).max())})
            if not rec["parity_sampled"]["ok"]:
                failures.append(name)
            out["also"][name] = rec
            del qa, ka, va, oa, la
    if not args.no_cpu_baseline and bias is None and not args.bwd and not args.mxfp8:
        cb, parity = cpu_baseline(Q, K, V, w, args.cpu_seconds, o, lse, causal=args.causal)
        out["cpu_baseline"] = cb
        out["parity_sampled"] = gate(parity)
        if not parity["ok"]:
            failures.append(w.name)
    out["parity_ok"] = not failures
    print(json.dumps(out), flush=True)
    if failures:
        print(f"parity gates failed for {failures}: the throughput above is not valid", file=sys.stderr)
        sys.exit(3)


def gate(p):
    """Adds the parity verdict (the forward's gates: max|dO| <= 2e-2,
    mean|dO| <= 2e-3, max|dLSE| <= 1e-3) to a parity record."""
    p["ok"] = bool(p["max_abs_dO"] <= 2e-2 and p["mean_abs_dO"] <= 2e-3 and p["max_abs_dLSE"] <= 1e-3)
    return p


if __name__ == "__main__":
    main()
