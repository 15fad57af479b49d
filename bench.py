#!/usr/bin/env python3
"""Benchmark of the fused norm + FP8 hot path on one MI355X.

A step is one pass of the path over one batch of the headline workload (bf16 LayerNorm,
16384 rows x hidden 4096): the forward of batch k and the backward of batch k-1 (the
backward reads data written a full step earlier, as in training, instead of x still held in
the Infinity Cache by the forward just before). Buffer sets rotate so that the working set
of consecutive steps exceeds the 256 MB Infinity Cache. Inputs are resident in HBM before
the timed region starts.

Printed: one JSON line. `value` is achieved GB/s = minimal algorithmic bytes of the step
(each input read once, each output written once) / step time, the steps timed back to back
with nothing between the launches; `roofline` gives the dominant call (the backward) against
the 8 TB/s HBM peak, its average launch duration taken over back-to-back launches of that
call bracketed by HIP events on the launch stream;
`cpu_baseline` times the float64 CPU oracle on a bounded row sample of the same workload;
`workloads` reports every other workload of the benchmark's list the same way.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_GBS = 8000.0
METRIC = "achieved HBM GB/s (% of peak) for norm fwd/bwd; rows/sec at hidden 4096–12288"
HEADLINE = "ln_bf16_16384x4096"
BYTES = {"f32": 4, "bf16": 2, "f16": 2}


# ------------------------------------------------------------------------------ byte model

def fwd_bytes(w: W.Workload) -> int:
    n, h, e = w.rows, w.hidden, BYTES[w.in_dtype]
    wb = BYTES[w.w_dtype]
    ln = w.norm == "layernorm"
    b = n * h * e + h * wb * (2 if ln else 1) + n * 4 * (2 if ln else 1)
    if w.scaling == "none":
        b += n * h * e
    else:
        b += n * h * (2 if w.colwise else 1)
        if w.scaling == "mxfp8":
            b += -(-h // 32) * n + (-(-n // 32) * h if w.colwise else 0)
        else:
            b += 4 + 4 + 4 + 4 + (4 if w.colwise else 0)   # scale, amax in; updated amax, scale_inv(s) out
    return b


def bwd_bytes(w: W.Workload, add: bool) -> int:
    n, h, e = w.rows, w.hidden, BYTES[w.in_dtype]
    wb = BYTES[w.w_dtype]
    ln = w.norm == "layernorm"
    return (n * h * e * (3 + (1 if add else 0)) + n * 4 * (2 if ln else 1) + h * wb
            + h * wb * (2 if ln else 1))


# ------------------------------------------------------------------------------ GPU runs

def upload(w: W.Workload, sets: int, nf):
    """`sets` distinct device buffer sets of the workload (same values, distinct memory)."""
    host = W.make_inputs(w)
    prior = W.make_inputs(w, prior=True)["x"] if w.scaling == "delayed" else None
    out = []
    for _ in range(sets):
        d = {k: v.cuda() for k, v in host.items()}
        out.append(d)
    if w.scaling == "delayed":
        # delayed scaling: the scale comes from the previous step's amax (the prior batch),
        # produced by the same forward, as a training loop would
        g = out[0]["gamma"]
        st = torch.ones(1, device="cuda")
        am = torch.zeros(1, device="cuda")
        r = nf.fwd(prior.cuda(), g, None, norm=w.norm, eps=w.eps, scaling="delayed", fp8=w.fp8, scale=st,
                   amax=am, layout="rowwise")
        torch.cuda.synchronize()
        fmax = 448.0 if w.fp8 == "e4m3" else 57344.0
        scale = torch.tensor([fmax], device="cuda") / r["amax"]
        for d in out:
            d["scale"] = scale.clone()
            d["amax_in"] = torch.zeros(1, device="cuda")
    del host
    return out


def run_workload(w: W.Workload, nf, steps: int, warmup: int, headline: bool):
    """Time `steps` steps; return per-call stats and the step time."""
    e = BYTES[w.in_dtype]
    per_set = w.rows * w.hidden * e * (4 if "bwd" in w.passes or "bwd_add" in w.passes else 2)
    sets = max(2, min(6, -(-(1 << 30) // max(per_set, 1)) + 1))
    bufs = upload(w, sets, nf)
    st = torch.cuda.current_stream()

    fwd_kw = dict(norm=w.norm, eps=w.eps, zero_centered_gamma=w.zero_centered_gamma)
    if w.scaling == "delayed":
        fwd_kw.update(scaling="delayed", fp8=w.fp8, layout="rowwise_colwise" if w.colwise else "rowwise")
    elif w.scaling == "mxfp8":
        fwd_kw.update(scaling="mxfp8", fp8=w.fp8, layout="rowwise_colwise" if w.colwise else "rowwise")

    has_fwd = "fwd" in w.passes
    has_bwd = "bwd" in w.passes or "bwd_add" in w.passes
    # one prepared forward and backward per buffer set: a single foreign call per launch
    fcalls, bcalls = [], []
    for d in bufs:
        kw = dict(fwd_kw)
        if w.scaling == "delayed":
            kw.update(scale=d["scale"], amax=d["amax_in"])
        fo, fc = nf.prepare_fwd(d["x"], d["gamma"], d.get("beta"), **kw)
        fcalls.append(fc)
        if has_bwd:
            fc()          # statistics for this set's backward
            if "bwd_add" in w.passes:
                _, bc = nf.prepare_bwd_add(d["dy"], d["x"], d["residual_dy"], fo["rsigma"], d["gamma"],
                                           zero_centered_gamma=w.zero_centered_gamma)
            else:
                _, bc = nf.prepare_bwd(d["dy"], d["x"], fo["mu"], fo["rsigma"], d["gamma"], norm=w.norm,
                                       zero_centered_gamma=w.zero_centered_gamma)
            bcalls.append(bc)
    torch.cuda.synchronize()

    def step(k):
        i = k % sets
        j = (k - 1) % sets
        if has_fwd:
            fcalls[i]()
        if has_bwd:
            bcalls[j]()

    for k in range(max(warmup, sets)):
        step(k)
    torch.cuda.synchronize()

    # the timed region: exactly `steps` steps with nothing between the launches (an event
    # recorded between two kernels adds a gap to the stream)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(st)
    for k in range(steps):
        step(warmup + k)
    t1.record(st)
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / steps
    # the per-call breakdown: each call's average launch duration over `steps` back-to-back
    # launches on rotating buffer sets, bracketed by two HIP events on the launch stream (three
    # such runs; an event recorded between every two launches would add its own gap to each)
    def per_call(calls):
        out = []
        for _ in range(3):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            calls[-1]()  # untimed: the first event then waits behind a kernel, not behind the host
            a.record(st)
            for k in range(steps):
                calls[k % len(calls)]()
            b.record(st)
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b) * 1e3 / steps)
        return out
    fwd_us = per_call(fcalls) if has_fwd else []
    bwd_us = per_call(bcalls) if has_bwd else []

    res = {"rows": w.rows, "hidden": w.hidden, "norm": w.norm, "in_dtype": w.in_dtype,
           "scaling": w.scaling, "colwise": w.colwise, "step_ms": step_ms}
    tot_bytes = 0
    if has_fwd:
        b = fwd_bytes(w)
        t = float(np.mean(fwd_us))
        res["fwd"] = {"bytes": b, "us_mean": t, "us_min": float(np.min(fwd_us)), "GBps": b / t / 1e3,
                      "pct_peak": 100.0 * b / t / 1e3 / PEAK_GBS, "rows_per_s": w.rows / (t * 1e-6)}
        tot_bytes += b
    if has_bwd:
        b = bwd_bytes(w, "bwd_add" in w.passes)
        t = float(np.mean(bwd_us))
        res["bwd"] = {"bytes": b, "us_mean": t, "us_min": float(np.min(bwd_us)), "GBps": b / t / 1e3,
                      "pct_peak": 100.0 * b / t / 1e3 / PEAK_GBS, "rows_per_s": w.rows / (t * 1e-6),
                      "kernels": "row kernel + finalize"}
        tot_bytes += b
    res["step_bytes"] = tot_bytes
    res["GBps"] = tot_bytes / (step_ms * 1e-3) / 1e9
    del bufs, fcalls, bcalls
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------------------ HBM traffic

COUNTERS = os.path.join(ROOT, "profiles", "hbm_counters.txt")
BWD_SOURCES = ["rmsnorm_fp8_quantization_amd/csrc/bwd.hip", "rmsnorm_fp8_quantization_amd/csrc/device_common.hpp",
               "rmsnorm_fp8_quantization_amd/csrc/plan.hpp", "rmsnorm_fp8_quantization_amd/csrc/api.cpp"]


def sources_sha256(paths):
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per backward call from the committed rocprofv3 counter summary, scaled by the
    copy-kernel calibration recorded with it; None when the summary is missing or the backward
    sources have changed since the counters were taken."""
    if not os.path.exists(COUNTERS):
        return None
    kv = {}
    with open(COUNTERS) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#") and "=" in line:
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    try:
        if kv.get("bwd_sources_sha256") != sources_sha256(BWD_SOURCES):
            return None
        return float(kv["bwd_call_hbm_bytes"])
    except (KeyError, ValueError):
        return None


def copy_calibration(nbytes: int = 1 << 30, reps: int = 3):
    """A plain device copy of known size (run under rocprofv3 --pmc to calibrate FETCH_SIZE and
    WRITE_SIZE): prints its bytes and mean time."""
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps,
                      "us_per_copy": dt * 1e6, "GBps": 2 * nbytes / dt / 1e9}))


# ------------------------------------------------------------------------------ CPU baseline

def cpu_baseline(w: W.Workload, min_s: float = 10.0, max_passes: int = 8):
    """The float64 oracle (numpy, one thread) on the workload's whole batch, forward + backward,
    in chunks of 4096 rows, repeated until at least `min_s` seconds of CPU work (bounded by
    `max_passes` passes); reported in the metric's unit (GB/s over the same byte model)."""
    import oracle
    host = W.make_inputs(w)
    xb = W.to_numpy_bits(host["x"])
    dyb = W.to_numpy_bits(host["dy"]) if "dy" in host else None
    g = W.to_numpy_bits(host["gamma"])
    b = W.to_numpy_bits(host["beta"]) if "beta" in host else None
    del host
    chunk = 4096
    passes = 0
    t0 = time.perf_counter()
    while True:
        for r0 in range(0, w.rows, chunk):
            sl = slice(r0, min(w.rows, r0 + chunk))
            f = oracle.forward_stored(xb[sl], g, b, norm=w.norm, eps=w.eps, in_dtype=w.in_dtype,
                                      w_dtype=w.w_dtype, zero_centered_gamma=w.zero_centered_gamma)
            oracle.plain_output(f["v"], w.in_dtype)
            if dyb is not None:
                oracle.backward_stored(dyb[sl], xb[sl], f["mu"], f["rsigma"], g, norm=w.norm,
                                       in_dtype=w.in_dtype, w_dtype=w.w_dtype,
                                       zero_centered_gamma=w.zero_centered_gamma)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_s or passes >= max_passes:
            break
    nbytes = passes * (fwd_bytes(w) + (bwd_bytes(w, False) if dyb is not None else 0))
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} pass(es) over the whole {w.name} batch ({w.rows} rows), fwd+bwd, "
                      f"float64 numpy on one thread, {dt:.1f} s",
            "rows_per_s": passes * w.rows / dt}


# ------------------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for rocprofv3 counter calibration)")
    ap.add_argument("--workload", choices=sorted(W.WORKLOADS), default=None,
                    help="only time this workload and print its figures (for rocprofv3 runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the method shards by rows "
              "with no communication on the hot path); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    import rmsnorm_fp8_quantization_amd as nf

    if args.workload:
        res = run_workload(W.WORKLOADS[args.workload], nf, args.steps, args.warmup, args.workload == HEADLINE)
        print(json.dumps({"workload": args.workload, **res}))
        return

    hw = W.WORKLOADS[HEADLINE]
    head = run_workload(hw, nf, args.steps, args.warmup, True)
    print(f"[bench] {HEADLINE}: step {head['step_ms']*1e3:.1f} us, {head['GBps']:.0f} GB/s", file=sys.stderr,
          flush=True)
    others = {}
    if not args.headline_only:
        for name, w in W.WORKLOADS.items():
            if name == HEADLINE:
                continue
            others[name] = run_workload(w, nf, args.steps, args.warmup, False)
            print(f"[bench] {name}: step {others[name]['step_ms']*1e3:.1f} us, "
                  f"{others[name]['GBps']:.0f} GB/s", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(hw)
        print(f"[bench] cpu oracle: {cpu['value']:.3f} GB/s ({cpu['sample']})", file=sys.stderr, flush=True)

    bwd = head["bwd"]
    line = {
        "metric": METRIC,
        "value": round(head["GBps"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["step_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "pct_of_peak": round(100.0 * head["GBps"] / PEAK_GBS, 2),
        "rows_per_s": round(hw.rows / (head["step_ms"] * 1e-3), 1),
        "config": {"workload": f"{HEADLINE} LayerNorm fwd+bwd", "rows": hw.rows, "hidden": hw.hidden,
                   "in_dtype": hw.in_dtype, "w_dtype": hw.w_dtype, "eps": hw.eps,
                   "step": "fwd(batch k) + bwd(batch k-1)"},
        "roofline": {"bound": "hbm", "achieved": round(bwd["GBps"], 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(bwd["GBps"] / PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": "norm_bwd (bwd_kernel + bwd_finalize_kernel)",
                     "bytes_per_launch": bwd["bytes"], "us_per_launch": round(bwd["us_mean"], 2)},
        "cpu_baseline": cpu,
        "fwd": head["fwd"],
        "bwd": head["bwd"],
        "workloads": others,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
