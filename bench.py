"""Benchmark of the DV-SSQ linear layer on one MI355X.

Headline (one JSON line on stdout): effective weight GB/s of the Spark-shaped
up_proj decode call (K=2560, N=10240, r=16, M=1) = the packed layer's own bytes
(algo_bytes) per call / time per call, with the prefill TFLOP/s of the fused
gate+up layer (K=2560, N=2x10240, r=24, M=2048) beside it.

Inputs are synthetic and already resident in HBM when timing starts.  The
timed blob is a random, well-formed packed layer of the workload's shape
(timing does not depend on the code values); C distinct copies totalling >= 1
GiB are cycled so the 256 MB last-level cache cannot serve repeats.

A "step" is one dvssq_linear_decode call: rotation, group sums, t = x_rot V^T,
both tiers, the low-rank term, the split-K reduction and the bf16 scatter.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "effective weight GB/s (M=1 decode) and TFLOP/s (M=2048 prefill), % of roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--decode-m", type=int, default=1)
    ap.add_argument("--prefill-steps", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    return ap.parse_args()


def make_copies(dv, torch, lay, M_max, min_bytes=1 << 30, max_copies=256):
    import synth
    L = dv.pack_info(lay.N, lay.K, lay.r, lay.block, lay.n_seg, M_max)
    parts = synth.random_packed_parts(1, lay.N, lay.K, lay.r, lay.n_seg)
    blob = dv.pack_blob(L, parts)
    C = max(2, min(max_copies, math.ceil(min_bytes / L.blob_bytes)))
    dev = torch.empty((C, L.blob_bytes), dtype=torch.uint8, device="cuda")
    src = torch.from_numpy(blob).to("cuda")
    for i in range(C):
        dev[i].copy_(src)
    torch.cuda.synchronize()
    return L, blob, dev, C


def time_calls(torch, fn, steps, warmup):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


def cpu_baseline(lay, blob, x_bits, seconds):
    import oracle
    threads = min(len(os.sched_getaffinity(0)), 16)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(blob, lay.N, lay.K, lay.r, lay.block, lay.n_seg, x_bits, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    L = oracle.layout(lay.N, lay.K, lay.r, lay.n_seg)
    return {"value": round(L["algo_bytes"] * reps / el / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{reps} full fp64 oracle forwards of the same layer and x (M={x_bits.shape[0]}), "
                      f"{el:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the layer's multi-GPU "
              "sharding is described, not run.", file=sys.stderr)
        sys.exit(2)
    import torch

    import bit_linear_amd as dv
    import synth

    torch.cuda.set_device(0)
    up = synth.WORKLOADS["spark_up"].layers[0]
    M = args.decode_m
    L, blob, copies, C = make_copies(dv, torch, up, 32)
    x_bits = synth.activations_bf16(0, up.outlier_tag, M, up.K)
    x = torch.from_numpy(x_bits.view(np.int16)).to("cuda").view(torch.bfloat16)
    y = torch.empty((M, up.N), dtype=torch.bfloat16, device="cuda")
    ws = dv.device_buffer(L.ws_bytes)
    stream = torch.cuda.current_stream().cuda_stream
    ptrs = [copies[i].data_ptr() for i in range(C)]
    lib, Lref = dv.lib(), L
    import ctypes as Cc
    Lp = Cc.byref(Lref)
    xp, yp, wp = x.data_ptr(), y.data_ptr(), ws.data_ptr()

    def dec(i):
        rc = lib.dvssq_linear_decode(Lp, ptrs[i % C], xp, yp, M, wp, 0, stream)
        if rc:
            raise dv.DvssqError(rc, "dvssq_linear_decode")

    ms, wall = time_calls(torch, dec, args.steps, args.warmup)
    gbs = L.algo_bytes / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"spark_up decode K={up.K} N={up.N} r={up.r} H_{up.block} M={M}",
                   "algo_bytes": L.algo_bytes, "blob_copies": C},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
    }
    if not args.no_prefill:
        gu = synth.WORKLOADS["spark_gateup"].layers[0]
        Mp = 2048
        Lg, _, gcopies, Cg = make_copies(dv, torch, gu, Mp, min_bytes=256 << 20, max_copies=16)
        xg = torch.from_numpy(synth.activations_bf16(0, gu.outlier_tag, Mp, gu.K).view(np.int16)).to("cuda").view(torch.bfloat16)
        yg = torch.empty((Mp, gu.N), dtype=torch.bfloat16, device="cuda")
        wsg = dv.device_buffer(Lg.ws_bytes)
        gptr = [gcopies[i].data_ptr() for i in range(Cg)]
        Lgp = Cc.byref(Lg)

        def pre(i):
            rc = lib.dvssq_linear_prefill(Lgp, gptr[i % Cg], xg.data_ptr(), yg.data_ptr(), Mp,
                                          wsg.data_ptr(), 0, stream)
            if rc:
                raise dv.DvssqError(rc, "dvssq_linear_prefill")

        msp, _ = time_calls(torch, pre, args.prefill_steps, 5)
        flops = 2.0 * Mp * gu.N * gu.K + 2.0 * Mp * gu.r * (gu.n_seg * gu.K + gu.N)
        tf = flops / (msp * 1e-3) / 1e12
        out["prefill"] = {"workload": f"spark_gateup prefill K={gu.K} N={gu.N} r={gu.r} M={Mp}",
                          "ms_per_call": round(msp, 5), "tflops": round(tf, 2),
                          "frac": round(tf / BF16_PEAK_TFLOPS, 4)}
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(up, blob, x_bits, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
