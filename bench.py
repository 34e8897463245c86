"""Benchmark of the DV-SSQ linear layer on one MI355X.

Headline (one JSON line on stdout): effective weight GB/s of the Spark-shaped
up_proj decode call (K=2560, N=10240, r=16, H_256, M=1) = the packed layer's
bytes (algo_bytes) per call / time per call.  A "step" is one
dvssq_linear_decode call: rotation, t = x_rot V^T, both weight tiers, the
low-rank term, any split-K reduction and the bf16 scatter, in one launch.

Beside it: the roofline of that kernel (HBM bound; achieved = algorithmic
bytes per launch -- packed layer + x + y -- over the average launch time
measured with HIP events on the launch stream), a table of the other decode
shapes and of the prefill GEMM (TFLOP/s against the bf16 dense MFMA peak),
and the oracle timed on the host cores as a baseline.

Inputs are synthetic and already resident in HBM when timing starts.  The
timed blobs are random, well-formed packed layers of each shape (timing does
not depend on the code values); C distinct copies totalling >= 1 GiB are
cycled so the 256 MB last-level cache cannot serve repeats.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_spark_up_m1_traffic.json")
KERNEL_SOURCES = ("decode_gemv.hip", "decode_small.hip", "dvssq_internal.h", "api.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--decode-m", type=int, default=1)
    ap.add_argument("--prefill-steps", type=int, default=30)
    ap.add_argument("--table-steps", type=int, default=400, help="calls per secondary decode shape")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-table", action="store_true", help="skip the secondary shapes")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--only-prefill", action="store_true",
                    help="time only the prefill shapes (for kernel traces of the prefill path)")
    ap.add_argument("--only-attention", action="store_true",
                    help="time only the attention shapes (for kernel traces of the attention kernel)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one 256 MiB device copy (scale reference for HBM byte counters)")
    return ap.parse_args()


def kernel_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bit_linear_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


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
    """Average ms per call over `steps` back-to-back calls between two events on
    the launch stream, after `warmup` untimed calls.  fn(i) takes blob copy
    i mod C; the timed calls continue the index after the warm-up's, so the
    copies the warm-up just read are the last ones the timed calls reach."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(warmup, warmup + steps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


class Runner:
    """Decode / prefill calls of one layer shape through the C ABI."""

    def __init__(self, dv, torch, lay, M, M_max, min_bytes=1 << 30, max_copies=256):
        import synth
        self.torch, self.lay, self.M = torch, lay, M
        self.L, self.blob, self.copies, self.C = make_copies(dv, torch, lay, M_max, min_bytes, max_copies)
        self.x_bits = synth.activations_bf16(0, lay.outlier_tag or lay.name, M, lay.K)
        self.x = torch.from_numpy(self.x_bits.view(np.int16)).to("cuda").view(torch.bfloat16)
        self.y = torch.empty((M, lay.N), dtype=torch.bfloat16, device="cuda")
        self.ws = dv.device_buffer(self.L.ws_bytes)
        self.stream = torch.cuda.current_stream().cuda_stream
        self.ptrs = [self.copies[i].data_ptr() for i in range(self.C)]
        self.lib, self.Lp = dv.lib(), ctypes.byref(self.L)
        self.dv = dv

    def decode(self, i):
        rc = self.lib.dvssq_linear_decode(self.Lp, self.ptrs[i % self.C], self.x.data_ptr(), self.y.data_ptr(),
                                          self.M, self.ws.data_ptr(), 0, self.stream)
        if rc:
            raise self.dv.DvssqError(rc, "dvssq_linear_decode")

    def prefill(self, i):
        rc = self.lib.dvssq_linear_prefill(self.Lp, self.ptrs[i % self.C], self.x.data_ptr(), self.y.data_ptr(),
                                           self.M, self.ws.data_ptr(), 0, self.stream)
        if rc:
            raise self.dv.DvssqError(rc, "dvssq_linear_prefill")

    def algo_bytes(self):
        return self.L.algo_bytes + 2 * self.M * (self.lay.K + self.lay.N)

    def flops(self):
        lay, M = self.lay, self.M
        return 2.0 * M * lay.N * lay.K + 2.0 * M * lay.r * (lay.n_seg * lay.K + lay.N)

    def free(self):
        del self.copies, self.x, self.y, self.ws
        self.torch.cuda.empty_cache()


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
            "sample": f"{reps} complete fp64 oracle forwards of the headline layer (spark_up, M={x_bits.shape[0]}) "
                      f"on the same packed layer and x, {el:.1f} s"}


def traffic_record():
    """HBM bytes per launch from the committed counter summary, if it was taken on
    the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_hash") != kernel_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


class MlpRunner:
    """The gated MLP block (fused gate+up, then down) through dvssq_mlp_decode,
    both layers' blobs cycled over replicas like the single-layer runs."""

    def __init__(self, dv, torch, gu, down, M, prefill=False):
        import synth
        self.M, self.gu, self.down = M, gu, down
        mm, nb, nc = (M, 256 << 20, 16) if prefill else (32, 1 << 30, 128)
        self.fn = dv.mlp_prefill if prefill else dv.mlp_decode
        self.Lg, _, self.cg, self.C = make_copies(dv, torch, gu, mm, nb, nc)
        self.Ld, _, self.cd, Cd = make_copies(dv, torch, down, mm, nb, nc)
        self.C = min(self.C, Cd)
        x_bits = synth.activations_bf16(0, gu.outlier_tag or gu.name, M, gu.K)
        self.x = torch.from_numpy(x_bits.view(np.int16)).to("cuda").view(torch.bfloat16)
        self.y = torch.empty((M, down.N), dtype=torch.bfloat16, device="cuda")
        self.ws = dv.device_buffer(dv.mlp_ws_bytes(self.Lg, self.Ld))
        self.stream = torch.cuda.current_stream().cuda_stream
        self.dv = dv

    def call(self, i):
        k = i % self.C
        self.fn(self.Lg, self.cg[k].data_ptr(), self.Ld, self.cd[k].data_ptr(), self.x.data_ptr(),
                self.y.data_ptr(), self.M, self.ws.data_ptr(), 0, self.stream)

    def algo_bytes(self):
        return self.Lg.algo_bytes + self.Ld.algo_bytes

    def flops(self):
        return 2.0 * self.M * (self.gu.N * self.gu.K + self.down.N * self.down.K)

    def free(self):
        del self.cg, self.cd, self.ws


def dense_table(dv, torch, layers, steps):
    """Materialization of the fused gate+up layer into dense bf16, and a plain
    bf16 GEMM (torch's library GEMM) on that dense weight at M = 2048, beside
    this library's prefill of the packed layer."""
    import torch.nn.functional as F
    lay = layers["spark_gateup"]
    r = Runner(dv, torch, lay, 2048, 2048, min_bytes=256 << 20, max_copies=16)
    w = torch.empty((lay.N, lay.K), dtype=torch.bfloat16, device="cuda")

    def mat(i):
        dv.materialize(r.L, r.ptrs[i % r.C], w, r.stream)
    t, _ = time_calls(torch, mat, steps, 3)
    out = [{"workload": f"spark_gateup materialize to dense bf16 (N={lay.N}, K={lay.K})",
            "us_per_call": round(t * 1e3, 2), "gbs_written": round(2.0 * lay.N * lay.K / (t * 1e-3) / 1e9, 1)}]
    y = torch.empty((2048, lay.N), dtype=torch.bfloat16, device="cuda")
    t, _ = time_calls(torch, lambda i: torch.matmul(r.x, w.t(), out=y), steps, 3)
    tf = 2.0 * 2048 * lay.N * lay.K / (t * 1e-3) / 1e12
    out.append({"workload": "dense bf16 GEMM (torch.matmul) on the materialized spark_gateup, M=2048",
                "us_per_call": round(t * 1e3, 2), "tflops": round(tf, 1),
                "frac_mfma_bf16": round(tf / BF16_PEAK_TFLOPS, 4)})
    del w, y
    r.free()
    return out


def ceiling_table(dv, torch, steps):
    """The achievable-bandwidth reference: dvssq_stream_read (a plain streaming
    read, nothing computed) of the packed sizes of spark_up (one decode layer)
    and of the fused gate+up layer, over >= 1 GiB of distinct bytes cycled like
    the decode runs."""
    out = []
    total = 1 << 30
    buf = torch.empty(total + (64 << 20), dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    for name, nbytes in (("spark_up packed layer", 15_918_080), ("spark_gateup packed layer", 32_245_760)):
        span = (nbytes + 4095) // 4096 * 4096
        C = total // span
        base = buf.data_ptr()
        t, _ = time_calls(torch, lambda i: dv.stream_read(base + (i % C) * span, nbytes, sink, st), steps, 20)
        g = nbytes / (t * 1e-3) / 1e9
        out.append({"workload": f"streaming read of {nbytes} B ({name}), no computation: achievable ceiling",
                    "us_per_call": round(t * 1e3, 3), "gbs": round(g, 1), "frac_hbm": round(g / HBM_PEAK_GBS, 4)})
    del buf, sink
    return out


def fwht_table(dv, torch, steps):
    """dvssq_fwht alone (bf16 in, bf16 out) on the prefill activation shapes:
    HBM-bound, 2MK bytes read + 2MK written per call."""
    import synth
    out = []
    src = torch.from_numpy(synth.activations_bf16(0, "fwht", 4096, 6144).view(np.int16)).cuda().view(torch.bfloat16)
    for M, K, b in ((2048, 2560, 256), (4096, 2048, 2048), (4096, 6144, 2048)):
        x = src[:M, :K].contiguous()
        xr = torch.empty_like(x)
        st = torch.cuda.current_stream().cuda_stream
        t, _ = time_calls(torch, lambda i: dv.fwht(x, xr, M, K, b, st), steps, 3)
        g = 4.0 * M * K / (t * 1e-3) / 1e9
        out.append({"workload": f"fwht M={M} K={K} H_{b}", "us_per_call": round(t * 1e3, 2), "gbs": round(g, 1),
                    "frac_hbm": round(g / HBM_PEAK_GBS, 4)})
        del x, xr
    del src
    return out


def prefill_table(dv, torch, layers, steps):
    table = fwht_table(dv, torch, steps)
    for name, m in (("spark_gateup", 512), ("spark_gateup", 2048), ("minicpm_gate", 4096),
                    ("minicpm_down", 4096), ("spark_down", 512)):
        r = Runner(dv, torch, layers[name], m, m, min_bytes=256 << 20, max_copies=16)
        t, _ = time_calls(torch, r.prefill, steps, 3)
        tf = r.flops() / (t * 1e-3) / 1e12
        table.append({"workload": f"{name} prefill M={m}", "us_per_call": round(t * 1e3, 2),
                      "tflops": round(tf, 1), "frac_mfma_bf16": round(tf / BF16_PEAK_TFLOPS, 4)})
        r.free()
    table += dense_table(dv, torch, layers, steps)
    r = MlpRunner(dv, torch, layers["spark_gateup"], layers["spark_down"], 2048, prefill=True)
    t, _ = time_calls(torch, r.call, steps, 3)
    tf = r.flops() / (t * 1e-3) / 1e12
    table.append({"workload": "spark MLP block (gate+up, GELU, down) prefill M=2048", "us_per_call": round(t * 1e3, 2),
                  "tflops": round(tf, 1), "frac_mfma_bf16": round(tf / BF16_PEAK_TFLOPS, 4)})
    r.free()
    return table


def attention_pairs(Mq, Nk, window):
    """(query, visible key) pairs of one head: causal, optional sliding window."""
    p = np.arange(Nk - Mq, Nk, dtype=np.int64)
    lo = np.maximum(0, p - window + 1) if window > 0 else np.zeros_like(p)
    return int((p - lo + 1).sum())


def attention_table(dv, torch, steps=20):
    """dvssq_kvbss_attention on the Spark attention heads (16 query heads, 4 KV
    heads, head_dim 256): a 2048-token prefill of a full layer and of a sliding
    (window 512) layer, against the dense bf16 matrix-core peak (algorithmic
    FLOPs: 4 D per (query, visible key) pair and head, Q K^T and P V); and one
    decode step over a 32768-token context (1 and 8 sequences), against the HBM
    peak (algorithmic bytes: the visible keys' K and V, q and o)."""
    import synth
    out = []
    D = 256
    scale = float(np.float32(1.10 / math.sqrt(D)))
    st = torch.cuda.current_stream().cuda_stream
    B, Mq, Nk, Hq, Hkv = 1, 2048, 2048, 16, 4
    q, k, v = synth.attention_qkv(0, "spark_prefill", B, Mq, Nk, Hq, Hkv, D)
    qd, kd, vd = (torch.from_numpy(a.view(np.int16)).cuda() for a in (q, k, v))
    o = torch.empty_like(qd)
    for window in (0, 512):
        sh = dv.AttnShape(B=B, Mq=Mq, Nk=Nk, Hq=Hq, Hkv=Hkv, D=D, window=window, scale=scale, haze=12.0)
        t, _ = time_calls(torch, lambda i: dv.kvbss_attention(sh, qd, kd, vd, o, None, st), steps, 3)
        fl = 4.0 * D * Hq * B * attention_pairs(Mq, Nk, window)
        tf = fl / (t * 1e-3) / 1e12
        out.append({"workload": f"KV-BSS attention prefill, Spark heads (Hq=16, Hkv=4, D=256), {Mq} tokens, "
                                f"window {window or 'none'}", "us_per_call": round(t * 1e3, 2),
                    "tflops": round(tf, 1), "frac_mfma_bf16": round(tf / BF16_PEAK_TFLOPS, 4)})
    del qd, kd, vd, o
    Nk = 32768
    q, k, v = synth.attention_qkv(0, "spark_decode", 1, 1, Nk, Hq, Hkv, D)
    for B in (1, 8):
        # B sequences: the one generated sequence's q, k and v repeated (same timing, distinct memory)
        qd, kd, vd = (torch.from_numpy(np.ascontiguousarray(np.repeat(a, B, axis=0)).view(np.int16)).cuda()
                      for a in (q, k, v))
        o = torch.empty_like(qd)
        sh = dv.AttnShape(B=B, Mq=1, Nk=Nk, Hq=Hq, Hkv=Hkv, D=D, window=0, scale=scale, haze=12.0)
        ws = dv.device_buffer(max(dv.kvbss_attention_ws_bytes(sh), 1))
        t, _ = time_calls(torch, lambda i: dv.kvbss_attention(sh, qd, kd, vd, o, ws, st), steps, 3)
        nbytes = B * (2 * Nk * Hkv * D * 2 + 2 * 2 * Hq * D)
        g = nbytes / (t * 1e-3) / 1e9
        out.append({"workload": f"KV-BSS attention decode step, Spark heads, {Nk}-token context, {B} sequence(s)",
                    "us_per_call": round(t * 1e3, 2), "gbs": round(g, 1), "frac_hbm": round(g / HBM_PEAK_GBS, 4)})
        del qd, kd, vd, o, ws
    return out


def quantize_table(dv, torch, layers, steps=3):
    """dvssq_quantize (weights to packed layer, on the GPU) on the spark MLP
    shapes, sketch width l = r + 8 and two power iterations."""
    import synth
    out = []
    for name in ("spark_gateup", "spark_down"):
        lay = layers[name]
        l = lay.r + 8
        L = dv.pack_info(lay.N, lay.K, lay.r, lay.block, lay.n_seg)
        W = torch.from_numpy(synth.weights_bf16(0, lay).view(np.int16)).cuda()
        om = torch.from_numpy(np.stack([synth.sketch(0, lay, s, l) for s in range(lay.n_seg)])).cuda()
        blob = dv.device_buffer(L.blob_bytes)
        ws = dv.device_buffer(dv.quantize_ws_bytes(L, l))
        st = torch.cuda.current_stream().cuda_stream
        t, _ = time_calls(torch, lambda i: dv.quantize(L, W, om, l, 2, blob, ws, st), steps, 1)
        out.append({"workload": f"{name} quantize on the GPU (N={lay.N}, K={lay.K}, r={lay.r}, l={l}, 2 power "
                                f"iterations)", "ms_per_call": round(t, 2)})
        del W, om, blob, ws
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the layer runs on a single GPU; "
              "how it would shard over several is described in the design notes, not run.", file=sys.stderr)
        sys.exit(2)
    import torch

    import bit_linear_amd as dv
    import synth

    torch.cuda.set_device(0)
    layers = {l.name: l for w in synth.WORKLOADS.values() for l in w.layers}
    if args.only_prefill:
        print(json.dumps({"prefill_table": prefill_table(dv, torch, layers, args.prefill_steps)}), flush=True)
        return
    if args.only_attention:
        print(json.dumps({"attention_table": attention_table(dv, torch)}), flush=True)
        return
    up = layers["spark_up"]
    M = args.decode_m
    head = Runner(dv, torch, up, M, 32)
    ms, wall = time_calls(torch, head.decode, args.steps, args.warmup)
    gbs = head.L.algo_bytes / (ms * 1e-3) / 1e9
    achieved = head.algo_bytes() / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8*i8->i32+f32",
        "arithmetic": "INT4/INT8 codes times the rotated activations held as 15-bit integers (two int8 planes) "
                      "on the int8 matrix cores (exact int32 products); group and row scales and all sums in "
                      "fp32; bf16 output",
        "data": "synthetic",
        "config": {"workload": f"spark_up decode K={up.K} N={up.N} r={up.r} H_{up.block} M={M}",
                   "packed_bytes": head.L.algo_bytes, "blob_copies": head.C, "wall_s": round(wall, 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_record(),
                     "kernel": "gemv_kernel", "algo_bytes_per_launch": head.algo_bytes(),
                     "us_per_launch": round(ms * 1e3, 3)},
    }
    head_blob, head_x = head.blob, head.x_bits
    head.free()

    if args.copy_probe:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    if not args.no_table:
        table = ceiling_table(dv, torch, args.table_steps)
        for name, Ms in (("spark_up", (4, 16, 32)), ("spark_down", (1, 8, 32)), ("minicpm_gate", (1,)),
                         ("minicpm_down", (1,)), ("spark_gateup", (1,))):
            for m in Ms:
                r = Runner(dv, torch, layers[name], m, 32)
                t, _ = time_calls(torch, r.decode, args.table_steps, 20)
                g = r.algo_bytes() / (t * 1e-3) / 1e9
                table.append({"workload": f"{name} decode M={m}", "us_per_call": round(t * 1e3, 3),
                              "gbs": round(g, 1), "frac_hbm": round(g / HBM_PEAK_GBS, 4)})
                r.free()
        for m in (1, 4):
            r = MlpRunner(dv, torch, layers["spark_gateup"], layers["spark_down"], m)
            t, _ = time_calls(torch, r.call, args.table_steps, 20)
            g = r.algo_bytes() / (t * 1e-3) / 1e9
            table.append({"workload": f"spark MLP block (gate+up, GELU, down) decode M={m}",
                          "us_per_call": round(t * 1e3, 3), "gbs": round(g, 1), "frac_hbm": round(g / HBM_PEAK_GBS, 4)})
            r.free()
        table += prefill_table(dv, torch, layers, args.prefill_steps)
        table += attention_table(dv, torch)
        table += quantize_table(dv, torch, layers)
        out["table"] = table
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(up, head_blob, head_x, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
