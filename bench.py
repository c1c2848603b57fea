#!/usr/bin/env python3
"""Benchmark of the NVFP4 / MXFP4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]   (defaults 10 / 5)

One step runs every call of the hot path once per input copy, each at its
workload's shape:
  activation   8192x8192 bf16, N(0,1), 8 outlier channels x40:
               nvfp4_quantize (dynamic amax), nvfp4_quantize (static amax),
               mxfp4_quantize, NVFP4 and MXFP4 dequantize to bf16;
               NVFP4 scale variants (static amax): blocks of 8 and 32, and the
               E4M3 scale search over +-2 codes, each with its round-trip MSE
  decode GEMV  W 27648x5120 NVFP4, x bf16 [B, 5120] quantized on the fly, B = 1, 4, 16
  prefill GEMM 8192 x 28672 x 8192, NVFP4 and MXFP4 operands, bf16 output;
               NVFP4 again with the output requantized in the epilogue to FP8 E4M3,
               and to NVFP4 at a given (calibrated) amax
  MoE          grouped GEMM, 64 experts x (N 2048, K 7168), 32768 routed rows with
               uneven expert loads, NVFP4, bf16 output, one launch
  rotate       16384x8192 bf16, 16 outlier channels x60: FWHT-128 + NVFP4, RNE and SR;
               FWHT-128 + MXFP4 (one pass), RNE and SR; FWHT-128 alone
Each call kind is captured in its own HIP graph of R back-to-back calls that
cycle through input copies totalling >= 1 GiB (more than the 256 MiB Infinity
Cache), so consecutive calls never find their inputs in cache and no host
launch overhead is timed.  HIP events on the capture/replay stream bracket
every replay.

The printed JSON line's `value` is the NVFP4 quantize throughput at a static
(calibrated) amax on the activation workload, one pass over x, in GB/s of
algorithmic bytes (x once, codes, scale bytes and the two scalars); every other
call is reported under `components`.  Calls with a computed amax (dynamic
quantize, rotation) read x twice (the global scale has to be known before any
block is encoded): their rate and HBM fraction count x once, and the bytes
they move are given beside (`bytes_moved_per_call`, `moved_GBs`).

After the timed steps the CPU-baseline leg runs the oracle on a bounded sample
of every call's workload (timed: `cpu_baseline`, with `per_call`) and compares
its outputs with the GPU's for the same sample (`parity`, mismatch counts per
call; `parity_mismatches` is their sum).  --no-cpu-baseline skips the leg.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"fp4": 10100.0, "fp16": 2500.0, "bf16": 2500.0, "fp8": 5000.0}
GiB = 1 << 30


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--only", default="", help="comma list of call names to run (profiling)")
    p.add_argument("--sweep", action="store_true",
                   help="instead of the step: throughput against size of the GEMV (B = 1, K = 5120) "
                        "and the static NVFP4 quantize (8192 columns), one JSON line per size")
    return p.parse_args()


# ------------------------------------------------------------------ helpers --
def _src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "micro_scaled_fp4_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM traffic per launch measured by rocprofv3 counters (profiles/traffic.json),
    used only while the kernel source it was measured on is unchanged."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        return json.load(f)


class Op:
    """One call kind: R calls captured in a graph, cycling over input copies."""

    def __init__(self, name, launch, n_copies, unit, per_call, peak, bound, kernel, src, moved=None):
        self.name, self.launch, self.n = name, launch, n_copies
        self.unit, self.per_call, self.peak, self.bound = unit, per_call, peak, bound
        self.kernel, self.src = kernel, src
        # bytes the call moves when it reads its input twice (a computed amax):
        # reported beside the rate on unique algorithmic bytes, not as an HBM fraction
        self.moved = moved
        self.extra = {}
        self.graph = None
        self.times_ms = []

    def capture(self, torch):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(self.n):          # eager warm-up (first-call setup outside capture)
                self.launch(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            for i in range(self.n):
                self.launch(i)
        torch.cuda.synchronize()

    def replay_timed(self, torch):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        self.graph.replay()
        e1.record()
        return e0, e1


def size_sweep(torch, fp4, dev, reps):
    """Throughput against size: each size timed as the step's calls are (a
    graph of back-to-back calls over >= 1 GiB of inputs, median per call), on
    uniformly random valid codes and scale bytes (GEMV) or N(0,1) bf16 (quantize)."""
    def timed(fn, n):
        op = Op("sweep", fn, n, "GB/s", 0, HBM_PEAK_GBS, "hbm", "", None)
        op.capture(torch)
        ts = []
        for _ in range(reps):
            e0, e1 = op.replay_timed(torch)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / n)
        return float(np.median(ts)) * 1e3

    def line(d, nbytes, us):
        d.update({"bytes_per_call": nbytes, "us_median": round(us, 2),
                  "GB_per_s": round(nbytes / us / 1e3, 1), "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)})
        print(json.dumps(d), flush=True)

    seed = 1400
    gen = torch.Generator(device=dev).manual_seed(seed)
    K = 5120
    gw = torch.tensor([0.02], dtype=torch.float32, device=dev)
    x = torch.randn(1, K, device=dev, dtype=torch.bfloat16, generator=gen)
    ws = torch.empty(fp4.gemv_workspace_bytes(1, K), dtype=torch.uint8, device=dev)
    for N in (6912, 13824, 27648, 55296, 110592, 221184):
        wbytes = N * (K // 2 + K // 16)
        n = max(2, -(-GiB // wbytes))
        Ws = [torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=dev, generator=gen) for _ in range(n)]
        Ss = [torch.randint(0x18, 0x58, (N, K // 16), dtype=torch.uint8, device=dev, generator=gen)
              for _ in range(n)]
        y = torch.empty((1, N), dtype=torch.bfloat16, device=dev)
        us = timed(lambda i: fp4.fp4_gemv_batched(x, Ws[i], Ss[i], gw, K, 1.0, torch.bfloat16,
                                                  workspace=ws, out=y), n)
        line({"call": "gemv_b1", "N": N, "K": K, "seed": seed}, wbytes + 4 + 2 * K + 2 * N, us)
        del Ws, Ss
        torch.cuda.empty_cache()
    C = 8192
    amax = torch.tensor([40.0], dtype=torch.float32, device=dev)
    for R in (256, 1024, 4096, 8192, 32768):
        n = max(2, -(-GiB // (2 * R * C)))
        Xs = [torch.randn(R, C, device=dev, dtype=torch.bfloat16, generator=gen) for _ in range(n)]
        us = timed(lambda i: fp4.nvfp4_quantize(Xs[i], amax=amax), n)
        line({"call": "nvfp4_quantize_static", "rows": R, "cols": C, "seed": seed},
             2 * R * C + R * C // 2 + R * C // 16 + 8, us)
        del Xs
        torch.cuda.empty_cache()


def same_size_copy_gbs(torch, dev, traffic_bytes, steps):
    """Read + write GB/s of a plain device copy moving traffic_bytes per call,
    timed as the calls are: a graph of back-to-back copies over >= 1 GiB of
    buffers (so no copy is served from the on-die cache), median per copy."""
    half = traffic_bytes // 2
    n = max(2, -(-GiB // traffic_bytes))
    srcs = [torch.zeros(half, dtype=torch.uint8, device=dev) for _ in range(n)]
    dsts = [torch.empty_like(t) for t in srcs]

    def copy(i):
        dsts[i].copy_(srcs[i])

    op = Op("copy", copy, n, "GB/s", 2 * half, HBM_PEAK_GBS, "hbm", "copy", None)
    op.capture(torch)
    times = []
    for _ in range(steps):
        e0, e1 = op.replay_timed(torch)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / n)
    del op, srcs, dsts
    return 2 * half / (float(np.median(times)) * 1e-3) / 1e9


def same_size_read_gbs(torch, dev, read_bytes, steps):
    """GB/s of a plain read-only pass over read_bytes per call: a row-wise max
    over an int32 [R, 4096] tensor (writing R values, 0.02% of the bytes read),
    timed as the calls are (graph over >= 1 GiB of buffers, median per call)."""
    cols = 4096
    rows = max(1, read_bytes // (4 * cols))
    nbytes = rows * cols * 4
    n = max(2, -(-GiB // nbytes))
    srcs = [torch.zeros((rows, cols), dtype=torch.int32, device=dev) for _ in range(n)]
    outs = [torch.empty(rows, dtype=torch.int32, device=dev) for _ in range(n)]

    def red(i):
        torch.amax(srcs[i], dim=1, out=outs[i])

    op = Op("read", red, n, "GB/s", nbytes, HBM_PEAK_GBS, "hbm", "amax", None)
    op.capture(torch)
    times = []
    for _ in range(steps):
        e0, e1 = op.replay_timed(torch)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / n)
    del op, srcs, outs
    return nbytes / (float(np.median(times)) * 1e-3) / 1e9


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "bench.py measures one GPU; --gpus above 1 is not supported "
                                   "(the library runs on one device per process)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import micro_scaled_fp4_amd as fp4
    import workloads

    lib = fp4.load_library()
    if args.sweep:
        size_sweep(torch, fp4, "cuda:0", max(args.steps, 5))
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    only = set(filter(None, args.only.split(",")))
    stream_of = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def bf16_from_bits(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def copies(t, total_bytes=GiB):
        n = max(2, -(-total_bytes // (t.numel() * t.element_size())))
        return [t] + [t.clone() for _ in range(n - 1)]

    ops = []
    t_setup = time.time()
    L = LegInputs()    # what the CPU-baseline leg needs

    # ---------------------------------------------------------- activation --
    R_A, C_A = 8192, 8192
    L.xa_bits = workloads.activation(R_A, C_A)
    xa = bf16_from_bits(L.xa_bits)
    xa_c = copies(xa)
    nA = len(xa_c)
    q_nv = [torch.empty((R_A, C_A // 2), dtype=torch.uint8, device=dev) for _ in range(nA)]
    s_nv = [torch.empty((R_A, C_A // 16), dtype=torch.uint8, device=dev) for _ in range(nA)]
    amax = [torch.empty(1, dtype=torch.float32, device=dev) for _ in range(nA)]
    gsc = [torch.empty(1, dtype=torch.float32, device=dev) for _ in range(nA)]
    wsp = [torch.empty(fp4.AMAX_WORKSPACE_BYTES, dtype=torch.uint8, device=dev) for _ in range(nA)]
    # the static (calibrated) amax: max |x| of the input, taken on the host
    L.static_amax = float(np.max(np.abs((L.xa_bits.astype(np.uint32) << 16).view(np.float32))))
    static_amax = torch.tensor([L.static_amax], dtype=torch.float32, device=dev)
    q_mx = [torch.empty((R_A, C_A // 2), dtype=torch.uint8, device=dev) for _ in range(nA)]
    s_mx = [torch.empty((R_A, C_A // 32), dtype=torch.uint8, device=dev) for _ in range(nA)]
    y_bf = torch.empty((R_A, C_A), dtype=torch.bfloat16, device=dev)
    elems = R_A * C_A
    b_nv = elems * 2 + elems // 2 + elems // 16 + 8
    b_nv_moved = b_nv + elems * 2        # the amax pass reads x a second time
    b_mx = elems * 2 + elems // 2 + elems // 32

    def nv_dyn(i):
        st = lib.nvfp4_quantize(P(xa_c[i]), fp4.FP4_BF16, R_A, C_A, P(q_nv[i]), P(s_nv[i]), P(amax[i]),
                                0, P(gsc[i]), P(wsp[i]), fp4.AMAX_WORKSPACE_BYTES, stream_of())
        assert st == 0, st

    def nv_static(i):
        st = lib.nvfp4_quantize(P(xa_c[i]), fp4.FP4_BF16, R_A, C_A, P(q_nv[i]), P(s_nv[i]),
                                P(static_amax), 1, P(gsc[i]), None, 0, stream_of())
        assert st == 0, st

    def mx_q(i):
        st = lib.mxfp4_quantize(P(xa_c[i]), fp4.FP4_BF16, R_A, C_A, P(q_mx[i]), P(s_mx[i]), stream_of())
        assert st == 0, st

    def nv_deq(i):
        st = lib.fp4_dequantize(fp4.FP4_NVFP4, P(q_nv[i]), P(s_nv[i]), P(gsc[i]), R_A, C_A, P(y_bf),
                                fp4.FP4_BF16, stream_of())
        assert st == 0, st

    def mx_deq(i):
        st = lib.fp4_dequantize(fp4.FP4_MXFP4, P(q_mx[i]), P(s_mx[i]), None, R_A, C_A, P(y_bf),
                                fp4.FP4_BF16, stream_of())
        assert st == 0, st

    qsrc = _src_hash("quantize.hip", "fp4_device.h")
    ops += [
        Op("nvfp4_quantize_dynamic", nv_dyn, nA, "GB/s", b_nv, HBM_PEAK_GBS, "hbm",
           "k_amax + k_nv_quant_fast", qsrc, moved=b_nv_moved),
        Op("nvfp4_quantize_static", nv_static, nA, "GB/s", b_nv, HBM_PEAK_GBS, "hbm",
           "k_nv_quant_fast", qsrc),
        Op("mxfp4_quantize", mx_q, nA, "GB/s", b_mx, HBM_PEAK_GBS, "hbm", "k_mx_quant_fast", qsrc),
        Op("nvfp4_dequantize_bf16", nv_deq, nA, "GB/s", b_nv - 4, HBM_PEAK_GBS, "hbm",
           "k_dequant_fast<NV>", qsrc),
        Op("mxfp4_dequantize_bf16", mx_deq, nA, "GB/s", b_mx, HBM_PEAK_GBS, "hbm",
           "k_dequant_fast<MX>", qsrc),
    ]

    # NVFP4 scale variants on the same tensor (static amax: the encode pass
    # alone, comparable with nvfp4_quantize_static): block sizes 8 and 32, and
    # the least-squared-error E4M3 scale search over +-2 codes at block 16.
    # Each reports the round-trip MSE of the whole tensor next to its rate.
    def roundtrip_mse(block, W):
        if block == 0:                                   # MXFP4
            q, sc = fp4.mxfp4_quantize(xa)
            y = fp4.fp4_dequantize(fp4.FP4_MXFP4, q, sc, None, C_A, torch.float32)
        else:
            q, sc, _, g = fp4.nvfp4_quantize_ex(xa, block, W, amax=static_amax)
            y = fp4.nvfp4_dequantize_ex(q, sc, g, C_A, block, torch.float32)
        d = y.double() - xa.double()
        return float((d * d).mean())

    block_mse = block_error_report(torch, fp4, xa, static_amax)
    for op in ops:
        if op.name == "nvfp4_quantize_static":
            op.extra["roundtrip_mse"] = roundtrip_mse(16, 0)
        if op.name == "mxfp4_quantize":
            op.extra["roundtrip_mse"] = roundtrip_mse(0, 0)
    q_v = [torch.empty((R_A, C_A // 2), dtype=torch.uint8, device=dev) for _ in range(nA)]
    g_v = torch.empty(1, dtype=torch.float32, device=dev)
    L.q_nv0, L.s_nv0, L.gsc0, L.amax0 = q_nv[0], s_nv[0], gsc[0], amax[0]
    L.q_mx0, L.s_mx0, L.y_bf, L.q_v0, L.s_v = q_mx[0], s_mx[0], y_bf, q_v[0], {}
    for block, W in ((8, 0), (32, 0), (16, 2)):
        s_v = [torch.empty((R_A, C_A // block), dtype=torch.uint8, device=dev) for _ in range(nA)]
        L.s_v[block] = s_v[0]

        def nv_var(i, block=block, W=W, s_v=s_v):
            st = lib.nvfp4_quantize_ex(P(xa_c[i]), fp4.FP4_BF16, R_A, C_A, block, W, P(q_v[i]),
                                       P(s_v[i]), P(static_amax), 1, P(g_v), None, 0, stream_of())
            assert st == 0, st

        name = f"nvfp4_quantize_block{block}" + (f"_search{W}" if W else "")
        op = Op(name, nv_var, nA, "GB/s", elems * 2 + elems // 2 + elems // block + 8, HBM_PEAK_GBS,
                "hbm", f"k_nv_quant_fast<block {block}{', scale search +-%d' % W if W else ''}>", qsrc)
        op.extra["roundtrip_mse"] = roundtrip_mse(block, W)
        ops.append(op)

    # --------------------------------------------------------- decode GEMV --
    Nv, Kv = 27648, 5120
    L.gemv_w_bits = workloads.gemv_weight(Nv, Kv)
    wv = bf16_from_bits(L.gemv_w_bits)
    wq0, ws0, _, gw0 = fp4.nvfp4_quantize(wv)
    L.gemv_wq, L.gemv_ws, L.gemv_gw, L.gemv = wq0, ws0, gw0, {}
    del wv
    w_bytes = wq0.numel() + ws0.numel() + 4
    nG = max(2, -(-GiB // w_bytes))
    Wq = [wq0] + [wq0.clone() for _ in range(nG - 1)]
    Wsc = [ws0] + [ws0.clone() for _ in range(nG - 1)]
    gsrc = _src_hash("gemv.hip", "fp4_device.h")
    for B in (1, 4, 16):
        xv_bits = workloads.gemv_x(B, Kv)
        xv = bf16_from_bits(xv_bits)
        yv = torch.empty((B, Nv), dtype=torch.bfloat16, device=dev)
        L.gemv[B] = (xv_bits, yv)
        wsz = fp4.gemv_workspace_bytes(B, Kv)
        wsv = torch.empty(wsz, dtype=torch.uint8, device=dev)

        def gemv(i, xv=xv, yv=yv, wsv=wsv, wsz=wsz, B=B):
            st = lib.fp4_gemv_batched(P(xv), fp4.FP4_BF16, B, P(Wq[i]), P(Wsc[i]), P(gw0), Nv, Kv,
                                      1.0, P(yv), fp4.FP4_BF16, P(wsv), wsz, stream_of())
            assert st == 0, st

        kern = ("k_gemv_fp4 (x quantized in every workgroup, W codes into the FP4 MFMA)" if B <= 4 else
                "k_gemv_xquant + k_gemv_xreg (x quantized once and dequantized once per wave into "
                "registers, W dequantized to fp16 in registers)")
        ops.append(Op(f"gemv_b{B}", gemv, nG, "GB/s", w_bytes + B * Kv * 2 + B * Nv * 2,
                      HBM_PEAK_GBS, "hbm", kern, gsrc))

    # -------------------------------------------------------- prefill GEMM --
    Mg, Ng, Kg = 8192, 28672, 8192
    ga_bits = workloads.gemm_a(Mg, Kg)
    aq_nv, as_nv, _, ga_nv = fp4.nvfp4_quantize(bf16_from_bits(ga_bits))
    aq_mx, as_mx = fp4.mxfp4_quantize(bf16_from_bits(ga_bits))
    gw_bits = workloads.gemm_w(Ng, Kg)
    wt = bf16_from_bits(gw_bits)
    L.gemm_shape, L.gemm_a_bits, L.gemm_w_bits = (Mg, Ng, Kg), ga_bits, gw_bits
    wq_nv, wsc_nv, _, gw_nv = fp4.nvfp4_quantize(wt)
    wq_mx, wsc_mx = fp4.mxfp4_quantize(wt)
    rotation_error = rotation_error_report(torch, fp4, bf16_from_bits(workloads.gemm_a(Mg, Kg)[:1024]),
                                           wt, (wq_nv, wsc_nv, gw_nv), (wq_mx, wsc_mx))
    # calibrated amax of D for the NVFP4-output GEMM: 1.25 x the largest |x W^T|
    # over the first 1024 rows, from torch's float32 product of the bf16 inputs
    a_cal = bf16_from_bits(ga_bits[:1024]).float()
    L.d_amax = float(np.float32(1.25 * float(torch.mm(a_cal, wt.float().t().contiguous()).abs().max())))
    del wt, a_cal
    Dg = torch.empty((Mg, Ng), dtype=torch.bfloat16, device=dev)
    L.Dg = Dg
    flops = 2 * Mg * Ng * Kg
    msrc = _src_hash("gemm.hip", "fp4_device.h")

    def gemm_nv(i):
        st = lib.fp4_scaled_gemm(fp4.FP4_NVFP4, P(aq_nv), P(as_nv), P(ga_nv), P(wq_nv), P(wsc_nv),
                                 P(gw_nv), 1.0, Mg, Ng, Kg, P(Dg), fp4.FP4_BF16, stream_of())
        assert st == 0, st

    D8 = torch.empty((Mg, Ng), dtype=torch.float8_e4m3fn, device=dev)
    L.D8 = D8

    def gemm_nv_e4m3(i):
        st = lib.fp4_scaled_gemm(fp4.FP4_NVFP4, P(aq_nv), P(as_nv), P(ga_nv), P(wq_nv), P(wsc_nv),
                                 P(gw_nv), 1.0, Mg, Ng, Kg, P(D8), fp4.FP4_E4M3, stream_of())
        assert st == 0, st

    # NVFP4 output at the calibrated amax of D (computed above)
    d_amax = torch.tensor([L.d_amax], dtype=torch.float32, device=dev)
    Dq4 = torch.empty((Mg, Ng // 2), dtype=torch.uint8, device=dev)
    Dsc4 = torch.empty((Mg, Ng // 16), dtype=torch.uint8, device=dev)
    Dgs4 = torch.empty(1, dtype=torch.float32, device=dev)
    L.Dq4, L.Dsc4, L.Dgs4 = Dq4, Dsc4, Dgs4

    def gemm_nv_nv4(i):
        st = lib.fp4_scaled_gemm_nvfp4_out(fp4.FP4_NVFP4, P(aq_nv), P(as_nv), P(ga_nv), P(wq_nv),
                                           P(wsc_nv), P(gw_nv), 1.0, Mg, Ng, Kg, P(Dq4), P(Dsc4),
                                           P(d_amax), P(Dgs4), stream_of())
        assert st == 0, st

    def gemm_mx(i):
        st = lib.fp4_scaled_gemm(fp4.FP4_MXFP4, P(aq_mx), P(as_mx), None, P(wq_mx), P(wsc_mx), None,
                                 1.0, Mg, Ng, Kg, P(Dg), fp4.FP4_BF16, stream_of())
        assert st == 0, st

    ops += [
        Op("gemm_nvfp4", gemm_nv, 3, "TFLOP/s", flops, MFMA_PEAK_TFLOPS["fp16"], "mfma",
           "k_gemm<NV> (fp16 MFMA after exact in-register dequant)", msrc),
        Op("gemm_mxfp4", gemm_mx, 3, "TFLOP/s", flops, MFMA_PEAK_TFLOPS["fp4"], "mfma",
           "k_gemm_mx8 (scaled FP4 MFMA, 8 waves, persistent)", msrc),
        Op("gemm_nvfp4_e4m3_out", gemm_nv_e4m3, 3, "TFLOP/s", flops, MFMA_PEAK_TFLOPS["fp16"], "mfma",
           "k_gemm<NV, E4M3 out> (output requantized to FP8 E4M3 in the epilogue)", msrc),
        Op("gemm_nvfp4_nvfp4_out", gemm_nv_nv4, 3, "TFLOP/s", flops, MFMA_PEAK_TFLOPS["fp16"],
           "mfma", "k_gemm<NV, NVFP4 out> (output requantized to NVFP4 at a given amax)", msrc),
    ]

    # ------------------------------------------------------ MoE grouped GEMM --
    # 64 experts with N = 2048, K = 7168 (one launch); 32768 routed rows
    # (4096 tokens x top-8) with uneven expert loads; NVFP4, bf16 output
    E_m, N_m, K_m = 64, 2048, 7168
    sizes_m = workloads.moe_group_sizes(E_m, 32768)
    M_m = sum(sizes_m)
    am_bits = workloads.gemm_a(M_m, K_m, seed=workloads.SEED_MOE)
    aq_m, as_m, _, ga_m = fp4.nvfp4_quantize(bf16_from_bits(am_bits))
    L.moe_a_bits, L.moe_w_bits = am_bits, []
    # 8 distinct expert weights (N(0, 0.02^2), each quantized with its own
    # tensor scale), stored 8 times over: the values do not change the work
    wq_m = torch.empty((E_m * N_m, K_m // 2), dtype=torch.uint8, device=dev)
    ws_m = torch.empty((E_m * N_m, K_m // 16), dtype=torch.uint8, device=dev)
    gb_m = torch.empty(E_m, dtype=torch.float32, device=dev)
    for e8 in range(8):
        L.moe_w_bits.append(workloads.gemm_w(N_m, K_m, seed=workloads.SEED_MOE + 1 + e8))
        wt8 = bf16_from_bits(L.moe_w_bits[-1])
        q, sc, _, g = fp4.nvfp4_quantize(wt8)
        for e in range(e8, E_m, 8):
            wq_m[e * N_m:(e + 1) * N_m] = q
            ws_m[e * N_m:(e + 1) * N_m] = sc
            gb_m[e] = g[0]
        del wt8
    offs_m = torch.tensor([0] + list(np.cumsum(sizes_m)), dtype=torch.int32, device=dev)
    D_m = torch.empty((M_m, N_m), dtype=torch.bfloat16, device=dev)
    L.moe_offsets, L.D_m = np.concatenate([[0], np.cumsum(sizes_m)]), D_m

    def moe(i):
        st = lib.fp4_grouped_gemm(fp4.FP4_NVFP4, P(aq_m), P(as_m), P(ga_m), P(wq_m), P(ws_m), P(gb_m),
                                  1.0, E_m, P(offs_m), M_m, N_m, K_m, P(D_m), fp4.FP4_BF16, stream_of())
        assert st == 0, st

    ops.append(Op("grouped_gemm_moe_nvfp4", moe, 3, "TFLOP/s", 2 * M_m * N_m * K_m,
                  MFMA_PEAK_TFLOPS["fp16"], "mfma", "k_gemm<NV, grouped> (64 experts, one launch)",
                  msrc))

    # -------------------------------------------------------------- rotate --
    R_H, C_H = 16384, 8192
    L.rot_bits = workloads.rotate_input(R_H, C_H)
    xh = bf16_from_bits(L.rot_bits)
    xh_c = copies(xh)
    nH = len(xh_c)
    qh = torch.empty((R_H, C_H // 2), dtype=torch.uint8, device=dev)
    sh = torch.empty((R_H, C_H // 16), dtype=torch.uint8, device=dev)
    ah = torch.empty(1, dtype=torch.float32, device=dev)
    gh = torch.empty(1, dtype=torch.float32, device=dev)
    wh = torch.empty(fp4.AMAX_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    eh = R_H * C_H
    b_h = eh * 2 + eh // 2 + eh // 16 + 8
    b_h_moved = b_h + eh * 2                         # computed amax: x is read twice
    hsrc = _src_hash("hadamard.hip", "fp4_device.h")
    for mode, nm in ((fp4.FP4_RNE, "rne"), (fp4.FP4_SR, "sr")):
        def had(i, mode=mode):
            st = lib.hadamard_quantize(P(xh_c[i]), fp4.FP4_BF16, R_H, C_H, 128, mode,
                                       ctypes.c_uint64(workloads.SEED_SR), P(qh), P(sh), P(ah), 0,
                                       P(gh), P(wh), fp4.AMAX_WORKSPACE_BYTES, stream_of())
            assert st == 0, st
        ops.append(Op(f"hadamard_quantize_{nm}", had, nH, "GB/s", b_h, HBM_PEAK_GBS, "hbm",
                      "k_had_amax + k_had_quant", hsrc, moved=b_h_moved))
    # the leg's GPU rotation at a given amax (max |x| of the unrotated input)
    L.rot_amax = float(np.max(np.abs((L.rot_bits.astype(np.uint32) << 16).view(np.float32))))
    L.seed_sr = workloads.SEED_SR
    rot_amax_t = torch.tensor([L.rot_amax], dtype=torch.float32, device=dev)

    def rot_given(mode):
        st = lib.hadamard_quantize(P(xh_c[0]), fp4.FP4_BF16, R_H, C_H, 128, mode,
                                   ctypes.c_uint64(workloads.SEED_SR), P(qh), P(sh), P(rot_amax_t), 1,
                                   P(gh), None, 0, stream_of())
        assert st == 0, st
        torch.cuda.synchronize()
    L.rot_given, L.qh, L.sh = rot_given, qh, sh

    # rotation alone (offline W H, bf16 -> bf16) and rotation + MXFP4 (one pass)
    yh = torch.empty((R_H, C_H), dtype=torch.bfloat16, device=dev)
    qhm = torch.empty((R_H, C_H // 2), dtype=torch.uint8, device=dev)
    shm = torch.empty((R_H, C_H // 32), dtype=torch.uint8, device=dev)
    L.yh, L.qhm, L.shm = yh, qhm, shm

    def had_rot(i):
        st = lib.hadamard_rotate(P(xh_c[i]), fp4.FP4_BF16, R_H, C_H, 128, P(yh), fp4.FP4_BF16,
                                 stream_of())
        assert st == 0, st

    def had_mx(i, mode=fp4.FP4_RNE):
        st = lib.hadamard_quantize_mx(P(xh_c[i]), fp4.FP4_BF16, R_H, C_H, 128, mode,
                                      ctypes.c_uint64(workloads.SEED_SR), P(qhm), P(shm), stream_of())
        assert st == 0, st

    def had_mx_sr(i):
        had_mx(i, fp4.FP4_SR)

    ops += [
        Op("hadamard_rotate_bf16", had_rot, nH, "GB/s", eh * 4, HBM_PEAK_GBS, "hbm",
           "k_had_rotate (FWHT-128 alone)", hsrc),
        Op("hadamard_quantize_mx", had_mx, nH, "GB/s", eh * 2 + eh // 2 + eh // 32, HBM_PEAK_GBS,
           "hbm", "k_had_quant_mx (FWHT-128 + MXFP4, one pass)", hsrc),
        Op("hadamard_quantize_mx_sr", had_mx_sr, nH, "GB/s", eh * 2 + eh // 2 + eh // 32, HBM_PEAK_GBS,
           "hbm", "k_had_quant_mx (FWHT-128 + MXFP4, stochastic rounding, one pass)", hsrc),
    ]

    L.ops = {op.name: op for op in ops}
    if only:
        ops = [op for op in ops if op.name in only]
    setup_s = time.time() - t_setup

    # ------------------------------------------------------------- capture --
    for op in ops:
        op.capture(torch)
    # graph replays reproduce the eager result (checked on the dynamic quantize)
    if any(op.name == "nvfp4_quantize_dynamic" for op in ops):
        ref = [t.clone() for t in (q_nv[0], s_nv[0], amax[0], gsc[0])]
        q_nv[0].zero_()
        next(op for op in ops if op.name == "nvfp4_quantize_dynamic").graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (q_nv[0], s_nv[0], amax[0], gsc[0])):
            assert torch.equal(a, b), "graph replay differs from eager result"

    # ------------------------------------------------------------- warm-up --
    for _ in range(args.warmup):
        for op in ops:
            op.graph.replay()
    torch.cuda.synchronize()

    # --------------------------------------------------------- timed steps --
    events = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for op in ops:
            events.append((op, *op.replay_timed(torch)))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for op, e0, e1 in events:
        op.times_ms.append(e0.elapsed_time(e1) / op.n)
    ms_per_step = (t1 - t0) * 1000.0 / args.steps

    # context: a plain device copy of 1 GiB (read + write) on the same GPU
    src = torch.empty(GiB // 2, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst
    # and a copy moving as many bytes per call as the decode GEMV (W 27648x5120),
    # captured and replayed like the calls above: the rate a kernel of that size
    # reaches, launch ramp and tail included
    gemv_ops = [op for op in ops if op.name.startswith("gemv_b")]
    copy_small_gbs = read_small_gbs = None
    if gemv_ops:
        copy_small_gbs = same_size_copy_gbs(torch, dev, gemv_ops[0].per_call, max(args.steps, 3))
        read_small_gbs = same_size_read_gbs(torch, dev, gemv_ops[0].per_call, max(args.steps, 3))

    traffic = load_traffic()
    comps = {}
    for op in ops:
        t_ms = float(np.mean(op.times_ms))
        if op.unit == "GB/s":
            achieved = op.per_call / (t_ms * 1e-3) / 1e9
        else:
            achieved = op.per_call / (t_ms * 1e-3) / 1e12
        tr = traffic.get(op.name)
        tr_bytes = tr["bytes_per_call"] if tr and tr.get("src") == op.src else None
        comps[op.name] = {
            "us_per_call": round(t_ms * 1e3, 2),
            "us_median": round(float(np.median(op.times_ms)) * 1e3, 2),
            "us_p10": round(float(np.percentile(op.times_ms, 10)) * 1e3, 2),
            "us_p90": round(float(np.percentile(op.times_ms, 90)) * 1e3, 2),
            "achieved": round(achieved, 1), "unit": op.unit, "peak": op.peak,
            "frac": round(achieved / op.peak, 4), "bound": op.bound,
            ("bytes_per_call" if op.unit == "GB/s" else "flop_per_call"): op.per_call,
            "kernels": op.kernel, "calls_per_replay": op.n, "traffic": tr_bytes,
        }
        comps[op.name].update(op.extra)
        if op.moved is not None:
            comps[op.name]["bytes_moved_per_call"] = op.moved
            comps[op.name]["moved_GBs"] = round(op.moved / (t_ms * 1e-3) / 1e9, 1)
            comps[op.name]["moved_note"] = ("the amax pass reads x before the encode pass reads it again; "
                                            "the rate and HBM fraction above count x once")
        if op.unit == "GB/s":
            comps[op.name]["frac_of_copy"] = round(achieved / copy_gbs, 4)
        if op in gemv_ops:
            comps[op.name]["frac_of_same_size_copy"] = round(achieved / copy_small_gbs, 4)
            comps[op.name]["frac_of_same_size_read"] = round(achieved / read_small_gbs, 4)
        if op.name in ("gemm_nvfp4", "gemm_nvfp4_e4m3_out", "gemm_nvfp4_nvfp4_out"):
            comps[op.name]["frac_of_fp4_peak"] = round(achieved / MFMA_PEAK_TFLOPS["fp4"], 4)

    head = comps.get("nvfp4_quantize_static") or next(iter(comps.values()))
    enc = head
    result = {
        "metric": "NVFP4 quantize GB/s; FP4 scaled-GEMM TFLOPS; GEMV GB/s (% roofline)",
        "value": head["achieved"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in, e2m1+e4m3 out",
        "data": "synthetic (seeded)",
        "config": {
            "workload": "activation quantization: bf16 8192x8192, N(0,1), 8 outlier channels x40, "
                        "nvfp4_quantize at a static (calibrated) amax, one pass over x",
            "rows": R_A, "cols": C_A,
            "value_bytes_per_call": b_nv,
            "seeds": {"tiny": workloads.SEED_TINY, "activation": workloads.SEED_ACTIVATION,
                      "gemv": workloads.SEED_GEMV, "gemm": workloads.SEED_GEMM,
                      "rotate": workloads.SEED_ROTATE, "stochastic_rounding": workloads.SEED_SR,
                      "moe": workloads.SEED_MOE},
            "value_bytes_note": "x once (bf16) + codes + scale bytes + 2 floats; the computed-amax call "
                                "(components.nvfp4_quantize_dynamic) is rated on the same unique bytes",
            "step_also_runs": "mxfp4_quantize, NV/MX dequantize, NVFP4 block 8/32 and scale-search "
                              "variants (8192x8192); GEMV W 27648x5120 "
                              "B=1,4,16; GEMM 8192x28672x8192 NVFP4 and MXFP4 (bf16 out), NVFP4 "
                              "(E4M3 out, NVFP4 out); MoE grouped GEMM 64x2048x7168 (32768 rows); FWHT+NVFP4 "
                              "16384x8192 RNE and SR",
        },
        "roofline": {
            "kernel": "k_nv_quant_fast (NVFP4 encode pass; timed alone as the static-amax call)",
            "bound": "hbm", "achieved": enc["achieved"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(enc["achieved"] / HBM_PEAK_GBS, 4), "traffic": enc["traffic"],
            "algorithmic_bytes_per_launch": b_nv,
            "avg_launch_us": enc["us_per_call"],
        },
        "components": comps,
        "block_mse": block_mse,
        "rotation_error": rotation_error,
        "context": {"device_copy_GBs_read_plus_write": round(copy_gbs, 1),
                    "note": "torch copy_ of 512 MiB, for reference against the 8 TB/s peak",
                    "device_copy_gemv_size_GBs": None if copy_small_gbs is None else round(copy_small_gbs, 1),
                    "gemv_size_note": "torch copy_ moving the GEMV's bytes per call (half read, half "
                                      "written), as a graph cycling over >= 1 GiB of buffers",
                    "device_read_gemv_size_GBs": None if read_small_gbs is None else round(read_small_gbs, 1),
                    "gemv_read_note": "torch amax over rows of an int32 tensor of the GEMV's bytes per "
                                      "call (read only), as a graph cycling over >= 1 GiB of buffers"},
        "setup_s": round(setup_s, 1),
    }

    if not args.no_cpu_baseline and not only:
        import contextlib
        with contextlib.redirect_stdout(sys.stderr):     # stdout carries the JSON line only
            result["cpu_baseline"], result["parity"] = oracle_leg(L, args.cpu_seconds)
        result["parity_mismatches"] = int(sum(v["mismatches"] for v in result["parity"].values()))
    print(json.dumps(result), flush=True)


def block_error_report(torch, fp4, x, amax):
    """Squared error per 16-value block of the activation after an NVFP4 and an
    MXFP4 round trip (the same 16-value blocks for both): mean, p99, and the
    means over blocks that hold an outlier channel (columns with mean |x| > 10,
    the x40 channels) and over the other blocks; NV / MX ratio of the means.
    Information only: not timed."""
    R, C = x.shape
    xf = x.float()
    outlier_cols = (xf.abs().mean(dim=0) > 10.0)
    outlier_blocks = outlier_cols.reshape(C // 16, 16).any(dim=1)          # [C/16]

    def stats(y):
        e = ((y.double() - xf.double()) ** 2).reshape(R, C // 16, 16).mean(dim=2)
        o = e[:, outlier_blocks]
        c = e[:, ~outlier_blocks]
        p99 = float(torch.quantile(e.flatten().float(), 0.99))    # 4.2 M blocks
        return {"mean": float(e.mean()), "p99": p99, "outlier_blocks_mean": float(o.mean()),
                "clean_blocks_mean": float(c.mean())}

    q, sc, _, g = fp4.nvfp4_quantize(x, amax=amax)
    nv = stats(fp4.fp4_dequantize(fp4.FP4_NVFP4, q, sc, g, C, torch.float32))
    qm, sm = fp4.mxfp4_quantize(x)
    mx = stats(fp4.fp4_dequantize(fp4.FP4_MXFP4, qm, sm, None, C, torch.float32))
    return {"nvfp4": nv, "mxfp4": mx, "nv_over_mx_mean": round(nv["mean"] / mx["mean"], 4),
            "outlier_block_fraction": round(float(outlier_blocks.float().mean()), 5),
            "block": 16, "workload": "activation 8192x8192 (static amax for NVFP4)"}


def rotation_error_report(torch, fp4, x, w, w_nv, w_mx):
    """Relative Frobenius error against x W^T (float32 product of the bf16
    inputs) of the FP4 linear layer, unrotated and with both operands rotated
    ((x H)(W H)^T = x W^T), for NVFP4 and MXFP4, on 1024 rows of the prefill
    activations (outlier channels x40) and the full 28672 x 8192 weight.
    Information only: not timed."""
    K = x.shape[1]
    exact = torch.mm(x.float(), w.float().t().contiguous()).double()
    ref = float(exact.norm())

    def rel(D):
        return round(float((D.double() - exact).norm()) / ref, 5)

    def gemm(fmt, a, w_ops):
        if fmt == fp4.FP4_NVFP4:
            return fp4.fp4_scaled_gemm(fmt, a[0], a[1], a[3], w_ops[0], w_ops[1], w_ops[2], K, 1.0,
                                       torch.float32)
        return fp4.fp4_scaled_gemm(fmt, a[0], a[1], None, w_ops[0], w_ops[1], None, K, 1.0,
                                   torch.float32)

    out = {"shape": [x.shape[0], w.shape[0], K]}
    out["nvfp4_plain"] = rel(gemm(fp4.FP4_NVFP4, fp4.nvfp4_quantize(x), w_nv))
    rw = fp4.hadamard_quantize(w)
    out["nvfp4_rotated"] = rel(gemm(fp4.FP4_NVFP4, fp4.hadamard_quantize(x), (rw[0], rw[1], rw[3])))
    out["mxfp4_plain"] = rel(gemm(fp4.FP4_MXFP4, fp4.mxfp4_quantize(x), w_mx))
    out["mxfp4_rotated"] = rel(gemm(fp4.FP4_MXFP4, fp4.hadamard_quantize_mx(x), fp4.hadamard_quantize_mx(w)))
    return out


class LegInputs:
    """What the CPU-baseline leg needs: the seeded inputs as the workload
    generators made them (host arrays), and, per call, a way to run the GPU call
    once more and the tensors it writes."""

    def __init__(self):
        self.ops = {}
        self.dev = "cuda:0"

    def run(self, name):
        import torch
        self.ops[name].launch(0)
        torch.cuda.synchronize()


def oracle_leg(L, seconds):
    """The CPU-baseline leg, the only part of the benchmark that runs the oracle.

    For every call kind the NumPy oracle computes a bounded sample of the same
    workload from the seeded inputs (never from GPU results), timed on the host
    (element-wise NumPy on one thread; the float64 products of the GEMM/GEMV
    references through BLAS), and its outputs are compared with what the GPU
    call wrote for the same sample:
      - quantize, dequantize, scale variants, rotations: byte-exact on sampled rows
        (the headline's oracle runs for about `seconds` on 256-row slices);
      - GEMV: every output of B = 1, 4, 16 (the oracle quantizes all of W), within
        the tolerance rule, after W's codes, scale bytes and tensor scale are
        compared byte for byte;
      - GEMMs: sampled entries (and, for the NVFP4 output, sampled 16-column
        blocks) within the tolerance rule, requantized outputs checked to be
        admissible under it (the same checks as the GPU tests).
    Returns (cpu_baseline, parity)."""
    import torch
    from oracle import fp4_oracle as o

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from requant_checks import check_e4m3_against_reference, check_nvfp4_against_reference

    rng = np.random.default_rng(2024)
    parity, per_call = {}, {}
    GB = 1e9

    def host(t):
        return t.detach().cpu().numpy()

    def bits16(t):
        return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)

    def f32_bits(v):
        return int(np.array(v, np.float32).view(np.uint32))

    def record(name, checked, mismatches, what):
        parity[name] = {"checked": int(checked), "mismatches": int(mismatches), "what": what}

    def timed(fn):
        t0 = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t0

    def rate(name, nbytes, dt, sample, unit="GB/s"):
        per_call[name] = {"value": round(nbytes / dt / (GB if unit == "GB/s" else 1e12), 5),
                          "unit": unit, "seconds": round(dt, 2), "sample": sample}

    # ------------------------------------------------------------ activation --
    xf = o.bf16_bits_to_f32(L.xa_bits)
    R, C = xf.shape
    per_el = 2 + 0.5 + 1 / 16
    # headline: the static-amax quantize on 256-row slices for about `seconds`
    L.run("nvfp4_quantize_static")
    q_g, s_g, g_g = host(L.q_nv0), host(L.s_nv0), host(L.gsc0)
    n_rows, bad, r0 = 0, 0, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds and n_rows < R:
        q, sc, _, sg = o.nvfp4_quantize(xf[r0:r0 + 256], amax=L.static_amax)
        bad += int(np.count_nonzero(q != q_g[r0:r0 + 256]) + np.count_nonzero(sc != s_g[r0:r0 + 256]))
        bad += int(f32_bits(sg) != f32_bits(g_g[0]))
        n_rows += 256
        r0 += 256
    dt = time.perf_counter() - t0
    head_value = round(n_rows * C * per_el / dt / GB, 4)
    head_sample = (f"nvfp4_quantize at the static amax on rows 0..{n_rows - 1} (256-row slices) of the "
                   f"{R}x{C} activation, {dt:.1f} s, element-wise NumPy on one thread")
    record("nvfp4_quantize_static", n_rows * C * (0.5 + 1 / 16), bad,
           f"codes and scale bytes of rows 0..{n_rows - 1} and s_global, byte-exact")
    rate("nvfp4_quantize_static", n_rows * C * per_el, dt, f"rows 0..{n_rows - 1} (256-row slices)")

    rows = np.sort(rng.choice(R, 128, replace=False))
    xs = xf[rows]

    def quant_check(name, fn_gpu_out, fn_oracle, nbytes_per_el, what):
        L.run(name)
        gpu = fn_gpu_out()
        ref, dt = timed(fn_oracle)
        bad = sum(int(np.count_nonzero(np.asarray(a) != np.asarray(b))) for a, b in zip(gpu, ref))
        record(name, sum(np.asarray(a).size for a in gpu), bad, what)
        rate(name, len(rows) * C * nbytes_per_el, dt, f"{len(rows)} sampled rows")

    # dynamic amax: G over the whole tensor, then the sampled rows at that G
    def dyn_oracle():
        G = o.global_amax(xf)
        q, sc, G2, sg = o.nvfp4_quantize(xs, amax=G)
        return q, sc, np.array([f32_bits(G2), f32_bits(sg)])

    quant_check("nvfp4_quantize_dynamic",
                lambda: (host(L.q_nv0)[rows], host(L.s_nv0)[rows],
                         np.array([f32_bits(host(L.amax0)[0]), f32_bits(host(L.gsc0)[0])])),
                dyn_oracle, 2 + per_el, "codes, scale bytes of 128 rows; computed amax and s_global bits")
    quant_check("mxfp4_quantize", lambda: (host(L.q_mx0)[rows], host(L.s_mx0)[rows]),
                lambda: o.mxfp4_quantize(xs), 2 + 0.5 + 1 / 32, "codes and E8M0 bytes of 128 rows")

    # dequantize: the oracle dequantizes its own quantization of the sampled rows
    qn, sn, _, sgn = o.nvfp4_quantize(xs, amax=L.static_amax)
    qm, sm = o.mxfp4_quantize(xs)
    L.run("nvfp4_quantize_static")
    L.run("mxfp4_quantize")
    for name, fn in (("nvfp4_dequantize_bf16", lambda: o.f32_to_bf16_bits(o.nvfp4_dequantize(qn, sn, sgn, C))),
                     ("mxfp4_dequantize_bf16", lambda: o.f32_to_bf16_bits(o.mxfp4_dequantize(qm, sm, C)))):
        L.run(name)
        gpu = bits16(L.y_bf)[rows]
        ref, dt = timed(fn)
        record(name, gpu.size, np.count_nonzero(gpu != ref), f"bf16 bits of {len(rows)} rows")
        rate(name, len(rows) * C * per_el, dt, f"{len(rows)} sampled rows")

    # NVFP4 scale variants (static amax)
    for block, W in ((8, 0), (32, 0), (16, 2)):
        name = f"nvfp4_quantize_block{block}" + (f"_search{W}" if W else "")
        quant_check(name, lambda: (host(L.q_v0)[rows], host(L.s_v[block])[rows]),
                    lambda b=block, w=W: o.nvfp4_quantize_ex(xs, b, w, amax=L.static_amax)[:2],
                    2 + 0.5 + 1 / block, f"codes and scale bytes of 128 rows (block {block}, search {W})")

    # ---------------------------------------------------------------- GEMV --
    Wf = o.bf16_bits_to_f32(L.gemv_w_bits)
    (Wq, Ws, _, gw), dt_w = timed(lambda: o.nvfp4_quantize(Wf))
    bad = int(np.count_nonzero(Wq != host(L.gemv_wq)) + np.count_nonzero(Ws != host(L.gemv_ws)))
    bad += int(f32_bits(gw) != f32_bits(host(L.gemv_gw)[0]))
    record("gemv_weight_quantize", Wq.size + Ws.size + 1, bad,
           "W 27648x5120 codes, scale bytes and s_global (the GEMV's operand), byte-exact")
    K = Wf.shape[1]
    for B, (x_bits, y_t) in L.gemv.items():
        name = f"gemv_b{B}"
        L.run(name)
        y = host(y_t.float())
        (ref, mag), dt = timed(lambda: o.gemv_ref(o.bf16_bits_to_f32(x_bits), Wq, Ws, gw, 1.0, K))
        ok, err, bound = o.gemm_within_tolerance(y, ref, mag, out_bf16=True)
        record(name, y.size, np.count_nonzero(err > bound),
               "every output within the tolerance rule (bf16 output)")
        rate(name, Wq.size + Ws.size + 4 + B * K * 2 + B * y.shape[1] * 2, dt,
             "the whole call (float64 product through BLAS; W quantized by the oracle beforehand)")
    del Wf

    # ---------------------------------------------------------------- GEMM --
    M, N, Kg = L.gemm_shape
    Af_all = o.bf16_bits_to_f32(L.gemm_a_bits)
    Wf_all = o.bf16_bits_to_f32(L.gemm_w_bits)
    GA, GW = o.global_amax(Af_all), o.global_amax(Wf_all)
    ii = rng.integers(0, M, 1024)
    jj = rng.integers(0, N, 1024)
    ui, ia = np.unique(ii, return_inverse=True)
    uj, ja = np.unique(jj, return_inverse=True)
    ops_nv = (o.nvfp4_quantize(Af_all[ui], amax=GA), o.nvfp4_quantize(Wf_all[uj], amax=GW))
    Ah_nv = o.nv_operand_f64(ops_nv[0][0], ops_nv[0][1], ops_nv[0][3], Kg)[ia]
    Wh_nv = o.nv_operand_f64(ops_nv[1][0], ops_nv[1][1], ops_nv[1][3], Kg)[ja]
    qma, sma = o.mxfp4_quantize(Af_all[ui])
    qmw, smw = o.mxfp4_quantize(Wf_all[uj])
    Ah_mx = o.mx_operand_f64(qma, sma, Kg)[ia]
    Wh_mx = o.mx_operand_f64(qmw, smw, Kg)[ja]
    ti, tj = torch.from_numpy(ii).to(L.dev), torch.from_numpy(jj).to(L.dev)
    for name, Ah, Wh, out in (("gemm_nvfp4", Ah_nv, Wh_nv, "bf16"), ("gemm_mxfp4", Ah_mx, Wh_mx, "bf16"),
                              ("gemm_nvfp4_e4m3_out", Ah_nv, Wh_nv, "e4m3")):
        L.run(name)
        got = L.Dg[ti, tj] if out == "bf16" else L.D8.view(torch.uint8)[ti, tj]
        ref = np.sum(Ah * Wh, axis=1)
        mag = np.sum(np.abs(Ah * Wh), axis=1)
        if out == "bf16":
            ok, err, bound = o.gemm_within_tolerance(host(got.float()), ref, mag, True)
            record(name, len(ii), np.count_nonzero(err > bound), "1024 sampled entries within the tolerance rule")
        else:
            try:   # every byte admissible; the open fraction is reported, not capped
                open_frac = check_e4m3_against_reference(host(got), ref, mag, "bench sample", max_open=1.0)
                bad = 0
            except AssertionError:
                open_frac, bad = None, 1
            record(name, len(ii), bad, "1024 sampled E4M3 bytes admissible under the tolerance rule "
                                       "(1 = the check failed)")
            parity[name]["open_fraction"] = open_frac
    # NVFP4 output: 32 sampled (row, 16-column block) pairs
    rb = rng.integers(0, M, 32)
    cb = rng.integers(0, N // 16, 32)
    L.run("gemm_nvfp4_nvfp4_out")
    q4, s4, g4 = host(L.Dq4), host(L.Dsc4), float(host(L.Dgs4)[0])
    refs, mags = [], []
    for r, c in zip(rb, cb):
        a = o.nvfp4_quantize(Af_all[r:r + 1], amax=GA)
        w = o.nvfp4_quantize(Wf_all[16 * c:16 * c + 16], amax=GW)
        ref, mag = o.scaled_gemm_ref(o.nv_operand_f64(a[0], a[1], a[3], Kg),
                                     o.nv_operand_f64(w[0], w[1], w[3], Kg), 1.0)
        refs.append(ref[0])
        mags.append(mag[0])
    qs = np.stack([q4[r, 8 * c:8 * c + 8] for r, c in zip(rb, cb)])
    ss = np.stack([s4[r, c:c + 1] for r, c in zip(rb, cb)])
    try:   # the 32 blocks as the rows of one [32, 16] output; open fractions reported, not capped
        opens = check_nvfp4_against_reference(qs, ss, g4, np.stack(refs), np.stack(mags), L.d_amax,
                                              "bench blocks", max_open=1.0)
        bad = 0
    except AssertionError:
        opens, bad = None, 1
    record("gemm_nvfp4_nvfp4_out", 32, bad, "32 sampled 16-column blocks (codes, scale bytes, tensor "
                                            "scale) admissible under the tolerance rule (1 = the check failed)")
    parity["gemm_nvfp4_nvfp4_out"]["open_fraction_blocks_elements"] = opens
    # the GEMM oracle's rate: a 64 x 1024 slice of the product, scaled by FLOP
    s_rows = min(64, len(Ah_nv))
    _, dt = timed(lambda: o.scaled_gemm_ref(Ah_nv[:s_rows], Wh_nv, 1.0))
    rate("gemm_nvfp4", 2 * s_rows * len(Wh_nv) * Kg, dt,
         f"{s_rows} x {len(Wh_nv)} x {Kg} slice of the float64 product (BLAS), operands dequantized "
         "beforehand; scaled by FLOP", unit="TFLOP/s")
    del Af_all, Wf_all

    # ------------------------------------------------------------------ MoE --
    Am = o.bf16_bits_to_f32(L.moe_a_bits)
    GAm = o.global_amax(Am)
    offs = L.moe_offsets
    L.run("grouped_gemm_moe_nvfp4")
    Dm = L.D_m
    bad, checked = 0, 0
    t0 = time.perf_counter()
    for e in rng.choice(len(offs) - 1, 4, replace=False):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi == lo:
            continue
        r = np.sort(rng.choice(np.arange(lo, hi), min(16, hi - lo), replace=False))
        Wfe = o.bf16_bits_to_f32(L.moe_w_bits[e % 8])
        ce = np.sort(rng.choice(Wfe.shape[0], 128, replace=False))
        a = o.nvfp4_quantize(Am[r], amax=GAm)
        w = o.nvfp4_quantize(Wfe[ce], amax=o.global_amax(Wfe))
        ref, mag = o.scaled_gemm_ref(o.nv_operand_f64(a[0], a[1], a[3], Am.shape[1]),
                                     o.nv_operand_f64(w[0], w[1], w[3], Am.shape[1]), 1.0)
        got = host(Dm[torch.from_numpy(r).to(L.dev)][:, torch.from_numpy(ce).to(L.dev)].float())
        ok, err, bound = o.gemm_within_tolerance(got, ref, mag, True)
        bad += int(np.count_nonzero(err > bound))
        checked += got.size
    record("grouped_gemm_moe_nvfp4", checked, bad,
           "16 rows x 128 columns of 4 sampled experts within the tolerance rule")
    per_call["grouped_gemm_moe_nvfp4"] = {"seconds": round(time.perf_counter() - t0, 2),
                                          "sample": "parity sample only (operand quantization included)"}
    del Am

    # ------------------------------------------------------------- rotation --
    xh = o.bf16_bits_to_f32(L.rot_bits)
    rows_h = np.sort(rng.choice(xh.shape[0], 32, replace=False))
    xhs = xh[rows_h]
    for nm, mode in (("rne", 0), ("sr", 1)):
        name = f"hadamard_quantize_{nm}"
        L.rot_given(mode)     # the GPU call at the given amax (the dynamic amax is checked by the tests)
        gq, gs_ = host(L.qh)[rows_h], host(L.sh)[rows_h]
        # the oracle: rotate and quantize the sampled rows at the given amax; SR bits by flat index
        def fn(nm=nm):
            if nm == "rne":
                y = o.fwht_orthonormal(xhs)
                return o.nvfp4_quantize(y, amax=L.rot_amax)[:2]
            y = o.fwht_orthonormal(xhs)
            idx = rows_h[:, None].astype(np.int64) * xh.shape[1] + np.arange(xh.shape[1])[None, :]
            bits = o.sr_bits_at(idx, L.seed_sr)
            return o.nvfp4_quantize(y, amax=L.rot_amax, rounding="sr", sr_bits=bits)[:2]
        ref, dt = timed(fn)
        bad = int(np.count_nonzero(gq != ref[0]) + np.count_nonzero(gs_ != ref[1]))
        record(name, gq.size + gs_.size, bad, "codes and scale bytes of 32 rows at a given amax")
        rate(name, len(rows_h) * xh.shape[1] * per_el, dt, "32 sampled rows (one pass, given amax)")
    L.run("hadamard_rotate_bf16")
    gy = bits16(L.yh)[rows_h]
    ref, dt = timed(lambda: o.f32_to_bf16_bits(o.fwht_orthonormal(xhs)))
    record("hadamard_rotate_bf16", gy.size, np.count_nonzero(gy != ref), "bf16 bits of 32 rows")
    rate("hadamard_rotate_bf16", len(rows_h) * xh.shape[1] * 4, dt, "32 sampled rows")
    L.run("hadamard_quantize_mx")
    gq, gs_ = host(L.qhm)[rows_h], host(L.shm)[rows_h]
    ref, dt = timed(lambda: o.hadamard_quantize_mx(xhs))
    record("hadamard_quantize_mx", gq.size + gs_.size,
           np.count_nonzero(gq != ref[0]) + np.count_nonzero(gs_ != ref[1]), "codes and E8M0 bytes of 32 rows")
    rate("hadamard_quantize_mx", len(rows_h) * xh.shape[1] * (2 + 0.5 + 1 / 32), dt, "32 sampled rows")
    # stochastic rounding on rows 0..31, whose flat element indices (the SR
    # counters) are the same in the 32-row sample as in the whole tensor
    L.run("hadamard_quantize_mx_sr")
    gq, gs_ = host(L.qhm)[:32], host(L.shm)[:32]
    ref, dt = timed(lambda: o.hadamard_quantize_mx(xh[:32], rounding="sr", seed=L.seed_sr))
    record("hadamard_quantize_mx_sr", gq.size + gs_.size,
           np.count_nonzero(gq != ref[0]) + np.count_nonzero(gs_ != ref[1]), "codes and E8M0 bytes of rows 0..31")
    rate("hadamard_quantize_mx_sr", 32 * xh.shape[1] * (2 + 0.5 + 1 / 32), dt, "rows 0..31")

    cpu = {"value": head_value, "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": head_sample,
           "host_cpu_count": os.cpu_count(), "host_affinity": len(os.sched_getaffinity(0)),
           "blas_threads": os.environ.get("OMP_NUM_THREADS"),
           "per_call": per_call}
    return cpu, parity


if __name__ == "__main__":
    main()
