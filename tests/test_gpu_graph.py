"""GPU: the calls' execution model.

- Every entry point captured in one HIP graph (torch.cuda.CUDAGraph) and
  replayed several times, with new input and unrelated eager work between the
  replays.  Each replay must give exactly the bytes the same calls give eagerly
  on the same input: the calls enqueue no memset nodes, allocate nothing and
  keep no state between calls, so a captured graph is reusable.
- Calls issued at the same time from two host threads, each on its own
  stream, give exactly the bytes of the same calls made one after another.
"""
import os
import threading

import numpy as np
import pytest
import torch

import micro_scaled_fp4_amd as fp4
import workloads
from oracle import fp4_oracle as o
from gpu_util import announce, to_gpu_bf16

pytestmark = pytest.mark.gpu

R, C = 256, 1024          # activation
N, K = 520, 1024          # weight: N rows of K


def _weights(dev):
    W = torch.from_numpy(o.bf16_bits_to_f32(workloads.gemm_w(N, K, seed=1201))).to(dev)
    qw, sw, _, gw = fp4.nvfp4_quantize(W)
    mq, ms = fp4.mxfp4_quantize(W)
    return qw, sw, gw, mq, ms


def _calls(x, w, offsets, d_amax):
    """One pass over the entry points on input x (device bf16 [R, C])."""
    qw, sw, gw, mq, ms = w
    out = []
    q, s, G, sg = fp4.nvfp4_quantize(x)                                   # computed amax
    out += [q, s, G, sg]
    out += list(fp4.nvfp4_quantize_ex(x, 8, 2))                           # block 8, scale search
    qm, sm = fp4.mxfp4_quantize(x)
    out += [qm, sm]
    out.append(fp4.fp4_dequantize(fp4.FP4_NVFP4, q, s, sg, C, torch.bfloat16))
    out.append(fp4.fp4_dequantize(fp4.FP4_MXFP4, qm, sm, None, C, torch.float32))
    out += list(fp4.hadamard_quantize(x, mode=fp4.FP4_SR, seed=77))
    out += list(fp4.hadamard_quantize_mx(x, mode=fp4.FP4_RNE))
    out.append(fp4.hadamard_rotate(x, 128, torch.bfloat16))
    out.append(fp4.fp4_scaled_gemm(fp4.FP4_NVFP4, q, s, sg, qw, sw, gw, K, 1.0, torch.bfloat16))
    out.append(fp4.fp4_scaled_gemm(fp4.FP4_MXFP4, qm, sm, None, mq, ms, None, K, 0.5, torch.float32))
    out.append(fp4.fp4_scaled_gemm(fp4.FP4_NVFP4, q, s, sg, qw, sw, gw, K, 0.25, torch.float8_e4m3fn))
    out += list(fp4.fp4_scaled_gemm_nvfp4_out(fp4.FP4_NVFP4, q, s, sg, qw, sw, gw, K, d_amax))
    out.append(fp4.fp4_grouped_gemm(fp4.FP4_NVFP4, q, s, sg, torch.stack([qw, qw]), torch.stack([sw, sw]),
                                    torch.cat([gw, gw]), offsets, K, 1.0, torch.float32))
    out.append(fp4.fp4_gemv_batched(x[:5], qw, sw, gw, K, 1.0, torch.float32))
    return out


def test_every_call_replays_in_a_graph():
    announce("graph capture and replay of every entry point")
    dev = "cuda:0"
    w = _weights(dev)
    inputs = [to_gpu_bf16(workloads.activation(R, C, seed=1210 + k)) for k in range(4)]
    x = inputs[0].clone()                       # the graph's static input buffer
    offsets = torch.tensor([0, 100, R], dtype=torch.int32, device=dev)
    d_amax = torch.tensor([3000.0], dtype=torch.float32, device=dev)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):               # first calls outside the capture
        _calls(x, w, offsets, d_amax)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = _calls(x, w, offsets, d_amax)

    for k in (1, 2, 3, 1):
        x.copy_(inputs[k])
        junk = torch.randn(1 << 20, device=dev).sum()   # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        eager = _calls(inputs[k], w, offsets, d_amax)
        torch.cuda.synchronize()
        assert len(eager) == len(captured)
        for i, (a, b) in enumerate(zip(captured, eager)):
            assert a.dtype == b.dtype and a.shape == b.shape, i
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {k}, output {i}"
        del junk


def test_gemv_register_path_replays_in_a_graph():
    """The GEMV path whose fp16 x' does not fit LDS (16 rows, K = 2560: the
    prep launch, then x' in registers) captured in a graph and replayed with
    new inputs and eager work between, byte-equal to eager calls."""
    announce("graph capture and replay of the register-x GEMV")
    dev = "cuda:0"
    Nw, Kw, B = 300, 2560, 16
    qw = torch.from_numpy(workloads.random_codes((Nw, Kw // 2), 1401)).to(dev)
    sw = torch.from_numpy(workloads.random_bytes((Nw, Kw // 16), 0x18, 0x58, 1402)).to(dev)
    gw = torch.tensor([0.02], dtype=torch.float32, device=dev)
    inputs = [to_gpu_bf16(workloads.gemv_x(B, Kw, seed=1410 + k)) for k in range(4)]
    x = inputs[0].clone()

    def call(xx):
        return fp4.fp4_gemv_batched(xx, qw, sw, gw, Kw, 1.0, torch.bfloat16)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(x)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y = call(x)
    for k in (1, 2, 3, 1):
        x.copy_(inputs[k])
        junk = torch.randn(1 << 20, device=dev).sum()
        g.replay()
        torch.cuda.synchronize()
        ref = call(inputs[k])
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.uint8), ref.view(torch.uint8)), f"replay {k}"
        del junk


def test_concurrent_calls_from_two_threads_on_two_streams():
    announce("two host threads, two streams")
    dev = "cuda:0"
    w = _weights(dev)
    qw, sw, gw = w[0], w[1], w[2]
    xs = [to_gpu_bf16(workloads.activation(R, C, seed=1300 + i)) for i in range(2)]

    def work(x):
        q, s, G, sg = fp4.nvfp4_quantize(x)
        out = [q, s, G, sg, fp4.fp4_gemv_batched(x[:8], qw, sw, gw, K, 1.0, torch.float32)]
        out += list(fp4.hadamard_quantize(x, mode=fp4.FP4_SR, seed=5))
        out.append(fp4.fp4_scaled_gemm(fp4.FP4_NVFP4, q, s, sg, qw, sw, gw, K, 1.0, torch.float32))
        return out

    serial = [work(x) for x in xs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(2)]
    results, errors = [None, None], []
    barrier = threading.Barrier(2, timeout=30)

    def run(i):
        try:
            torch.cuda.set_device(0)
            barrier.wait()
            with torch.cuda.stream(streams[i]):
                for _ in range(8):
                    results[i] = work(xs[i])
            streams[i].synchronize()
        except Exception as e:          # reported on the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,), daemon=True) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    assert all(not t.is_alive() for t in threads)
    for i in range(2):
        for j, (a, b) in enumerate(zip(results[i], serial[i])):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (i, j)


_FIRST_CALLS = r'''
import sys, threading
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
import micro_scaled_fp4_amd as fp4
import workloads
dev = "cuda:0"
torch.cuda.init()
M, N, K = 300, 520, 1024
qa = torch.from_numpy(workloads.random_codes((M, K // 2), 1))
qw = torch.from_numpy(workloads.random_codes((N, K // 2), 2))
sa = torch.from_numpy(workloads.random_bytes((M, K // 16), 0x20, 0x50, 3))
sw = torch.from_numpy(workloads.random_bytes((N, K // 16), 0x20, 0x50, 4))
sam = torch.from_numpy(workloads.random_bytes((M, K // 32), 120, 134, 5))
swm = torch.from_numpy(workloads.random_bytes((N, K // 32), 120, 134, 6))
qa, qw, sa, sw, sam, swm = (t.to(dev) for t in (qa, qw, sa, sw, sam, swm))
g = torch.ones(1, dtype=torch.float32, device=dev)
x = torch.from_numpy(workloads.normal((4, K), 7)).to(dev).to(torch.bfloat16)
K2 = 2560                      # 16 rows: the GEMV path with x' in registers
qw2 = torch.from_numpy(workloads.random_codes((N, K2 // 2), 8)).to(dev)
sw2 = torch.from_numpy(workloads.random_bytes((N, K2 // 16), 0x20, 0x50, 9)).to(dev)
x2 = torch.from_numpy(workloads.normal((16, K2), 10)).to(dev).to(torch.bfloat16)
torch.cuda.synchronize()

def work():
    return [fp4.fp4_scaled_gemm(fp4.FP4_NVFP4, qa, sa, g, qw, sw, g, K, 1.0, torch.bfloat16),
            fp4.fp4_scaled_gemm(fp4.FP4_MXFP4, qa, sam, None, qw, swm, None, K, 1.0, torch.float32),
            fp4.fp4_gemv_batched(x, qw, sw, g, K, 1.0, torch.float32),
            fp4.fp4_gemv_batched(x2, qw2, sw2, g, K2, 1.0, torch.float32)]

streams = [torch.cuda.Stream() for _ in range(2)]
results, errors = [None, None], []
barrier = threading.Barrier(2, timeout=60)

def run(i):
    try:
        torch.cuda.set_device(0)
        with torch.cuda.stream(streams[i]):
            barrier.wait()             # both threads make the library's first calls together
            results[i] = work()
        streams[i].synchronize()
    except Exception as e:
        errors.append(repr(e))

threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
for t in threads: t.start()
for t in threads: t.join(timeout=90)
assert not errors, errors
assert all(not t.is_alive() for t in threads)
serial = work()
torch.cuda.synchronize()
for i in range(2):
    for a, b in zip(results[i], serial):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
print("first-calls-ok", flush=True)
'''


def test_first_calls_of_a_fresh_process_from_two_threads():
    """The library's very first GEMM (NVFP4 and MXFP4) and GEMV calls in a
    fresh process, made at the same time from two host threads on two streams
    (each kernel's one-time per-device setup races), give the serial results."""
    import subprocess
    import sys
    announce("fresh process: first calls from two threads")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _FIRST_CALLS, root], capture_output=True, text=True,
                       timeout=110)
    assert r.returncode == 0 and "first-calls-ok" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
