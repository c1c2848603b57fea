"""GPU test of the allocation-free entry point nvfp4_quantize_no_workspace: its
outputs (codes, scale bytes, amax, s_global) must equal nvfp4_quantize's bit for
bit, on calls in a row whose second input is smaller than the first (the
library's scratch keeps the first call's partial maxima; the second call must
not read them), for bf16 and float32 input, the vectorized and the generic
kernels, and a static amax.  Calls go through the C ABI (ctypes)."""
import numpy as np
import pytest
import torch

import micro_scaled_fp4_amd as fp4
import workloads
from gpu_util import announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _same(a, b):
    return all(torch.equal(x.view(torch.uint8), y.view(torch.uint8)) for x, y in zip(a, b))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_no_workspace_quantize_equals_workspace_call(dtype):
    # 1: large (2048 amax workgroups' worth of data, the partial count at its cap),
    # 2: smaller with a much smaller amax (stale partials would raise it),
    # 3: ragged shape (generic kernels), 4: tiny
    shapes = [(4096, 8192, 1.0, 0), (300, 1024, 1e-3, 1), (37, 200, 5.0, 2), (1, 16, 1.0, 3)]
    for rows, cols, scale, seed in shapes:
        announce(f"no-workspace quantize {dtype} {rows}x{cols}")
        x32 = workloads.normal((rows, cols), 900 + seed) * np.float32(scale)
        x = torch.from_numpy(x32).to(DEV).to(dtype)
        ref = fp4.nvfp4_quantize(x)
        got = fp4.nvfp4_quantize_no_workspace(x)
        torch.cuda.synchronize()
        assert _same(ref, got), (rows, cols)
        # static amax through the same entry point
        amax = float(ref[2].item()) * 1.5
        ref_s = fp4.nvfp4_quantize(x, amax=amax)
        got_s = fp4.nvfp4_quantize_no_workspace(x, amax=amax)
        assert _same(ref_s, got_s), (rows, cols, "static")


def test_no_workspace_quantize_into_given_outputs_and_empty():
    announce("no-workspace quantize: caller outputs, empty tensor")
    x = torch.from_numpy(workloads.normal((64, 512), 950)).to(DEV).to(torch.bfloat16)
    out = (torch.empty((64, 256), dtype=torch.uint8, device=DEV),
           torch.empty((64, 32), dtype=torch.uint8, device=DEV),
           torch.empty(1, dtype=torch.float32, device=DEV),
           torch.empty(1, dtype=torch.float32, device=DEV))
    got = fp4.nvfp4_quantize_no_workspace(x, out=out)
    assert all(g is o for g, o in zip(got, out))
    assert _same(fp4.nvfp4_quantize(x), got)
    e = fp4.nvfp4_quantize_no_workspace(torch.empty((0, 16), dtype=torch.bfloat16, device=DEV))
    assert float(e[2].item()) == 0.0 and float(e[3].item()) == 1.0
