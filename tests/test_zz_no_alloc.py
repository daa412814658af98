"""nvfp4_quantize_noalloc (the entry point for callers that cannot allocate)
against nvfp4_quantize with a caller workspace: bit-identical codes, scales
and global scale, on two dynamic calls in a row (the second smaller, so it
reads back fewer partial maxima than the first left in the shared scratch)
and in static mode.  Calls go straight through the C ABI."""
import ctypes

import numpy as np
import pytest
import torch

import nvfp4_bit_block_amd as nv
import workloads as wl
from tests.gpu_common import dev_bf16, host_u8

pytestmark = pytest.mark.gpu


def _noalloc(x, static=None):
    L = nv.lib()
    f = L.nvfp4_quantize_noalloc
    f.restype = ctypes.c_int32
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 5
    rows, cols = x.shape
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=x.device)
    g = torch.empty(1, dtype=torch.float32, device=x.device)
    st = f(x.data_ptr(), rows, cols, None if static is None else static.data_ptr(), codes.data_ptr(),
           scales.data_ptr(), g.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, L.nvfp4_last_error().decode()
    return codes, scales, g


def _same(a, b, what):
    for u, v, n in zip(a, b, ("codes", "scales", "global scale")):
        assert np.array_equal(host_u8(u.view(torch.uint8)), host_u8(v.view(torch.uint8))), f"{what}: {n} differ"


def test_noalloc_equals_workspace_quantize(orc):
    shapes = [(4096, 6144), (300, 512)]      # 768 partial maxima, then far fewer
    for i, (rows, cols) in enumerate(shapes):
        print(f"noalloc dynamic call {i}: {rows}x{cols}", flush=True)
        xb = wl.heavy_tailed(rows, cols, seed=20 + i)
        x = dev_bf16(xb)
        got = _noalloc(x)
        ref = nv.quantize(x)
        torch.cuda.synchronize()
        _same(got, ref, f"dynamic call {i} ({rows}x{cols})")
        if i == 1:
            c0, s0, g0 = orc.quantize(xb)
            assert np.array_equal(host_u8(got[0]), c0) and np.array_equal(host_u8(got[1]), s0)
            assert np.float32(got[2].cpu().item()) == g0


def test_noalloc_static_mode():
    xb = wl.activations(64, 2048, seed=7)
    x = dev_bf16(xb)
    sc = torch.tensor([0.0015], dtype=torch.float32, device=x.device)
    got = _noalloc(x, sc)
    ref = nv.quantize(x, static_scale=sc)
    torch.cuda.synchronize()
    _same(got, ref, "static")
