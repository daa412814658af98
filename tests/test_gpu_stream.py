"""GPU parity of the weight-streaming small-batch GEMM (the planner sends
W4A4, pre-packed W4A4 and W4A16 products with M <= 64 to it on short rows,
W4A16 with M = 5..16 on long rows (bf16 activation streamed through LDS),
pre-packed/one-call W4A4 with M = 65..128 (512-K ring stages, the waves
split into four K units and two batch halves; on long rows with K split in
two), and
pre-packed/one-call W4A4 with M = 5..64 on long rows) against the
oracle, elementwise |y - ref| <= 1e-3 + 1e-2 |ref|, on sampled outputs of
problems large enough for the planner to pick it (at least 192 workgroups).

The shapes reach the kernel's edges: batch rows that fill 1, 2, 4 and 8 of
its 16-row blocks partly, weight rows that end inside a 64-row tile (and a row
count that is not a multiple of 4, the scalar-store path), K ranges whose last
1024-K chunk is partial (some waves idle), and K splits with the split-K
reduction (bf16 activation at M = 64, K = 4096; packed activation on
K = 32768).  The one-call W4A4 GEMM and the GEMM on the pre-packed
activation must agree bit for bit (the same quantized operand, the same
kernel).
"""
import numpy as np
import pytest
import torch

import nvfp4_bit_block_amd as nv
import workloads as wl
from tests.gpu_common import assert_close, dev_bf16, device, host_bf16_f32
from tests.test_gpu_products import _quant_both

pytestmark = pytest.mark.gpu

SHAPES = [(3, 12288, 2048), (17, 12288, 1152), (50, 12290, 640), (64, 12288, 4096), (8, 12288, 2048), (40, 6144, 16384),
          (5, 6144, 16384), (16, 3072, 32768), (33, 12352, 1024),
          (65, 12288, 2048), (100, 12290, 1152), (128, 16384, 640), (97, 12352, 4096),
          (100, 6144, 8320), (128, 6160, 16384), (65, 6146, 4224)]


def _sample(M, N, seed):
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(M, min(M, 24), replace=False))
    cols = np.unique(np.concatenate([rng.choice(N, 80, replace=False), [0, N - 1]]))
    return rows, cols


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_stream_w4a4_and_packed(orc, M, N, K):
    print(f"stream w4a4 M={M} N={N} K={K}", flush=True)
    w = wl.layer_weight((N, K), seed=M + N % 97)
    x = wl.activations(M, K, seed=M * 11 + K)
    (c0, s0, g0), (c, s, g) = _quant_both(orc, w)
    isc = np.float32(orc.global_scale(x))
    y = host_bf16_f32(nv.gemm_w4a4(dev_bf16(x), torch.tensor([isc], device=device()), c, s, g))
    ac, asc, ag = nv.quantize(dev_bf16(x), static_scale=float(isc))
    yp = host_bf16_f32(nv.gemm_w4a4_packed(ac, asc, ag, c, s, g))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(yp.view(np.uint32), y.view(np.uint32), err_msg="one-call vs pre-packed")
    rows, cols = _sample(M, N, M + K)
    ref = orc.gemm_w4a4(x[rows], isc, c0[cols], s0[cols], g0)
    assert_close(y[np.ix_(rows, cols)], ref, f"stream w4a4 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(3, 12288, 2048), (17, 12288, 1152), (50, 12290, 640), (64, 12288, 4096),
                                   (8, 16384, 2048), (5, 6144, 16384), (8, 6144, 16384), (16, 6160, 8192),
                                   (12, 3072, 32768)])
def test_stream_w4a16(orc, M, N, K):
    print(f"stream w4a16 M={M} N={N} K={K}", flush=True)
    w = wl.layer_weight((N, K), seed=M + 5 + N % 89)
    x = wl.activations(M, K, seed=M * 13 + K)
    (c0, s0, g0), (c, s, g) = _quant_both(orc, w)
    y = host_bf16_f32(nv.gemm_w4a16(dev_bf16(x), c, s, g))
    rows, cols = _sample(M, N, M + K + 1)
    ref = orc.gemv_w4a16(x[rows], c0[cols], s0[cols], g0)
    assert_close(y[np.ix_(rows, cols)], ref, f"stream w4a16 {M}x{N}x{K}")
    if M <= 8:
        # the GEMV entry point takes the same kernel when no K split is needed
        yv = host_bf16_f32(nv.gemv_w4a16(dev_bf16(x), c, s, g))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(yv.view(np.uint32), y.view(np.uint32), err_msg="gemv vs gemm entry")
