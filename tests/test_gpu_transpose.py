"""GPU parity of the two Dgrad layouts against the oracle.

nvfp4_quantize_columnwise(x) must equal the oracle's quantization of x^T bit
for bit (codes, scale bytes, global scale): the columnwise copy is a second,
independent quantization whose blocks run along the other axis.
nvfp4_dequantize_transpose must equal the transpose of the oracle's dequantized
bf16 tensor bit for bit."""
import numpy as np
import pytest
import torch

import nvfp4_bit_block_amd as nv
import workloads as wl
from tests import adversarial
from tests.gpu_common import dev, dev_bf16, device, host_u8

pytestmark = pytest.mark.gpu


def _pad_rows(xb, mult):
    r = (-xb.shape[0]) % mult
    return np.concatenate([xb, np.zeros((r, xb.shape[1]), xb.dtype)]) if r else xb


def _columnwise_matches(orc, xt, static=None):
    """xt [R, C] with R % 16 == 0: the columnwise copy of xt is the rowwise
    quantization of xt^T."""
    c0, s0, g0 = orc.quantize(np.ascontiguousarray(xt.T), static)
    st = None if static is None else torch.tensor([np.float32(static)], device=device())
    c, s, g = nv.quantize_columnwise(dev_bf16(xt), st)
    torch.cuda.synchronize()
    assert np.float32(g.cpu().item()) == g0 or (g0 == 0 and g.cpu().item() == 0)
    np.testing.assert_array_equal(host_u8(s), s0)
    np.testing.assert_array_equal(host_u8(c), c0)
    return c0, s0, g0


def test_tiny_weight(orc):
    w, _ = wl.tiny_end_to_end()                       # [256, 512]
    _columnwise_matches(orc, w)
    _columnwise_matches(orc, np.ascontiguousarray(w.T))


@pytest.mark.parametrize("case", sorted(adversarial.all_cases()))
def test_adversarial(orc, case):
    # the adversarial blocks run along rows of xb; as the columnwise copy of
    # xb^T they must come out identical (zero rows pad to a multiple of 8)
    xb, static = adversarial.all_cases()[case]
    xp = _pad_rows(xb, 8)
    _columnwise_matches(orc, np.ascontiguousarray(xp.T), static)


@pytest.mark.parametrize("rows,cols", [(16, 8), (144, 200), (4112, 72), (2048, 1536)])
def test_ragged_tiles(orc, rows, cols):
    # shapes that cut the 128 x 64 tile in both directions
    _columnwise_matches(orc, wl.heavy_tailed(rows, cols, seed=rows * 3 + cols))


def test_static_scale_saturating(orc):
    x = wl.activations(256, 384, seed=21)
    g = orc.global_scale(x)
    for f in (0.25, 4.0):
        _columnwise_matches(orc, x, static=g * f)


def test_layer_weight_differs_from_rowwise_relayout(orc):
    # the columnwise copy of a real-shaped weight is not a relayout of the
    # rowwise one: its scale set differs (blocks along the other axis)
    w = wl.layer_weight((512, 1024), seed=3)
    c0, s0, _ = _columnwise_matches(orc, w)
    _, sr, _ = orc.quantize(w)
    assert s0.shape == (1024, 512 // 16) and sr.shape == (512, 1024 // 16)
    assert not np.array_equal(np.sort(s0.ravel()), np.sort(sr.ravel()))


@pytest.mark.parametrize("rows,cols", [(8, 16), (200, 272), (1000, 2048), (6144, 1024)])
def test_dequantize_transpose(orc, rows, cols):
    xb = wl.heavy_tailed(rows, cols, seed=rows + 7 * cols)
    c0, s0, g0 = orc.quantize(xb)
    _, ref = orc.dequantize(c0, s0, g0, want_bf16=True)
    c, s, g = dev(c0), dev(s0), torch.tensor([g0], device=device())
    yt = nv.dequantize_transpose(c, s, g)
    y = nv.dequantize(c, s, g)
    torch.cuda.synchronize()
    yt_h = yt.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(yt_h, np.ascontiguousarray(ref.T))
    np.testing.assert_array_equal(yt_h, y.view(torch.int16).cpu().numpy().view(np.uint16).T)


def test_dgrad_bf16_path(orc):
    # the page's Dgrad: dX = dY * W with W reconstructed in bf16 from the
    # rowwise copy (transposed so both operands are contraction-innermost);
    # the product is a plain matmul, checked against fp64 on the oracle's
    # bf16-rounded dequantized weight
    N, K, M = 384, 512, 16
    w = wl.layer_weight((N, K), seed=31)
    c0, s0, g0 = orc.quantize(w)
    wt = nv.dequantize_transpose(dev(c0), dev(s0), torch.tensor([g0], device=device()))    # [K, N]
    dy = wl.activations(M, N, seed=32)
    dx = (dev_bf16(dy).view(torch.bfloat16).float() @ wt.float().t()).cpu().numpy()      # [M, K]
    _, wb = orc.dequantize(c0, s0, g0, want_bf16=True)      # the bf16 weight this path multiplies
    ref = wl.bf16_bits_to_f32(dy).astype(np.float64) @ wl.bf16_bits_to_f32(wb).astype(np.float64)
    np.testing.assert_allclose(dx, ref, rtol=1e-2, atol=1e-3)
