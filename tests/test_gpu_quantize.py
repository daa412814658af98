"""GPU parity of nvfp4_quantize / nvfp4_dequantize against the oracle: bit-exact
codes, scale bytes, global scale and dequantized bf16."""
import numpy as np
import pytest
import torch

import nvfp4_bit_block_amd as nv
import workloads as wl
from tests import adversarial
from tests.gpu_common import dev, dev_bf16, device, host_u8

pytestmark = pytest.mark.gpu


def _gpu_quant(xb, static=None):
    x = dev_bf16(xb)
    st = None if static is None else torch.tensor([np.float32(static)], device=device())
    c, s, g = nv.quantize(x, st)
    torch.cuda.synchronize()
    return host_u8(c), host_u8(s), np.float32(g.cpu().item())


def _assert_same(orc, xb, static=None):
    c0, s0, g0 = orc.quantize(xb, static)
    c1, s1, g1 = _gpu_quant(xb, static)
    assert g1 == g0 or (g0 == 0 and g1 == 0), (g1, g0)
    np.testing.assert_array_equal(s1, s0)
    np.testing.assert_array_equal(c1, c0)
    return c0, s0, g0


def test_tiny_end_to_end(orc):
    w, x = wl.tiny_end_to_end()
    _assert_same(orc, w)
    _assert_same(orc, x)
    _assert_same(orc, x, static=orc.global_scale(x))          # the W4A4 input_scale path


@pytest.mark.parametrize("case", sorted(adversarial.all_cases()))
def test_adversarial(orc, case):
    xb, static = adversarial.all_cases()[case]
    _assert_same(orc, xb, static)


@pytest.mark.parametrize("rows,cols", [(37, 1040), (2048, 6144), (1, 16), (3, 48)])
def test_heavy_tailed_ragged(orc, rows, cols):
    _assert_same(orc, wl.heavy_tailed(rows, cols, seed=rows + cols))


def test_static_scales(orc):
    x = wl.activations(64, 2048, seed=4)
    g = orc.global_scale(x)
    for f in (0.25, 1.0, 4.0, 1e-3):       # saturating ... generous
        _assert_same(orc, x, static=g * f)


@pytest.fixture(scope="module")
def full_size(orc):
    """The 65536 x 6144 heavy-tailed tensor, quantized by both sides."""
    xb = wl.heavy_tailed(65536, 6144, seed=1)
    c1, s1, g1 = _gpu_quant(xb)
    c0, s0, g0 = orc.quantize(xb)
    return xb, (c0, s0, g0), (c1, s1, g1)


def test_full_size_bitexact(full_size):
    """The whole 65536 x 6144 tensor: every code and scale byte and the global
    scale equal the oracle's."""
    _, (c0, s0, g0), (c1, s1, g1) = full_size
    assert g1 == g0
    np.testing.assert_array_equal(s1, s0)
    np.testing.assert_array_equal(c1, c0)


def test_full_size_dequantize_bitexact(orc, full_size):
    """Dequantize of the whole 65536 x 6144 quantized tensor, bit for bit
    against the oracle's bf16 rounding of fl(fl(q s) Sg)."""
    _, (c0, s0, g0), _ = full_size
    y = nv.dequantize(dev(c0), dev(s0), torch.tensor([g0], device=device()))
    torch.cuda.synchronize()
    yb = y.view(torch.int16).cpu().numpy().view(np.uint16)
    _, ref = orc.dequantize(c0, s0, g0, want_bf16=True)
    np.testing.assert_array_equal(yb, ref)


def test_deterministic():
    xb = wl.heavy_tailed(512, 4096, seed=3)
    a = _gpu_quant(xb)
    b = _gpu_quant(xb)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_dequantize_bitexact(orc):
    for xb, static in [(wl.tiny_end_to_end()[0], None), adversarial.scale_edge_cases(),
                       (wl.heavy_tailed(300, 2064, seed=9), None)]:
        c, s, g = orc.quantize(xb, static)
        _, ref = orc.dequantize(c, s, g, want_bf16=True)
        y = nv.dequantize(dev(c), dev(s), torch.tensor([g], device=device()))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), ref)


def test_outputs_do_not_spill():
    """Guard bytes after every output buffer stay untouched."""
    xb = wl.heavy_tailed(33, 2064, seed=5)
    rows, cols = xb.shape
    pad = 4096
    codes = torch.full((rows * cols // 2 + pad,), 0xA5, dtype=torch.uint8, device=device())
    scales = torch.full((rows * cols // 16 + pad,), 0x5A, dtype=torch.uint8, device=device())
    gs = torch.full((64,), 7.0, device=device())
    nv.quantize(dev_bf16(xb), None, codes[:rows * cols // 2].view(rows, cols // 2),
                scales[:rows * cols // 16].view(rows, cols // 16), gs[:1])
    torch.cuda.synchronize()
    assert (codes[rows * cols // 2:] == 0xA5).all() and (scales[rows * cols // 16:] == 0x5A).all()
    assert (gs[1:] == 7.0).all()
    y = torch.full((rows * cols + pad,), 1234, dtype=torch.int16, device=device())
    nv.dequantize(codes[:rows * cols // 2].view(rows, cols // 2), scales[:rows * cols // 16].view(rows, cols // 16),
                  gs[:1], out=y[:rows * cols].view(rows, cols))
    torch.cuda.synchronize()
    assert (y[rows * cols:] == 1234).all()


def test_empty_is_noop():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=device())
    c, s, g = nv.quantize(x)
    assert c.shape == (0, 32) and s.shape == (0, 4)
