"""The Python binding rejects mistyped, misshaped, non-contiguous and host
tensors before any address reaches the library (no GPU needed: every check
below fails before a HIP call is made)."""
import pytest
import torch

import nvfp4_bit_block_amd as nv

T, E, K_TOP, H, I = 8, 4, 2, 64, 128


def _moe_args(**over):
    a = dict(
        x=torch.zeros((T, H), dtype=torch.bfloat16),
        topk_ids=torch.zeros((T, K_TOP), dtype=torch.int32),
        topk_weights=torch.zeros((T, K_TOP), dtype=torch.float32),
        w13_codes=torch.zeros((E, 2 * I, H // 2), dtype=torch.uint8),
        w13_scales=torch.zeros((E, 2 * I, H // 16), dtype=torch.uint8),
        w13_global=torch.zeros(E, dtype=torch.float32),
        w2_codes=torch.zeros((E, H, I // 2), dtype=torch.uint8),
        w2_scales=torch.zeros((E, H, I // 16), dtype=torch.uint8),
        w2_global=torch.zeros(E, dtype=torch.float32),
    )
    a.update(over)
    return a


def test_moe_rejects_int64_ids():
    # torch.topk returns int64 indices; read as int32 pairs they would route
    # half the slots to expert 0
    ids = torch.topk(torch.randn(T, E), K_TOP, dim=1).indices
    assert ids.dtype == torch.int64
    with pytest.raises(TypeError, match="topk_ids"):
        nv.moe_grouped_gemm(**_moe_args(topk_ids=ids))


def test_moe_rejects_bad_weights_and_shapes():
    with pytest.raises(TypeError, match="topk_weights"):
        nv.moe_grouped_gemm(**_moe_args(topk_weights=torch.zeros((T, K_TOP), dtype=torch.float16)))
    with pytest.raises(ValueError, match="topk_weights"):
        nv.moe_grouped_gemm(**_moe_args(topk_weights=torch.zeros((T, K_TOP + 1), dtype=torch.float32)))
    with pytest.raises(ValueError, match="w13_scales"):
        nv.moe_grouped_gemm(**_moe_args(w13_scales=torch.zeros((E, 2 * I, H // 8), dtype=torch.uint8)))
    with pytest.raises(ValueError, match="w2_codes"):
        nv.moe_grouped_gemm(**_moe_args(w2_codes=torch.zeros((E, I, H // 2), dtype=torch.uint8)))
    with pytest.raises(TypeError, match="x"):
        nv.moe_grouped_gemm(**_moe_args(x=torch.zeros((T, H), dtype=torch.float32)))
    with pytest.raises(ValueError, match="a13_scale"):
        nv.moe_grouped_gemm(**_moe_args(), mode=nv.MODE_W4A4)


def test_moe_rejects_noncontiguous_and_host_tensors():
    x_t = torch.zeros((H, T), dtype=torch.bfloat16).t()
    with pytest.raises(ValueError, match="contiguous"):
        nv.moe_grouped_gemm(**_moe_args(x=x_t))
    # every dtype and shape is right: the first device check fails
    with pytest.raises(ValueError, match="CUDA"):
        nv.moe_grouped_gemm(**_moe_args())


def test_gemm_and_gemv_reject_mismatched_weights():
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    wc = torch.zeros((32, 64), dtype=torch.uint8)
    ws = torch.zeros((32, 8), dtype=torch.uint8)
    g = torch.ones(1, dtype=torch.float32)
    with pytest.raises(TypeError, match="x"):
        nv.gemv_w4a16(x.float(), wc, ws, g)
    with pytest.raises(ValueError, match="CUDA"):
        nv.gemv_w4a16(x, wc, ws, g)
    with pytest.raises(ValueError, match="contiguous"):
        nv.gemm_w4a4(torch.zeros((128, 4), dtype=torch.bfloat16).t(), 1.0, wc, ws, g)
    with pytest.raises(TypeError, match="codes"):
        nv.dequantize(wc.to(torch.int8), ws, g)
