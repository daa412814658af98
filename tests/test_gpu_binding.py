"""GPU checks of the binding's stream handling and of MoE routing edge cases.

* Calls on a side stream (not the current one) allocate their temporaries on
  that stream; the results match the oracle even when the current stream
  reuses freed memory right after the call returns.
* Routing ids outside [0, E) are skipped: such a slot adds nothing to its
  token (the oracle's reading), in both modes, with and without the LoRA
  overlay.
* The routed layer is bit-identical run to run: routing scatters slots into
  expert rows in atomic order, but every row is computed on its own and the
  combine sums a token's slots in slot order.
"""
import numpy as np
import pytest
import torch

import nvfp4_bit_block_amd as nv
import workloads as wl
from tests.gpu_common import assert_close, dev, dev_bf16, host_bf16_f32
from tests.test_gpu_products import _moe_case, _quant_both

pytestmark = pytest.mark.gpu


def _scribble(nbytes):
    """Allocate and overwrite memory on the current stream (reuses blocks the
    caching allocator just got back)."""
    for _ in range(4):
        torch.full((max(nbytes, 256) // 4,), -1.0e30, dtype=torch.float32, device="cuda").neg_()


@pytest.mark.parametrize("M,N,K", [(1, 256, 2048), (37, 320, 512), (200, 256, 256)])
def test_gemm_w4a4_on_side_stream(orc, M, N, K):
    print(f"gemm side stream M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M + N + K)
    w = wl.normal_bf16(rng, (N, K), 0.02)
    x = wl.normal_bf16(rng, (M, K), 1.0)
    c0, s0, g0 = orc.quantize(w)
    isc = np.float32(orc.global_scale(x))
    ref = orc.gemm_w4a4(x, isc, c0, s0, g0)
    _, (c, s, g) = _quant_both(orc, w)
    xd = dev_bf16(x)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    # a Python float input_scale: the wrapper makes the device scalar and the
    # workspace itself, on the side stream
    y = nv.gemm_w4a4(xd, float(isc), c, s, g, stream=side)
    _scribble(nv.gemm_w4a4_workspace_size(M, N, K))
    side.synchronize()
    torch.cuda.synchronize()
    assert_close(host_bf16_f32(y), ref, f"side-stream gemm M={M}")


@pytest.mark.parametrize("mode", [0, 1])
def test_moe_on_side_stream(orc, mode):
    T, E, k, H, I = 48, 6, 2, 256, 128
    print(f"moe side stream mode={mode}", flush=True)
    x, ids, wts, cw, gw = _moe_case(orc, T, E, k, H, I, seed=77)
    kw, gkw = {}, {}
    if mode == 1:
        _, h = orc.moe(x, ids, wts, *cw, mode=0, want_h=True)
        a13 = np.full(E, orc.global_scale(x), np.float32)
        a2 = np.full(E, orc.global_scale(h), np.float32)
        kw, gkw = dict(a13=a13, a2=a2), dict(a13_scale=dev(a13), a2_scale=dev(a2))
    ref = orc.moe(x, ids, wts, *cw, mode=mode, **kw)
    xd, idd, wd = dev_bf16(x), dev(ids), dev(wts)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    y = nv.moe_grouped_gemm(xd, idd, wd, *gw, mode=mode, stream=side, **gkw)
    _scribble(nv.moe_workspace_size(T, E, k, H, I, mode))
    side.synchronize()
    torch.cuda.synchronize()
    assert_close(host_bf16_f32(y), ref, f"side-stream moe mode={mode}")


def _lora(E, H, I, r, seed):
    lo = wl.moe_lora(E, H, I, rank=r, seed=seed, std=0.05)
    return lo, {"scale": 1.25, **{n: dev_bf16(v) for n, v in lo.items()}}


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("adapter", [False, True])
def test_moe_skips_out_of_range_ids(orc, mode, adapter):
    T, E, k, H, I = 40, 5, 3, 192, 128
    print(f"moe out-of-range ids mode={mode} adapter={adapter}", flush=True)
    x, ids, wts, cw, gw = _moe_case(orc, T, E, k, H, I, seed=91)
    ids = ids.copy()
    ids[0, 0] = -1          # below the range
    ids[1, :] = E           # a token whose every slot is past the range
    ids[5, 2] = E + 7
    ids[7, 1] = -3
    kw, gkw = {}, {}
    lo_np, lo_dev = _lora(E, H, I, 16, 93) if adapter else (None, None)
    lo_ref = None if lo_np is None else {"scale": 1.25, **lo_np}
    if mode == 1:
        _, h = orc.moe(x, ids, wts, *cw, mode=0, want_h=True, lora=lo_ref)
        a13 = np.full(E, orc.global_scale(x), np.float32)
        a2 = np.full(E, orc.global_scale(h), np.float32)
        kw, gkw = dict(a13=a13, a2=a2), dict(a13_scale=dev(a13), a2_scale=dev(a2))
    ref = orc.moe(x, ids, wts, *cw, mode=mode, lora=lo_ref, **kw)
    y = nv.moe_grouped_gemm(dev_bf16(x), dev(ids), dev(wts), *gw, mode=mode, lora=lo_dev, **gkw)
    torch.cuda.synchronize()
    got = host_bf16_f32(y)
    assert_close(got, ref, f"moe out-of-range ids mode={mode} adapter={adapter}")
    assert np.all(got[1] == 0.0), "a token with no valid slot must come out zero"


@pytest.mark.parametrize("mode", [0, 1])
def test_moe_bit_identical_run_to_run(orc, mode):
    # 512 tokens x 4 slots over 8 experts: about 256 rows per expert, so the
    # atomic scatter order of the routing differs between runs
    T, E, k, H, I = 512, 8, 4, 256, 128
    print(f"moe run-to-run mode={mode}", flush=True)
    x, ids, wts, cw, gw = _moe_case(orc, 1, E, 1, H, I, seed=101)
    x = wl.activations(T, H, seed=102)
    ids, wts = wl.moe_routing(T, E, k, seed=103)
    gkw = {}
    if mode == 1:
        sc = dev(np.full(E, orc.global_scale(x), np.float32))
        gkw = dict(a13_scale=sc, a2_scale=dev(np.full(E, 0.02, np.float32)))
    xd, idd, wd = dev_bf16(x), dev(ids), dev(wts)
    outs = []
    for _ in range(4):
        y = nv.moe_grouped_gemm(xd, idd, wd, *gw, mode=mode, **gkw)
        torch.cuda.synchronize()
        outs.append(y.view(torch.int16).cpu().numpy().copy())
    for o in outs[1:]:
        assert np.array_equal(o, outs[0]), "MoE output changed between identical calls"
