"""GPU parity of the MoE layer with a bf16 LoRA overlay on its NVFP4 experts
(one LoRA-A shared by the experts, one LoRA-B per expert, on the gate/up and
the down projection) against the oracle, elementwise
|y - ref| <= 1e-3 + 1e-2 |ref|.

The rank-r intermediate z = bf16(A v) is rounded on both sides from sums
taken in different orders, so a z can differ by one bf16 ulp; its effect on
an output is scale * |B| * 2^-8 |z| for one term of the rank sum, far inside
the tolerance at these magnitudes.  Both modes are covered; in W4A4 the
adapter reads the bf16 activations (tokens and h), not their quantization.
"""
import numpy as np
import pytest
import torch

import nvfp4_bit_block_amd as nv
import workloads as wl
from tests.gpu_common import assert_close, dev, dev_bf16, host_bf16_f32
from tests.test_gpu_products import _moe_case

pytestmark = pytest.mark.gpu


def _lora(E, H, I, r, seed, std=0.05, which=("13", "2")):
    lo = wl.moe_lora(E, H, I, rank=r, seed=seed, std=std)
    for p in ("13", "2"):
        if p not in which:
            lo["a" + p] = lo["b" + p] = None
    return lo


def _dev_lora(lo, scale):
    return {"scale": scale, **{n: None if v is None else dev_bf16(v) for n, v in lo.items()}}


def _run(orc, T, E, k, H, I, r, mode, seed, which=("13", "2"), scale=1.5, std=0.05):
    x, ids, wts, cw, gw = _moe_case(orc, T, E, k, H, I, seed=seed)
    lo = _lora(E, H, I, r, seed + 7, std=std, which=which)
    kw, gkw = {}, {}
    if mode == 1:
        _, h = orc.moe(x, ids, wts, *cw, mode=0, want_h=True, lora={"scale": scale, **lo})
        a13 = (orc.global_scale(x) * (1 + np.arange(E) / 16)).astype(np.float32)
        a2 = (orc.global_scale(h) * (1 + np.arange(E) / 8)).astype(np.float32)
        kw = dict(a13=a13, a2=a2)
        gkw = dict(a13_scale=dev(a13), a2_scale=dev(a2))
    ref = orc.moe(x, ids, wts, *cw, mode=mode, lora={"scale": scale, **lo}, **kw)
    y = nv.moe_grouped_gemm(dev_bf16(x), dev(ids), dev(wts), *gw, mode=mode, lora=_dev_lora(lo, scale), **gkw)
    base = nv.moe_grouped_gemm(dev_bf16(x), dev(ids), dev(wts), *gw, mode=mode, **gkw)
    torch.cuda.synchronize()
    return host_bf16_f32(y), ref, host_bf16_f32(base)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("T,E,k,H,I,r", [(64, 8, 2, 256, 128, 64), (100, 16, 4, 512, 192, 16),
                                         (3, 4, 4, 128, 64, 8), (40, 4, 2, 192, 128, 24)])
def test_moe_lora_matches_oracle(orc, mode, T, E, k, H, I, r):
    print(f"moe lora mode={mode} T={T} E={E} k={k} H={H} I={I} r={r}", flush=True)
    y, ref, base = _run(orc, T, E, k, H, I, r, mode, seed=T + E + r)
    assert_close(y, ref, f"moe lora mode={mode} T={T} r={r}")
    # the adapter is visible: the adapted layer differs from the base layer
    assert np.abs(y - base).max() > 0.05 * np.abs(ref).max()


@pytest.mark.parametrize("r", [96, 128])
def test_moe_lora_wide_ranks(orc, r):
    """Ranks that take three and four 32-column blocks of the projection."""
    y, ref, _ = _run(orc, 48, 8, 2, 256, 128, r, 0, seed=r, std=0.03)
    assert_close(y, ref, f"moe lora r={r}")


@pytest.mark.parametrize("which", [("13",), ("2",)])
def test_moe_lora_one_projection(orc, which):
    y, ref, base = _run(orc, 64, 8, 2, 256, 128, 32, 0, seed=5, which=which)
    assert_close(y, ref, f"moe lora only {which}")
    assert np.abs(y - base).max() > 0


@pytest.mark.parametrize("mode", [0, 1])
def test_moe_lora_zero_b_is_the_base_layer(orc, mode):
    """A freshly initialised adapter (B = 0) leaves the layer bit-identical."""
    T, E, k, H, I, r = 64, 8, 2, 256, 128, 64
    x, ids, wts, cw, gw = _moe_case(orc, T, E, k, H, I, seed=11)
    lo = wl.moe_lora(E, H, I, rank=r, seed=12)
    lo["b13"] = np.zeros_like(lo["b13"])
    lo["b2"] = np.zeros_like(lo["b2"])
    gkw = {}
    if mode == 1:
        gkw = dict(a13_scale=dev(np.full(E, orc.global_scale(x) * 2, np.float32)),
                   a2_scale=dev(np.full(E, 0.01, np.float32)))
    y = nv.moe_grouped_gemm(dev_bf16(x), dev(ids), dev(wts), *gw, mode=mode, lora=_dev_lora(lo, 2.0), **gkw)
    base = nv.moe_grouped_gemm(dev_bf16(x), dev(ids), dev(wts), *gw, mode=mode, **gkw)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), base.view(torch.int16))


# ------------------------------------------------------------- full size --

@pytest.fixture(scope="module")
def full_moe():
    """The layer at its full size (T 4096, 256 experts, top-8, H 6144,
    I 2048): seeded router and tokens as in the benchmark, random NVFP4
    expert bytes drawn on the device, and a rank-64 adapter."""
    from tests.gpu_common import device
    T, E, k, H, I = wl.MOE_T, wl.MOE_E, wl.MOE_TOPK, wl.MOE_H, wl.MOE_I
    ids, wts = wl.moe_routing(T, E, k, seed=5)
    x = wl.moe_tokens(T, H, seed=55)
    w13 = wl.random_nvfp4((E,), 2 * I, H, seed=60, device=device())
    w2 = wl.random_nvfp4((E,), H, I, seed=61, device=device())
    lo = wl.moe_lora(E, H, I, rank=64, seed=56)
    return dict(T=T, E=E, k=k, H=H, I=I, ids=ids, wts=wts, x=x, w13=w13, w2=w2, lora=lo)


@pytest.mark.parametrize("mode,adapter,shared", [(0, False, True), (1, False, True), (1, False, False),
                                                 (0, True, True), (1, True, True)])
def test_moe_full_size_sampled_tokens(orc, full_moe, mode, adapter, shared):
    """The GPU runs the whole layer in the benchmark's launch configuration;
    the oracle recomputes 6 sampled tokens (the first, the last and 4 drawn)
    from the experts they use (a token's output depends only on its own
    routing and the expert weights).  W4A4 runs with one gate/up input scale
    for all experts (tokens quantized once each) and with one per expert
    (one quantized row per slot)."""
    f = full_moe
    T, E, H, I = f["T"], f["E"], f["H"], f["I"]
    print(f"moe full size mode={mode} lora={adapter} shared_a13={shared}", flush=True)
    a13 = np.full(E, orc.global_scale(f["x"]) * 1.5, np.float32)
    if not shared:
        a13 = (a13 * (1 + np.arange(E) / 512)).astype(np.float32)
    a2 = np.full(E, 0.02, np.float32)
    scale = 1.0
    gkw = dict(a13_scale=dev(a13), a2_scale=dev(a2)) if mode == 1 else {}
    glora = _dev_lora(f["lora"], scale) if adapter else None
    y = nv.moe_grouped_gemm(dev_bf16(f["x"]), dev(f["ids"]), dev(f["wts"]), *f["w13"], *f["w2"], mode=mode,
                            lora=glora, **gkw)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(mode + 2 * adapter).choice(T, 4)]))
    used, remap = np.unique(f["ids"][rows], return_inverse=True)
    ids_s = remap.reshape(len(rows), -1).astype(np.int32)
    ut = torch.from_numpy(used).to(y.device)
    host = [t.index_select(0, ut).cpu().numpy() for t in (*f["w13"], *f["w2"])]
    lora = None
    if adapter:
        lo = f["lora"]
        lora = {"scale": scale, "a13": lo["a13"], "b13": lo["b13"][used], "a2": lo["a2"], "b2": lo["b2"][used]}
    kw = dict(a13=a13[used], a2=a2[used]) if mode == 1 else {}
    ref = orc.moe(f["x"][rows], ids_s, f["wts"][rows], *host, mode=mode, lora=lora, **kw)
    assert_close(host_bf16_f32(y)[rows], ref, f"moe full size mode={mode} lora={adapter} shared_a13={shared}")


@pytest.mark.parametrize("mode", [0, 1])
def test_moe_lora_zero_weight_scale(orc, mode):
    """Experts whose weight global scale is 0: the weight product vanishes and
    the grouped GEMM runs no K step at all for their tiles (the adapter term
    alone, scaled by lora_scale, reaches the epilogue)."""
    T, E, k, H, I, r, scale = 64, 8, 2, 256, 128, 32, 1.5
    print(f"moe lora zero weight scale mode={mode}", flush=True)
    x, ids, wts, cw, gw = _moe_case(orc, T, E, k, H, I, seed=21)
    zero = [1, 5]
    for i in (2, 5):
        cw[i] = cw[i].copy()
        cw[i][zero] = 0.0
        gw[i] = gw[i].clone()
        gw[i][zero] = 0.0
    lo = _lora(E, H, I, r, 22)
    kw, gkw = {}, {}
    if mode == 1:
        _, h = orc.moe(x, ids, wts, *cw, mode=0, want_h=True, lora={"scale": scale, **lo})
        a13 = np.full(E, orc.global_scale(x), np.float32)
        a2 = np.full(E, orc.global_scale(h), np.float32)
        kw = dict(a13=a13, a2=a2)
        gkw = dict(a13_scale=dev(a13), a2_scale=dev(a2))
    ref = orc.moe(x, ids, wts, *cw, mode=mode, lora={"scale": scale, **lo}, **kw)
    y = nv.moe_grouped_gemm(dev_bf16(x), dev(ids), dev(wts), *gw, mode=mode, lora=_dev_lora(lo, scale), **gkw)
    torch.cuda.synchronize()
    y = host_bf16_f32(y)
    assert_close(y, ref, f"moe lora zero weight scale mode={mode}")
    # tokens routed to a zeroed expert still get that expert's adapter output
    assert np.isin(ids, zero).any() and np.abs(ref).max() > 0
