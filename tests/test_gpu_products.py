"""GPU parity of the GEMV (W4A16), the W4A4 GEMM and the MoE layer against the
oracle, elementwise |y - ref| <= 1e-3 + 1e-2 |ref|.  Both sides quantize the
weights themselves (asserted bit-identical) and use their own copy."""
import functools

import numpy as np
import pytest
import torch

import nvfp4_bit_block_amd as nv
import workloads as wl
from tests.gpu_common import assert_close, dev, dev_bf16, device, host_bf16_f32, host_u8

pytestmark = pytest.mark.gpu


def _quant_both(orc, wb):
    c0, s0, g0 = orc.quantize(wb)
    c, s, g = nv.quantize(dev_bf16(wb))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_u8(c), c0)
    np.testing.assert_array_equal(host_u8(s), s0)
    assert np.float32(g.cpu().item()) == g0
    return (c0, s0, g0), (c, s, g)


@functools.lru_cache(maxsize=None)
def _layer(name):
    import oracle
    w, x = wl.gemv_inputs(name)
    cpu, gpu = _quant_both(oracle, w)
    return w, x, cpu, gpu


# -------------------------------------------------------------------- GEMV --

@pytest.mark.parametrize("M", [1, 2, 3, 4, 8])
def test_gemv_tiny(orc, M):
    w, x = wl.tiny_end_to_end()
    x = np.concatenate([x, wl.activations(4, 512, seed=77)])[:M]
    (c0, s0, g0), (c, s, g) = _quant_both(orc, w)
    y = nv.gemv_w4a16(dev_bf16(x), c, s, g)
    torch.cuda.synchronize()
    assert_close(host_bf16_f32(y), orc.gemv_w4a16(x, c0, s0, g0), f"gemv M={M}")


@pytest.mark.parametrize("N,K", [(200, 2080), (1, 32), (67, 4096), (37, 16384), (5, 2048)])
def test_gemv_ragged(orc, N, K):
    w = wl.layer_weight((N, K), seed=N)
    x = wl.activations(2, K, seed=K)
    (c0, s0, g0), (c, s, g) = _quant_both(orc, w)
    y = nv.gemv_w4a16(dev_bf16(x), c, s, g)
    torch.cuda.synchronize()
    assert_close(host_bf16_f32(y), orc.gemv_w4a16(x, c0, s0, g0), f"gemv {N}x{K}")


@pytest.mark.parametrize("name", ["o_proj", "q_b_proj"])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_gemv_layers_full(orc, name, M):
    # every output of the full-size layer (the oracle takes well under a second)
    w, x, (c0, s0, g0), (c, s, g) = _layer(name)
    xm = x[:M]
    y = host_bf16_f32(nv.gemv_w4a16(dev_bf16(xm), c, s, g))
    assert_close(y, orc.gemv_w4a16(xm, c0, s0, g0), f"gemv {name} M={M}")


@pytest.mark.parametrize("K", [4096, 8192, 32768])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_gemv_fixed_layouts(orc, K, M):
    # the register-resident chunk layouts for K = 2048 times 2, 4 and 16 (the
    # benchmark layers use 1 and 8): W4A16 at every batch size, the batch-1
    # W4A4 that quantizes its activation in registers, and the W4A4 on a
    # pre-packed activation decoded in registers (bit-identical to the
    # one-call product on the same quantized activation)
    N = 1000
    w = wl.layer_weight((N, K), seed=K + M)
    x = wl.activations(M, K, seed=K + 2 * M)
    (c0, s0, g0), (c, s, g) = _quant_both(orc, w)
    y = host_bf16_f32(nv.gemv_w4a16(dev_bf16(x), c, s, g))
    assert_close(y, orc.gemv_w4a16(x, c0, s0, g0), f"gemv K={K} M={M}")
    isc = np.float32(orc.global_scale(x))
    y4 = host_bf16_f32(nv.gemm_w4a4(dev_bf16(x), torch.tensor([isc], device=device()), c, s, g))
    assert_close(y4, orc.gemm_w4a4(x, isc, c0, s0, g0), f"w4a4 K={K} M={M}")
    ac, asc, ag = nv.quantize(dev_bf16(x), static_scale=float(isc))
    yp = host_bf16_f32(nv.gemm_w4a4_packed(ac, asc, ag, c, s, g))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(yp.view(np.uint32), y4.view(np.uint32), err_msg=f"packed K={K} M={M}")


# -------------------------------------------------------------------- GEMM --

def _gemm_case(orc, M, N, K, seed):
    w = wl.layer_weight((N, K), seed=seed)
    x = wl.activations(M, K, seed=seed + 1)
    (c0, s0, g0), (c, s, g) = _quant_both(orc, w)
    isc = np.float32(orc.global_scale(x))
    y = nv.gemm_w4a4(dev_bf16(x), torch.tensor([isc], device=device()), c, s, g)
    torch.cuda.synchronize()
    assert_close(host_bf16_f32(y), orc.gemm_w4a4(x, isc, c0, s0, g0), f"gemm {M}x{N}x{K}")


def test_gemm_tiny_end_to_end(orc):
    w, x = wl.tiny_end_to_end()
    (c0, s0, g0), (c, s, g) = _quant_both(orc, w)
    isc = np.float32(orc.global_scale(x))          # amax(X) / (6 * 448)
    y = nv.gemm_w4a4(dev_bf16(x), torch.tensor([isc], device=device()), c, s, g)
    torch.cuda.synchronize()
    assert_close(host_bf16_f32(y), orc.gemm_w4a4(x, isc, c0, s0, g0), "gemm tiny")


# (9, 201, 2048) and (13, 75, 4096) split K four and eight ways with M N odd,
# which takes the split-K reduce's one-output-per-thread path; (9, 256,
# 131072) gives each workgroup 128 K steps, more than the small-M tiles'
# scale preload holds (64), so they load the scales per step; (9, 200, 320)
# has 5 K steps, an odd count for the small-M tiles' two-step stages
@pytest.mark.parametrize("M,N,K", [(1, 128, 1024), (8, 256, 512), (9, 200, 256), (37, 200, 256),
                                   (64, 384, 1024), (130, 384, 512), (256, 256, 2048), (300, 136, 640),
                                   (9, 201, 2048), (13, 75, 4096), (9, 256, 131072), (9, 200, 320)])
def test_gemm_shapes(orc, M, N, K):
    _gemm_case(orc, M, N, K, seed=M * 7 + N)


# long rows above M = 128 take the 256 x 256 tile with K split 256 / tiles
# ways: (300, 3072, 8192) 24 tiles, split 10 (the last split 11 of 128 K
# steps); (300, 6144, 4352) 48 tiles, split 5 over 68 steps; (600, 3072,
# 8192) 36 tiles, split 7; (600, 6144, 8192) 72 tiles, split 3
@pytest.mark.parametrize("M,N,K", [(300, 3072, 8192), (300, 6144, 4352), (600, 3072, 8192), (600, 6144, 8192)])
def test_gemm_long_row_splits(orc, M, N, K):
    w = wl.layer_weight((N, K), seed=M + N % 89)
    x = wl.activations(M, K, seed=M * 5 + K)
    (c0, s0, g0), (c, s, g) = _quant_both(orc, w)
    isc = np.float32(orc.global_scale(x))
    y = host_bf16_f32(nv.gemm_w4a4(dev_bf16(x), torch.tensor([isc], device=device()), c, s, g))
    y16 = host_bf16_f32(nv.gemm_w4a16(dev_bf16(x), c, s, g))
    rng = np.random.default_rng(M + N)
    rows = np.sort(np.concatenate([rng.choice(M, 40, replace=False), [0, M - 1]]))
    rows = np.unique(rows)
    cols = np.unique(np.sort(np.concatenate([rng.choice(N, 80, replace=False), [0, N - 1]])))
    assert_close(y[np.ix_(rows, cols)], orc.gemm_w4a4(x[rows], isc, c0[cols], s0[cols], g0),
                 f"gemm {M}x{N}x{K}")
    assert_close(y16[np.ix_(rows, cols)], orc.gemv_w4a16(x[rows], c0[cols], s0[cols], g0),
                 f"gemm w4a16 {M}x{N}x{K}")


# Long rows on the 256 x 256 tile take stream-K where the one-per-CU split
# leaves most CUs idle, and with 256-511 tiles: 256 workgroups share the
# tiles' K steps evenly, so a tile's K range is cut at arbitrary steps into
# parts summed afterwards, and a tile held whole by one workgroup is written
# by the GEMM.  (1400, 6001, 4160): 144 tiles of 65 K steps, 36.6 steps per
# workgroup, N odd (the finish's one-column-per-thread path), ragged row and
# column tiles; (1536, 5888, 4352): 138 tiles; (1700, 5000, 16384): 140
# tiles of 256 steps; (1024, 5632, 8192): 88 tiles otherwise split 2, up to
# 4 parts per tile; (3000, 6000, 8320): 288 tiles of 130 steps, 146.25 per
# workgroup, so some tiles whole and the rest in two parts.  Every 256 x 256
# tile is sampled.
@pytest.mark.parametrize("M,N,K", [(1400, 6001, 4160), (1536, 5888, 4352), (1700, 5000, 16384), (1024, 5632, 8192),
                                   (3000, 6000, 8320)])
def test_gemm_stream_k(orc, M, N, K):
    w = wl.layer_weight((N, K), seed=M + 3 * N)
    x = wl.activations(M, K, seed=M * 7 + K)
    (c0, s0, g0), (c, s, g) = _quant_both(orc, w)
    isc = np.float32(orc.global_scale(x))
    y = host_bf16_f32(nv.gemm_w4a4(dev_bf16(x), torch.tensor([isc], device=device()), c, s, g))
    y16 = host_bf16_f32(nv.gemm_w4a16(dev_bf16(x), c, s, g))
    # the pre-packed entry runs the same tiles on the same quantized operand
    ac, asc, ag = nv.quantize(dev_bf16(x), static_scale=float(isc))
    yp = host_bf16_f32(nv.gemm_w4a4_packed(ac, asc, ag, c, s, g))
    np.testing.assert_array_equal(yp.view(np.uint32), y.view(np.uint32), err_msg="stream-K packed vs one-call")
    rng = np.random.default_rng(M + N + K)
    rows = np.unique(np.concatenate([np.minimum(M - 1, r0 + rng.choice(256, 6, replace=False))
                                     for r0 in range(0, M, 256)] + [[0, M - 1]]))
    cols = np.unique(np.concatenate([np.minimum(N - 1, c0_ + rng.choice(256, 4, replace=False))
                                     for c0_ in range(0, N, 256)] + [[0, N - 1]]))
    assert_close(y[np.ix_(rows, cols)], orc.gemm_w4a4(x[rows], isc, c0[cols], s0[cols], g0),
                 f"gemm stream-K {M}x{N}x{K}")
    assert_close(y16[np.ix_(rows, cols)], orc.gemv_w4a16(x[rows], c0[cols], s0[cols], g0),
                 f"gemm w4a16 stream-K {M}x{N}x{K}")


@pytest.mark.parametrize("name", ["o_proj", "q_b_proj"])
@pytest.mark.parametrize("M", list(wl.GEMM_M_SWEEP))
def test_gemm_layers_sampled(orc, name, M):
    w, _, (c0, s0, g0), (c, s, g) = _layer(name)
    x = wl.activations(M, w.shape[1], seed=4)
    isc = np.float32(orc.global_scale(x))
    y = host_bf16_f32(nv.gemm_w4a4(dev_bf16(x), torch.tensor([isc], device=device()), c, s, g))
    rng = np.random.default_rng(M)
    rows = np.sort(rng.choice(M, min(M, 48), replace=False))
    cols = np.sort(rng.choice(w.shape[0], 96, replace=False))
    ref = orc.gemm_w4a4(x[rows], isc, c0[cols], s0[cols], g0)
    assert_close(y[np.ix_(rows, cols)], ref, f"gemm {name} M={M}")


# ------------------------------------------- W4A4 on a pre-packed activation --

def _packed_matches(orc, x, isc, c, s, g, what):
    y = host_bf16_f32(nv.gemm_w4a4(dev_bf16(x), torch.tensor([isc], device=device()), c, s, g))
    ac, asc, ag = nv.quantize(dev_bf16(x), static_scale=float(isc))
    yp = host_bf16_f32(nv.gemm_w4a4_packed(ac, asc, ag, c, s, g))
    np.testing.assert_array_equal(yp.view(np.uint32), y.view(np.uint32), err_msg=what)
    return yp


@pytest.mark.parametrize("M,N,K", [(1, 128, 1024), (3, 200, 2048), (5, 67, 16384), (9, 200, 256), (37, 200, 256),
                                   (130, 384, 512), (300, 136, 640), (13, 75, 4096)])
def test_gemm_packed_shapes(orc, M, N, K):
    # quantize once (static), then the GEMM on codes and scales: the same bits
    # as the one-call W4A4 GEMM, and within tolerance of the oracle
    w = wl.layer_weight((N, K), seed=M * 3 + N)
    x = wl.activations(M, K, seed=M + 2 * K)
    (c0, s0, g0), (c, s, g) = _quant_both(orc, w)
    isc = np.float32(orc.global_scale(x))
    yp = _packed_matches(orc, x, isc, c, s, g, f"packed {M}x{N}x{K}")
    assert_close(yp, orc.gemm_w4a4(x, isc, c0, s0, g0), f"packed {M}x{N}x{K}")


@pytest.mark.parametrize("name", ["o_proj", "q_b_proj"])
@pytest.mark.parametrize("M", [1, 8, 128, 1024])
def test_gemm_packed_layers(orc, name, M):
    w, _, _, (c, s, g) = _layer(name)
    x = wl.activations(M, w.shape[1], seed=4)
    _packed_matches(orc, x, np.float32(orc.global_scale(x)), c, s, g, f"packed {name} M={M}")


# ------------------------------------------------------- W4A16 over any M --

@pytest.mark.parametrize("M,N,K", [(1, 128, 1024), (6, 200, 8192), (9, 200, 256), (37, 200, 256),
                                   (64, 384, 1024), (130, 384, 512), (256, 256, 2048), (300, 136, 640),
                                   (9, 201, 2048)])
def test_gemm_w4a16_shapes(orc, M, N, K):
    w = wl.layer_weight((N, K), seed=M * 5 + N)
    x = wl.activations(M, K, seed=M + K)
    (c0, s0, g0), (c, s, g) = _quant_both(orc, w)
    y = nv.gemm_w4a16(dev_bf16(x), c, s, g)
    torch.cuda.synchronize()
    assert_close(host_bf16_f32(y), orc.gemv_w4a16(x, c0, s0, g0), f"gemm_w4a16 {M}x{N}x{K}")


@pytest.mark.parametrize("name", ["o_proj", "q_b_proj"])
@pytest.mark.parametrize("M", list(wl.GEMM_M_SWEEP))
def test_gemm_w4a16_layers_sampled(orc, name, M):
    w, _, (c0, s0, g0), (c, s, g) = _layer(name)
    x = wl.activations(M, w.shape[1], seed=4)
    y = host_bf16_f32(nv.gemm_w4a16(dev_bf16(x), c, s, g))
    rng = np.random.default_rng(M + 1)
    rows = np.sort(rng.choice(M, min(M, 48), replace=False))
    cols = np.sort(rng.choice(w.shape[0], 96, replace=False))
    ref = orc.gemv_w4a16(x[rows], c0[cols], s0[cols], g0)
    assert_close(y[np.ix_(rows, cols)], ref, f"gemm_w4a16 {name} M={M}")


def test_gemm_w4a16_small_m_equals_gemv(orc):
    # at M <= 8 the GEMM entry point runs the GEMV kernels: same bits
    w, _, _, (c, s, g) = _layer("o_proj")
    x = wl.activations(4, w.shape[1], seed=8)
    a = host_bf16_f32(nv.gemm_w4a16(dev_bf16(x), c, s, g))
    b = host_bf16_f32(nv.gemv_w4a16(dev_bf16(x), c, s, g))
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


def _two_step_small_m(orc, x, isc, c, s, g):
    """The small-M W4A4 product written as two library calls: static quantize,
    then the W4A16 GEMV over the exact products q * s (bf16) under the
    combined global scale fl(w_global * input_scale)."""
    xc, xs, _ = nv.quantize(dev_bf16(x), static_scale=float(isc))
    torch.cuda.synchronize()
    _, qs = orc.dequantize(host_u8(xc), host_u8(xs), 1.0, want_bf16=True)
    gcomb = torch.tensor([np.float32(g.cpu().item()) * np.float32(isc)], device=device())
    y = nv.gemv_w4a16(dev_bf16(qs), c, s, gcomb)
    torch.cuda.synchronize()
    return host_bf16_f32(y)


@pytest.mark.parametrize("name,M", [("o_proj", 1), ("o_proj", 3), ("q_b_proj", 1), ("q_b_proj", 2)])
def test_gemm_small_m_equals_two_step(orc, name, M):
    # At M = 1 on these shapes the GEMM quantizes the activation inside the
    # GEMV; the other GEMV batch sizes (below the stream kernel's range: up to
    # 4 on o_proj, 2 on q_b_proj) run the quantize and the GEMV; either way the
    # result must be bit-identical to quantizing first.
    w, _, _, (c, s, g) = _layer(name)
    x = wl.activations(M, w.shape[1], seed=90 + M)
    isc = np.float32(orc.global_scale(x))
    y = host_bf16_f32(nv.gemm_w4a4(dev_bf16(x), torch.tensor([isc], device=device()), c, s, g))
    np.testing.assert_array_equal(y.view(np.uint32), _two_step_small_m(orc, x, isc, c, s, g).view(np.uint32))


@pytest.mark.parametrize("f", [0.02, 1.0, 64.0])
@pytest.mark.parametrize("K", [2048, 16384])
def test_gemm_batch1_edge_blocks(orc, f, K):
    # single rows with zero blocks, outlier blocks, tiny values and an input
    # scale far too small (saturated block scales) or too large (subnormal
    # block scales) for the activation
    N = 96
    w = wl.layer_weight((N, K), seed=12)
    x = wl.bf16_bits_to_f32(wl.activations(4, K, seed=13)).copy()
    x[0, :64] = 0.0
    x[1, 32:48] *= 3000.0
    x[2, ::17] = -1e-30
    x[3] *= 1e-6
    x = wl.to_bf16_bits(x)
    (c0, s0, g0), (c, s, g) = _quant_both(orc, w)
    for r in range(4):
        xr = x[r:r + 1]
        isc = np.float32(orc.global_scale(xr) * f)
        y = host_bf16_f32(nv.gemm_w4a4(dev_bf16(xr), torch.tensor([isc], device=device()), c, s, g))
        np.testing.assert_array_equal(y.view(np.uint32),
                                      _two_step_small_m(orc, xr, isc, c, s, g).view(np.uint32))
        assert_close(y, orc.gemm_w4a4(xr, isc, c0, s0, g0), f"gemm row {r} K={K} x{f}")


def test_gemm_generous_and_tight_input_scale(orc):
    w = wl.layer_weight((256, 1024), seed=5)
    x = wl.activations(160, 1024, seed=6)
    (c0, s0, g0), (c, s, g) = _quant_both(orc, w)
    for f in (4.0, 0.5):
        isc = np.float32(orc.global_scale(x) * f)
        y = nv.gemm_w4a4(dev_bf16(x), torch.tensor([isc], device=device()), c, s, g)
        torch.cuda.synchronize()
        assert_close(host_bf16_f32(y), orc.gemm_w4a4(x, isc, c0, s0, g0), f"gemm scale x{f}")


# --------------------------------------------------------------------- MoE --

def _moe_case(orc, T, E, k, H, I, seed):
    x = wl.activations(T, H, seed=seed)
    ids, wts = wl.moe_routing(T, E, k, seed=seed + 1)
    rng = np.random.default_rng(seed + 2)
    cpu13, cpu2, gpu13, gpu2 = [], [], [], []
    for e in range(E):
        a, b = _quant_both(orc, wl.normal_bf16(rng, (2 * I, H), 0.02))
        cpu13.append(a); gpu13.append(b)
        a, b = _quant_both(orc, wl.normal_bf16(rng, (H, I), 0.02))
        cpu2.append(a); gpu2.append(b)
    cw = [np.stack([q[i] for q in cpu13]) for i in range(2)] + [np.array([q[2] for q in cpu13], np.float32)]
    cw += [np.stack([q[i] for q in cpu2]) for i in range(2)] + [np.array([q[2] for q in cpu2], np.float32)]
    gw = [torch.stack([q[i] for q in gpu13]) for i in range(2)] + [torch.cat([q[2] for q in gpu13])]
    gw += [torch.stack([q[i] for q in gpu2]) for i in range(2)] + [torch.cat([q[2] for q in gpu2])]
    return x, ids, wts, cw, gw


@pytest.mark.parametrize("T,E,k,H,I", [(64, 8, 2, 256, 128), (100, 16, 4, 512, 192), (3, 4, 4, 128, 64)])
def test_moe_w4a16(orc, T, E, k, H, I):
    x, ids, wts, cw, gw = _moe_case(orc, T, E, k, H, I, seed=T + E)
    ref = orc.moe(x, ids, wts, *cw, mode=0)
    y = nv.moe_grouped_gemm(dev_bf16(x), dev(ids), dev(wts), *gw, mode=nv.MODE_W4A16)
    torch.cuda.synchronize()
    assert_close(host_bf16_f32(y), ref, f"moe w4a16 T={T}")


@pytest.mark.parametrize("T,E,k,H,I", [(64, 8, 2, 256, 128), (100, 16, 4, 512, 192)])
def test_moe_w4a4(orc, T, E, k, H, I):
    x, ids, wts, cw, gw = _moe_case(orc, T, E, k, H, I, seed=T + E + 1)
    _, h = orc.moe(x, ids, wts, *cw, mode=0, want_h=True)
    a13 = (orc.global_scale(x) * (1 + np.arange(E) / 16)).astype(np.float32)
    a2 = (orc.global_scale(h) * (1 + np.arange(E) / 8)).astype(np.float32)
    ref = orc.moe(x, ids, wts, *cw, mode=1, a13=a13, a2=a2)
    y = nv.moe_grouped_gemm(dev_bf16(x), dev(ids), dev(wts), *gw, mode=nv.MODE_W4A4,
                            a13_scale=dev(a13), a2_scale=dev(a2))
    torch.cuda.synchronize()
    assert_close(host_bf16_f32(y), ref, f"moe w4a4 T={T}")


def _skewed_routing(counts, k, seed):
    """Top-k ids with exact per-expert slot counts: the experts' slots laid
    out in expert order and dealt column by column (token t takes slots t,
    t + T, ...), which keeps a token's k experts distinct for these counts."""
    L = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    T = len(L) // k
    ids = np.ascontiguousarray(L.reshape(k, T).T)
    assert all(len(set(r)) == k for r in ids.tolist())
    w = np.random.default_rng(seed).random((T, k)).astype(np.float32) + 0.1
    return ids, (w / w.sum(1, keepdims=True)).astype(np.float32)


@pytest.mark.parametrize("mode", [0, 1])
def test_moe_rows_beyond_full_tiles(orc, mode):
    """Experts around the grouped GEMMs' 192-row tiles (four 96 x 64 waves; a
    tile of at most 128 rows splits them 64 / 64): 150, 160, 161 and 129 rows
    (one tile, the second wave row partly filled), 192 (one full tile), 193
    and 261 (a second tile of 1 and 69 rows), 128 (the largest 64 / 64
    split), 95, 64 and 39 rows (second wave row partly filled or empty)."""
    counts = [150, 160, 161, 129, 261, 39, 192, 193, 128, 64, 95]
    k, H, I = 3, 256, 128
    ids, wts = _skewed_routing(counts, k, seed=9)
    assert np.array_equal(np.bincount(ids.ravel(), minlength=len(counts)), counts)
    T, E = ids.shape[0], len(counts)
    x, _, _, cw, gw = _moe_case(orc, 1, E, 1, H, I, seed=31)
    x = wl.activations(T, H, seed=32)
    if mode == 0:
        ref = orc.moe(x, ids, wts, *cw, mode=0)
        y = nv.moe_grouped_gemm(dev_bf16(x), dev(ids), dev(wts), *gw, mode=nv.MODE_W4A16)
    else:
        _, h = orc.moe(x, ids, wts, *cw, mode=0, want_h=True)
        a13 = np.full(E, orc.global_scale(x), np.float32)
        a2 = np.full(E, orc.global_scale(h), np.float32)
        ref = orc.moe(x, ids, wts, *cw, mode=1, a13=a13, a2=a2)
        y = nv.moe_grouped_gemm(dev_bf16(x), dev(ids), dev(wts), *gw, mode=nv.MODE_W4A4,
                                a13_scale=dev(a13), a2_scale=dev(a2))
    torch.cuda.synchronize()
    assert_close(host_bf16_f32(y), ref, f"moe skewed routing mode {mode}")


def test_moe_w4a4_shared_input_scale(orc):
    """W4A4 with one a13 value for every expert quantizes each token once and
    gathers it by slot; with one value differing on an expert that receives
    no slot the layer quantizes per slot instead.  Both must give the same
    bits, and the oracle's result."""
    counts = [40, 90, 130, 0, 70, 150, 11, 109]
    k, H, I = 4, 256, 128
    ids, wts = _skewed_routing(counts, k, seed=21)
    T, E = ids.shape[0], len(counts)
    x, _, _, cw, gw = _moe_case(orc, 1, E, 1, H, I, seed=41)
    x = wl.activations(T, H, seed=42)
    _, h = orc.moe(x, ids, wts, *cw, mode=0, want_h=True)
    a13 = np.full(E, orc.global_scale(x), np.float32)
    a2 = np.full(E, orc.global_scale(h), np.float32)
    ref = orc.moe(x, ids, wts, *cw, mode=1, a13=a13, a2=a2)
    odd = a13.copy()
    odd[3] *= 2.0
    ys = [nv.moe_grouped_gemm(dev_bf16(x), dev(ids), dev(wts), *gw, mode=nv.MODE_W4A4,
                              a13_scale=dev(sc), a2_scale=dev(a2)) for sc in (a13, odd, a13)]
    torch.cuda.synchronize()
    assert_close(host_bf16_f32(ys[0]), ref, "moe w4a4 shared a13")
    assert torch.equal(ys[0].view(torch.int16), ys[1].view(torch.int16))
    assert torch.equal(ys[0].view(torch.int16), ys[2].view(torch.int16))


def test_moe_many_experts_many_runs(orc):
    """Routing over several workgroup runs of slots (2400 slots) and more
    experts than the scan has threads (1100), most experts with a few rows."""
    T, E, k, H, I = 600, 1100, 4, 64, 64
    x, ids, wts, cw, gw = _moe_case(orc, T, E, k, H, I, seed=77)
    ref = orc.moe(x, ids, wts, *cw, mode=0)
    y = nv.moe_grouped_gemm(dev_bf16(x), dev(ids), dev(wts), *gw, mode=nv.MODE_W4A16)
    torch.cuda.synchronize()
    assert_close(host_bf16_f32(y), ref, "moe many experts")


def _random_gemm_shapes(n=12, seed=2027):
    """Seeded (M, N, K) draws spread over the planner's regimes: batch rows
    1-64 (GEMV, weight streaming), 65-256 (stream kernel or tiles with K
    splits) and 257-3000 (256 x 256 tiles, split or stream-K), K a multiple
    of 64 from 64 to 12288, N from 16 to 6200 (odd counts included)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        band = i % 3
        M = int(rng.integers(1, 65) if band == 0 else rng.integers(65, 257) if band == 1 else rng.integers(257, 3001))
        K = 64 * int(rng.integers(1, 193))
        N = int(rng.integers(16, 6201))
        while N * K > 40_000_000:         # keep the oracle's weight quantize to a few seconds
            N //= 2
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", _random_gemm_shapes())
def test_gemm_random_shapes(orc, M, N, K):
    print(f"random gemm M={M} N={N} K={K}", flush=True)
    w = wl.layer_weight((N, K), seed=M + N + K)
    x = wl.activations(M, K, seed=3 * M + K)
    (c0, s0, g0), (c, s, g) = _quant_both(orc, w)
    isc = np.float32(orc.global_scale(x))
    y = host_bf16_f32(nv.gemm_w4a4(dev_bf16(x), torch.tensor([isc], device=device()), c, s, g))
    y16 = host_bf16_f32(nv.gemm_w4a16(dev_bf16(x), c, s, g))
    ac, asc, ag = nv.quantize(dev_bf16(x), static_scale=float(isc))
    yp = host_bf16_f32(nv.gemm_w4a4_packed(ac, asc, ag, c, s, g))
    np.testing.assert_array_equal(yp.view(np.uint32), y.view(np.uint32), err_msg="packed vs one-call")
    rng = np.random.default_rng(M * N + K)
    rows = np.unique(np.concatenate([rng.choice(M, min(M, 24), replace=False), [0, M - 1]]))
    cols = np.unique(np.concatenate([rng.choice(N, min(N, 64), replace=False), [0, N - 1]]))
    assert_close(y[np.ix_(rows, cols)], orc.gemm_w4a4(x[rows], isc, c0[cols], s0[cols], g0),
                 f"random gemm {M}x{N}x{K}")
    assert_close(y16[np.ix_(rows, cols)], orc.gemv_w4a16(x[rows], c0[cols], s0[cols], g0),
                 f"random gemm w4a16 {M}x{N}x{K}")


def _random_moe_shapes(n=6, seed=909):
    """Seeded (T, E, k, H, I) draws: 1-400 tokens, 2-40 experts, top-1..8,
    H and I multiples of 64 up to 512 and 320, so that experts hold from no
    rows to a few hundred (one or two 192-row tiles, the 64 / 64 split)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        E = int(rng.integers(2, 41))
        k = int(rng.integers(1, min(8, E) + 1))
        out.append((int(rng.integers(1, 401)), E, k, 64 * int(rng.integers(1, 9)), 64 * int(rng.integers(1, 6))))
    return out


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("T,E,k,H,I", _random_moe_shapes())
def test_moe_random_shapes(orc, T, E, k, H, I, mode):
    print(f"random moe T={T} E={E} k={k} H={H} I={I} mode={mode}", flush=True)
    x, ids, wts, cw, gw = _moe_case(orc, T, E, k, H, I, seed=T * 7 + E * 3 + k)
    if mode == 0:
        ref = orc.moe(x, ids, wts, *cw, mode=0)
        y = nv.moe_grouped_gemm(dev_bf16(x), dev(ids), dev(wts), *gw, mode=nv.MODE_W4A16)
    else:
        _, h = orc.moe(x, ids, wts, *cw, mode=0, want_h=True)
        a13 = (orc.global_scale(x) * (1 + np.arange(E) / 32)).astype(np.float32)
        a2 = (orc.global_scale(h) * (1 + np.arange(E) / 16)).astype(np.float32)
        ref = orc.moe(x, ids, wts, *cw, mode=1, a13=a13, a2=a2)
        y = nv.moe_grouped_gemm(dev_bf16(x), dev(ids), dev(wts), *gw, mode=nv.MODE_W4A4,
                                a13_scale=dev(a13), a2_scale=dev(a2))
    torch.cuda.synchronize()
    assert_close(host_bf16_f32(y), ref, f"random moe T={T} E={E} k={k} H={H} I={I} mode={mode}")
