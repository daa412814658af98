"""Pins of the oracle's GEMV / GEMM / MoE references.

Operands built from grid values x E4M3 values x a power-of-two global scale
quantize losslessly, so the oracle's products must equal a textbook numpy
fp64 matmul of the original tensors; non-square shapes catch a transposed
operand.  MoE reduces to a dense MLP for one expert, for identical experts,
and is invariant to the order of a token's slots.
"""
import numpy as np
import pytest
import torch

import workloads as wl

GRID = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])


def _e4m3_values():
    return torch.arange(0, 127, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def lossless_tensor(rng, rows, cols, sg_exp=-12, smin=48):
    """bf16 [rows, cols] whose NVFP4 quantization is exact: every element is
    q * s_block * 2^sg_exp with a +-6 in each block and the tensor amax block at
    scale 448 (so the dynamic Sg is exactly 2^sg_exp)."""
    e4 = _e4m3_values()
    q = GRID[rng.integers(0, 8, (rows, cols))] * rng.choice([-1.0, 1.0], (rows, cols))
    q[:, 5::16] = 6.0 * rng.choice([-1.0, 1.0], (rows, cols // 16))
    sb = e4[rng.integers(smin, 126, (rows, cols // 16))]
    sb[0, 0] = 448.0
    x = (q * np.repeat(sb, 16, axis=1) * 2.0 ** sg_exp).astype(np.float32)
    xb = wl.to_bf16_bits(x)
    assert (wl.bf16_bits_to_f32(xb) == x).all()
    return xb, x.astype(np.float64)


@pytest.mark.parametrize("M,N,K", [(1, 37, 64), (3, 16, 512), (8, 24, 2048)])
def test_gemv_lossless_equals_matmul(orc, M, N, K):
    rng = np.random.default_rng(M * 1000 + N)
    wb, wf = lossless_tensor(rng, N, K)
    x = wl.activations(M, K, seed=N)
    c, s, g = orc.quantize(wb)
    assert g == np.float32(2.0 ** -12)
    y = orc.gemv_w4a16(x, c, s, g)
    ref = wl.bf16_bits_to_f32(x).astype(np.float64) @ wf.T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("M,N,K", [(1, 40, 64), (5, 16, 256), (33, 48, 512)])
def test_gemm_w4a4_lossless_equals_matmul(orc, M, N, K):
    """X and W both exactly representable: the W4A4 reference is X . W^T."""
    rng = np.random.default_rng(K + M)
    wb, wf = lossless_tensor(rng, N, K, sg_exp=-10)
    xb, xf = lossless_tensor(rng, M, K, sg_exp=-3)
    c, s, g = orc.quantize(wb)
    y = orc.gemm_w4a4(xb, 2.0 ** -3, c, s, g)
    np.testing.assert_allclose(y, xf @ wf.T, rtol=1e-12, atol=1e-12)


def test_w4a4_is_w4a16_on_quantized_activation(orc):
    """W4A4(X) = W4A16(deq(quant(X, input_scale))) when the dequantized X is
    bf16-exact (power-of-two input scale)."""
    w, _ = wl.tiny_end_to_end()
    x = wl.activations(6, 512, seed=99)
    c, s, g = orc.quantize(w)
    isc = 2.0 ** -8
    xc, xs, _ = orc.quantize(x, isc)
    xd, xdb = orc.dequantize(xc, xs, isc, want_bf16=True)
    assert (wl.bf16_bits_to_f32(xdb) == xd).all()
    np.testing.assert_allclose(orc.gemm_w4a4(x, isc, c, s, g), orc.gemv_w4a16(xdb, c, s, g), rtol=1e-13, atol=1e-13)


def test_gemv_bruteforce_tiny(orc):
    """Tiny GEMV against Python loops over an independent dequantization."""
    rng = np.random.default_rng(5)
    N, K, M = 5, 32, 2
    wb = wl.normal_bf16(rng, (N, K), 0.02)
    x = wl.normal_bf16(rng, (M, K), 1.0)
    c, s, g = orc.quantize(wb)
    e4 = torch.from_numpy(s.copy()).view(torch.float8_e4m3fn).float().numpy()
    xf = wl.bf16_bits_to_f32(x)
    y = orc.gemv_w4a16(x, c, s, g)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                byte = int(c[n, k // 2])
                code = (byte >> 4) if k % 2 else (byte & 15)
                q = GRID[code & 7] * (-1.0 if code & 8 else 1.0)
                deq = np.float32(np.float32(q) * e4[n, k // 16]) * np.float32(g)
                acc += float(deq) * float(xf[m, k])
            assert abs(acc - y[m, n]) <= 1e-12 * max(1.0, abs(acc))


# --------------------------------------------------------------------- MoE --

def _silu(z):
    return z / (1.0 + np.exp(-z))


def _bf16_round(a):
    return wl.bf16_bits_to_f32(wl.to_bf16_bits(a.astype(np.float32))).astype(np.float64)


def _experts(rng, E, H, I, identical=False):
    w13b, w2b, w13f, w2f = [], [], [], []
    for e in range(E):
        if identical and e > 0:
            w13b.append(w13b[0]); w2b.append(w2b[0]); w13f.append(w13f[0]); w2f.append(w2f[0])
            continue
        a, af = lossless_tensor(rng, 2 * I, H, sg_exp=-9)
        b, bf = lossless_tensor(rng, H, I, sg_exp=-9)
        w13b.append(a); w2b.append(b); w13f.append(af); w2f.append(bf)
    return np.stack(w13b), np.stack(w2b), w13f, w2f


def _quant_experts(orc, w13b, w2b):
    q13 = [orc.quantize(w) for w in w13b]
    q2 = [orc.quantize(w) for w in w2b]
    return (np.stack([q[0] for q in q13]), np.stack([q[1] for q in q13]), np.array([q[2] for q in q13], np.float32),
            np.stack([q[0] for q in q2]), np.stack([q[1] for q in q2]), np.array([q[2] for q in q2], np.float32))


def _dense_mlp(x_f, w13f, w2f, I):
    g = x_f @ w13f[:I].T
    u = x_f @ w13f[I:].T
    h = _bf16_round(_silu(g) * u)
    return h @ w2f.T, h


def test_moe_single_expert_is_dense_mlp(orc):
    rng = np.random.default_rng(1)
    T, E, H, I = 6, 1, 64, 32
    w13b, w2b, w13f, w2f = _experts(rng, E, H, I)
    x = wl.activations(T, H, seed=2)
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    out, h = orc.moe(x, ids, w, *_quant_experts(orc, w13b, w2b), mode=0, want_h=True)
    ref, href = _dense_mlp(wl.bf16_bits_to_f32(x).astype(np.float64), w13f[0], w2f[0], I)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_array_equal(wl.bf16_bits_to_f32(h), href.astype(np.float32))


def test_moe_identical_experts_is_dense_mlp(orc):
    rng = np.random.default_rng(3)
    T, E, k, H, I = 5, 4, 3, 64, 32
    w13b, w2b, w13f, w2f = _experts(rng, E, H, I, identical=True)
    x = wl.activations(T, H, seed=4)
    ids, w = wl.moe_routing(T, E, k, seed=6)
    out = orc.moe(x, ids, w, *_quant_experts(orc, w13b, w2b), mode=0)
    ref, _ = _dense_mlp(wl.bf16_bits_to_f32(x).astype(np.float64), w13f[0], w2f[0], I)
    np.testing.assert_allclose(out, ref * w.astype(np.float64).sum(axis=1, keepdims=True), rtol=1e-10, atol=1e-12)


def test_moe_routed_matches_per_slot_dense(orc):
    """Distinct experts: out[t] = sum_j w[t,j] * MLP_{e(t,j)}(x_t)."""
    rng = np.random.default_rng(7)
    T, E, k, H, I = 7, 5, 2, 32, 16
    w13b, w2b, w13f, w2f = _experts(rng, E, H, I)
    x = wl.activations(T, H, seed=8)
    ids, w = wl.moe_routing(T, E, k, seed=9)
    out = orc.moe(x, ids, w, *_quant_experts(orc, w13b, w2b), mode=0)
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            y, _ = _dense_mlp(xf[t:t + 1], w13f[e], w2f[e], I)
            ref[t] += float(w[t, j]) * y[0]
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_moe_slot_order_invariant(orc):
    rng = np.random.default_rng(11)
    T, E, k, H, I = 6, 6, 4, 32, 16
    w13b, w2b, _, _ = _experts(rng, E, H, I)
    q = _quant_experts(orc, w13b, w2b)
    x = wl.activations(T, H, seed=12)
    ids, w = wl.moe_routing(T, E, k, seed=13)
    perm = np.random.default_rng(14).permutation(k)
    a = orc.moe(x, ids, w, *q, mode=0)
    b = orc.moe(x, ids[:, perm].copy(), w[:, perm].copy(), *q, mode=0)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_moe_w4a4_single_expert_composition(orc):
    """Mode 1 with one expert = W4A4 GEMM under a13, SiLU gating rounded to
    bf16, then W4A4 GEMM under a2."""
    rng = np.random.default_rng(15)
    T, E, H, I = 4, 1, 64, 32
    w13b, w2b, _, _ = _experts(rng, E, H, I)
    q = _quant_experts(orc, w13b, w2b)
    x = wl.activations(T, H, seed=16)
    a13 = np.array([orc.global_scale(x) * 2], np.float32)
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    # a2 from the h of the W4A16 pass, made generous
    _, h0 = orc.moe(x, ids, w, *q, mode=0, want_h=True)
    a2 = np.array([orc.global_scale(h0) * 2], np.float32)
    out, h = orc.moe(x, ids, w, *q, mode=1, a13=a13, a2=a2, want_h=True)
    gu = orc.gemm_w4a4(x, a13[0], q[0][0], q[1][0], q[2][0])
    href = _bf16_round(_silu(gu[:, :I]) * gu[:, I:])
    np.testing.assert_array_equal(wl.bf16_bits_to_f32(h).astype(np.float64), href)
    ref = orc.gemm_w4a4(h, a2[0], q[3][0], q[4][0], q[5][0])
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- MoE-LoRA --
# The bf16 adapter adds scale * B_e (A v) to each expert projection, with
# z = A v rounded to bf16.  Where z is exact in bf16 (ternary A over
# power-of-two-grid inputs, or A selecting single inputs), the adapted expert
# is the dense MLP with the merged weights W + scale * B_e A, a plain fp64
# matmul.

def _ternary_bf16(rng, shape):
    return wl.to_bf16_bits(rng.integers(-1, 2, size=shape).astype(np.float32))


def _grid_tokens(rng, T, H):
    # multiples of 1/8 in [-1/2, 1/2]: a ternary combination of 64 of them is
    # 1/8 times an integer of magnitude at most 256, exact in bf16
    assert H <= 64
    return wl.to_bf16_bits(rng.integers(-4, 5, size=(T, H)).astype(np.float32) / 8)


def _selector(rank, n, rng):
    a = np.zeros((rank, n), np.float32)
    a[np.arange(rank), rng.choice(n, rank, replace=False)] = 1.0
    return wl.to_bf16_bits(a)


def _f(b):
    return wl.bf16_bits_to_f32(b).astype(np.float64)


def test_moe_lora_merged_weights(orc):
    """Routed experts with an adapter on both projections equal per-slot dense
    MLPs with merged weights: a transposed operand, a swapped gate/up half of
    B13, a wrong expert's B or a misplaced scale all break the equality."""
    rng = np.random.default_rng(21)
    T, E, k, H, I, r = 6, 4, 2, 64, 32, 8
    w13b, w2b, w13f, w2f = _experts(rng, E, H, I)
    q = _quant_experts(orc, w13b, w2b)
    x = _grid_tokens(rng, T, H)
    ids, w = wl.moe_routing(T, E, k, seed=22)
    scale = 0.75
    lora = {"a13": _ternary_bf16(rng, (r, H)), "b13": wl.normal_bf16(rng, (E, 2 * I, r), 0.05),
            "a2": _selector(r, I, rng), "b2": wl.normal_bf16(rng, (E, H, r), 0.05), "scale": scale}
    out = orc.moe(x, ids, w, *q, mode=0, lora=lora)
    xf = _f(x)
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            m13 = w13f[e] + scale * _f(lora["b13"][e]) @ _f(lora["a13"])
            m2 = w2f[e] + scale * _f(lora["b2"][e]) @ _f(lora["a2"])
            y, _ = _dense_mlp(xf[t:t + 1], m13, m2, I)
            ref[t] += float(w[t, j]) * y[0]
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_moe_lora_rounds_the_rank_intermediate_to_bf16(orc):
    """With the base down projection zero and B2 = the identity on the first r
    outputs, the layer returns scale * bf16(A2 h): the rank-r intermediate is
    the bf16 rounding (RNE, torch's conversion) of the exact product."""
    rng = np.random.default_rng(23)
    T, E, H, I, r = 5, 1, 64, 32, 16
    w13b, _, _, _ = _experts(rng, E, H, I)
    w2b = np.zeros((E, H, I), np.uint16)
    q = _quant_experts(orc, w13b, w2b)
    x = wl.activations(T, H, seed=24)
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    b2 = np.zeros((E, H, r), np.float32)
    b2[0, np.arange(r), np.arange(r)] = 1.0
    lora = {"a13": None, "a2": wl.normal_bf16(rng, (r, I), 0.3), "b2": wl.to_bf16_bits(b2), "scale": 2.0}
    out, h = orc.moe(x, ids, w, *q, mode=0, want_h=True, lora=lora)
    exact = _f(h) @ _f(lora["a2"]).T
    z = torch.from_numpy(exact).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(out[:, :r], 2.0 * z)
    np.testing.assert_array_equal(out[:, r:], 0.0)


def test_moe_lora_zero_b_is_the_base_layer(orc):
    """An adapter whose B is all zero (its initial state) changes nothing, in
    both modes, bit for bit."""
    rng = np.random.default_rng(25)
    T, E, k, H, I, r = 5, 3, 2, 64, 32, 16
    w13b, w2b, _, _ = _experts(rng, E, H, I)
    q = _quant_experts(orc, w13b, w2b)
    x = wl.activations(T, H, seed=26)
    ids, w = wl.moe_routing(T, E, k, seed=27)
    lora = {"a13": wl.normal_bf16(rng, (r, H), 0.1), "b13": np.zeros((E, 2 * I, r), np.uint16),
            "a2": wl.normal_bf16(rng, (r, I), 0.1), "b2": np.zeros((E, H, r), np.uint16), "scale": 3.0}
    a13 = np.full(E, orc.global_scale(x) * 2, np.float32)
    a2 = np.full(E, 0.01, np.float32)
    for mode in (0, 1):
        base = orc.moe(x, ids, w, *q, mode=mode, a13=a13, a2=a2)
        got = orc.moe(x, ids, w, *q, mode=mode, a13=a13, a2=a2, lora=lora)
        np.testing.assert_array_equal(got, base)


def test_moe_lora_uses_the_bf16_activation_in_w4a4(orc):
    """In W4A4 mode the adapter reads the bf16 tokens, not their NVFP4
    quantization: with the base weights zero, the W4A4 and W4A16 layers are
    the same function of x."""
    rng = np.random.default_rng(28)
    T, E, k, H, I, r = 4, 2, 2, 64, 32, 8
    z13 = np.zeros((E, 2 * I, H), np.uint16)
    z2 = np.zeros((E, H, I), np.uint16)
    q = _quant_experts(orc, z13, z2)
    x = wl.activations(T, H, seed=29)
    ids, w = wl.moe_routing(T, E, k, seed=30)
    lora = {"a13": wl.normal_bf16(rng, (r, H), 0.1), "b13": wl.normal_bf16(rng, (E, 2 * I, r), 0.1),
            "a2": wl.normal_bf16(rng, (r, I), 0.1), "b2": wl.normal_bf16(rng, (E, H, r), 0.1), "scale": 1.0}
    a13 = np.full(E, 1e-3, np.float32)    # a badly saturating activation scale
    a2 = np.full(E, 1e-3, np.float32)
    w16 = orc.moe(x, ids, w, *q, mode=0, lora=lora)
    w4 = orc.moe(x, ids, w, *q, mode=1, a13=a13, a2=a2, lora=lora)
    assert np.abs(w16).max() > 0
    np.testing.assert_array_equal(w4, w16)
