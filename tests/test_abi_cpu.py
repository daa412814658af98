"""The C-ABI library loads, exports every declared entry point, and rejects
invalid arguments on the host (no GPU needed: checks run before any HIP call).

Every call below either fails a host-side check or is a zero-size no-op, so no
kernel is ever launched with the fake addresses used here."""
import ctypes
import os

import pytest

import nvfp4_bit_block_amd as nv

pytestmark = pytest.mark.skipif(not os.path.exists(nv.LIB_PATH), reason="libnvfp4.so not built")

OK, NULL, SHAPE, ALIGN, UNSUP, WS = 0, 1, 2, 3, 4, 5
A = 4096          # a fake, 16-byte aligned, never dereferenced address
MIS = 4097        # misaligned


def test_exports_every_header_symbol():
    L = ctypes.CDLL(nv.LIB_PATH)
    names = nv.header_functions()
    assert len(names) == 20
    for n in names:
        assert hasattr(L, n), n


def test_version_and_strings():
    L = nv.lib()
    assert L.nvfp4_version() >= 100
    for s in range(7):
        assert L.nvfp4_status_string(s)


def test_quantize_validation():
    L = nv.lib()
    q = L.nvfp4_quantize
    assert q(None, 4, 32, None, A, A, A, A, 1 << 20, None) == NULL
    assert q(A, 4, 33, None, A, A, A, A, 1 << 20, None) == SHAPE
    assert q(A, -1, 32, None, A, A, A, A, 1 << 20, None) == SHAPE
    assert q(A, 4, 0, None, A, A, A, A, 1 << 20, None) == SHAPE
    assert q(MIS, 4, 32, None, A, A, A, A, 1 << 20, None) == ALIGN
    assert q(A, 4, 32, None, A, A, A, None, 0, None) == WS          # dynamic needs workspace
    assert q(A, 4, 32, None, A, A, A, A, 4, None) == WS
    assert q(A, 0, 32, None, A, A, A, A, 1 << 20, None) == OK       # empty: no-op
    assert q(A, 0, 32, A, A, A, A, None, 0, None) == OK             # static, empty
    assert q(None, 0, 32, None, None, None, None, None, 0, None) == OK   # empty ignores pointers
    assert L.nvfp4_quantize_workspace_size(65536, 6144) > 0
    assert b"cols" in L.nvfp4_last_error() or True


def test_quantize_noalloc_validation():
    q = nv.lib().nvfp4_quantize_noalloc
    q.restype = ctypes.c_int32
    q.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 5
    assert q(None, 4, 32, None, A, A, A, None) == NULL
    assert q(A, 4, 33, None, A, A, A, None) == SHAPE
    assert q(A, -1, 32, None, A, A, A, None) == SHAPE
    assert q(A, 1 << 62, 32, None, A, A, A, None) == UNSUP           # rows * cols overflows
    assert q(MIS, 4, 32, None, A, A, A, None) == ALIGN
    assert q(A, 4, 32, MIS, A, A, A, None) == ALIGN
    assert q(A, 0, 32, None, None, None, None, None) == OK           # empty: no-op


def test_dequantize_validation():
    d = nv.lib().nvfp4_dequantize
    assert d(None, A, A, 4, 32, A, None) == NULL
    assert d(A, A, A, 4, 24, A, None) == SHAPE
    assert d(A, A, A, 4, 32, MIS, None) == ALIGN
    assert d(A, A, A, 0, 32, A, None) == OK


def test_columnwise_and_transpose_validation():
    L = nv.lib()
    q = L.nvfp4_quantize_columnwise
    assert q(None, 32, 16, None, A, A, A, A, 1 << 20, None) == NULL
    assert q(A, 24, 16, None, A, A, A, A, 1 << 20, None) == SHAPE           # rows % 16
    assert q(A, 32, 12, None, A, A, A, A, 1 << 20, None) == UNSUP           # cols % 8
    assert q(A, 32, 16, None, MIS, A, A, A, 1 << 20, None) == ALIGN
    assert q(A, 32, 16, None, A, A, A, None, 0, None) == WS                  # dynamic needs workspace
    assert q(A, 0, 16, None, A, A, A, None, 0, None) == OK
    assert q(A, 65536 * 128, 16, None, A, A, A, A, 1 << 40, None) == UNSUP  # row tiles past the grid's y limit
    d = L.nvfp4_dequantize_transpose
    assert d(None, A, A, 8, 32, A, None) == NULL
    assert d(A, A, A, 8, 24, A, None) == SHAPE                               # cols % 16
    assert d(A, A, A, 12, 32, A, None) == UNSUP                              # rows % 8
    assert d(A, A, A, 8, 32, MIS, None) == ALIGN
    assert d(A, A, A, 0, 32, A, None) == OK
    assert d(A, A, A, 8, 65536 * 128, A, None) == UNSUP                      # column tiles past the grid's y limit


def test_gemv_validation():
    g = nv.lib().nvfp4_gemv_w4a16
    assert g(A, 1, 8, 64, A, A, A, None, None) == NULL
    assert g(A, 1, 8, 40, A, A, A, A, None) == SHAPE
    assert g(A, 9, 8, 64, A, A, A, A, None) == UNSUP
    assert g(A, 1, 8, 48, A, A, A, A, None) == UNSUP                 # K % 32 != 0
    assert g(A, 1, 8, 64, A, A, MIS, A, None) == ALIGN
    assert g(A, 1, 8, 64, A, A, A, A + 2, None) == ALIGN
    assert g(A, 0, 8, 64, A, A, A, A, None) == OK
    assert g(A, 3, 0, 64, A, A, A, A, None) == OK


def test_gemm_validation():
    L = nv.lib()
    g = L.nvfp4_gemm_w4a4
    ws = L.nvfp4_gemm_w4a4_workspace_size(128, 256, 512)
    assert ws > 0
    assert g(A, None, 128, 256, 512, A, A, A, A, A, ws, None) == NULL
    assert g(A, A, 128, 256, 520, A, A, A, A, A, ws, None) == SHAPE
    assert g(A, A, 128, 256, 528, A, A, A, A, A, 1 << 30, None) == UNSUP   # K % 64 != 0
    assert g(A, A, 128, 256, 512, A, A, A, A, A, ws - 1, None) == WS
    assert g(A, A, 128, 256, 512, A, A, A, A, None, 0, None) == WS
    assert g(A, A, 128, 256, 512, A, A, A, A, MIS, ws, None) == ALIGN
    assert g(A, A, 0, 256, 512, A, A, A, A, None, 0, None) == OK


def test_gemm_packed_validation():
    L = nv.lib()
    g = L.nvfp4_gemm_w4a4_packed
    ws = L.nvfp4_gemm_w4a4_packed_workspace_size(128, 256, 512)
    assert ws == L.nvfp4_gemm_w4a4_workspace_size(128, 256, 512) > 0
    assert g(A, A, None, 128, 256, 512, A, A, A, A, A, ws, None) == NULL
    assert g(A, A, A, 128, 256, 520, A, A, A, A, A, ws, None) == SHAPE
    assert g(A, A, A, 128, 256, 528, A, A, A, A, A, 1 << 30, None) == UNSUP   # K % 64 != 0
    assert g(A, A, A, 128, 256, 512, A, A, A, A, A, ws - 1, None) == WS
    assert g(A, A, A, 128, 256, 512, A, A, A, A, None, 0, None) == WS
    assert g(A, MIS, A, 128, 256, 512, A, A, A, A, A, ws, None) == ALIGN
    assert g(A, A, A, 0, 256, 512, A, A, A, A, None, 0, None) == OK


def test_gemm_w4a16_validation():
    L = nv.lib()
    g = L.nvfp4_gemm_w4a16
    ws = L.nvfp4_gemm_w4a16_workspace_size(128, 256, 4096)
    assert ws > 0                                            # split K: partial sums
    assert L.nvfp4_gemm_w4a16_workspace_size(4096, 16384, 2048) == 0   # 1024 tiles, no split
    # o_proj at M = 4096: 384 tiles of 256 x 256, K split in two (two fp32 partials)
    assert L.nvfp4_gemm_w4a16_workspace_size(4096, 6144, 16384) == 2 * 4096 * 6144 * 4
    # M = 1536: 144 tiles, stream-K over 256 workgroups of 144 * 256 / 256 =
    # 144 K steps each; a tile's 256 steps meet at most 3 workgroups (3 slots)
    assert L.nvfp4_gemm_w4a16_workspace_size(1536, 6144, 16384) == 3 * 1536 * 6144 * 4
    # M = 1024, N = 5632, K = 8192: 88 tiles of 128 steps, 44 steps a
    # workgroup, so a tile spans at most 4 workgroups
    assert L.nvfp4_gemm_w4a16_workspace_size(1024, 5632, 8192) == 4 * 1024 * 5632 * 4
    assert g(None, 128, 256, 4096, A, A, A, A, A, ws, None) == NULL
    assert g(A, 128, 256, 4100, A, A, A, A, A, ws, None) == SHAPE
    assert g(A, 128, 256, 4128, A, A, A, A, A, 1 << 30, None) == UNSUP   # K % 64 != 0
    assert g(A, 128, 256, 4096, A, A, A, A, A, ws - 1, None) == WS
    assert g(A, 128, 256, 4096, A, A, A, A, None, 0, None) == WS
    assert g(A, 128, 256, 4096, A, A, A, MIS, A, ws, None) == ALIGN
    assert g(A, 0, 256, 4096, A, A, A, A, None, 0, None) == OK
    assert g(A, 5, 0, 4096, A, A, A, A, None, 0, None) == OK


def test_moe_validation():
    L = nv.lib()
    p = nv.MoeProblem(64, 8, 2, 256, 128, 0)
    t = nv.MoeTensors(*([A] * 9 + [None, None, A]))
    ws = L.nvfp4_moe_workspace_size(ctypes.byref(p))
    assert ws > 0
    run = lambda pp, tt, w, n: L.nvfp4_moe_grouped_gemm(ctypes.byref(pp), ctypes.byref(tt), w, n, None)
    assert run(p, t, None, 0) == WS
    assert run(p, t, A, ws - 1) == WS
    assert run(nv.MoeProblem(64, 8, 2, 250, 128, 0), t, A, ws) == SHAPE
    assert run(nv.MoeProblem(64, 8, 2, 256, 128, 2), t, A, ws) == SHAPE
    assert run(nv.MoeProblem(64, 8, 2, 272, 128, 0), t, A, 1 << 40) == UNSUP   # H % 64 != 0
    assert run(nv.MoeProblem(64, 8, 2, 256, 128, 1), t, A, 1 << 40) == NULL    # W4A4 needs a13/a2
    t_mis = nv.MoeTensors(*([A] * 8 + [MIS, None, None, A]))
    assert run(p, t_mis, A, ws) == ALIGN
    t_words = nv.MoeTensors(*([A, A + 4, A + 8, A, A, A + 12, A, A, A + 4, None, None, A]))
    assert run(p, t_words, A, ws - 1) == WS     # 4-byte aligned fp32/int32 arrays pass the alignment check
    assert run(nv.MoeProblem(0, 8, 2, 256, 128, 0), t, None, 0) == OK
    assert run(nv.MoeProblem(0, 8, 2, 256, 128, 1), nv.MoeTensors(), None, 0) == OK


def test_moe_lora_validation():
    L = nv.lib()
    p = nv.MoeProblem(64, 8, 2, 256, 128, 0)
    t = nv.MoeTensors(*([A] * 9 + [None, None, A]))
    lo = nv.MoeLora(64, 1.0, A, A, A, A)
    base = L.nvfp4_moe_workspace_size(ctypes.byref(p))
    ws = L.nvfp4_moe_lora_workspace_size(ctypes.byref(p), ctypes.byref(lo))
    # the layer's workspace plus z13 [T, r] and z2 [T*k, r] in bf16 (256-byte aligned pieces)
    assert ws >= base + 64 * 64 * 2 + 128 * 64 * 2
    assert L.nvfp4_moe_lora_workspace_size(ctypes.byref(p), None) == base
    run = lambda pp, tt, ll, w, n: L.nvfp4_moe_grouped_gemm_lora(
        ctypes.byref(pp), ctypes.byref(tt), None if ll is None else ctypes.byref(ll), w, n, None)
    assert run(p, t, lo, A, ws - 1) == WS
    assert run(p, t, None, A, base - 1) == WS
    assert run(p, t, nv.MoeLora(0, 1.0, A, A, A, A), A, ws) == SHAPE
    assert run(p, t, nv.MoeLora(-8, 1.0, A, A, A, A), A, ws) == SHAPE
    assert run(p, t, nv.MoeLora(12, 1.0, A, A, A, A), A, 1 << 40) == UNSUP    # rank % 8 != 0
    assert run(p, t, nv.MoeLora(136, 1.0, A, A, A, A), A, 1 << 40) == UNSUP   # rank > 128
    assert run(p, t, nv.MoeLora(64, 1.0, A, None, A, A), A, ws) == NULL       # a13 without b13
    assert run(p, t, nv.MoeLora(64, 1.0, A, A, None, A), A, ws) == NULL       # b2 without a2
    assert run(p, t, nv.MoeLora(64, 1.0, A, A, MIS, A), A, ws) == ALIGN
    # one adapted projection is enough; the workspace check still comes last
    assert run(p, t, nv.MoeLora(64, 1.0, None, None, A, A), A, ws - 1) == WS
    assert run(p, t, nv.MoeLora(64, 1.0, A, A, None, None), A, ws - 1) == WS
    assert run(nv.MoeProblem(0, 8, 2, 256, 128, 0), t, lo, None, 0) == OK


def _streamk_parts(M, N, K, wgs=256, tile=256):
    """Most parts one 256 x 256 tile is cut into when wgs workgroups take the
    tiles' K steps in order, workgroup w the steps [w S / wgs, (w + 1) S / wgs)
    (brute force over the workgroups' ranges)."""
    ks = K // 64
    tiles = -(-M // tile) * -(-N // tile)
    S = tiles * ks
    parts = [0] * tiles
    for w in range(wgs):
        lo, hi = w * S // wgs, (w + 1) * S // wgs
        for t in range(lo // ks, (hi - 1) // ks + 1):
            parts[t] += 1
    return max(parts)


# Long rows on the 256 x 256 tile that take stream-K (the GPU parity cases and
# o_proj at M = 1536, 3072, 4096): the W4A16 workspace is the fp32 parts,
# [most parts per tile, M, N], 256-byte aligned.
@pytest.mark.parametrize("M,N,K", [(1400, 6001, 4160), (1536, 5888, 4352), (1700, 5000, 16384),
                                   (1024, 5632, 8192), (3000, 6000, 8320), (1536, 6144, 16384),
                                   (3072, 6144, 16384), (4096, 6144, 16384)])
def test_streamk_workspace_matches_partition(M, N, K):
    L = nv.lib()
    parts = _streamk_parts(M, N, K)
    assert 2 <= parts <= 8
    want = -(-(parts * M * N * 4) // 256) * 256
    assert L.nvfp4_gemm_w4a16_workspace_size(M, N, K) == want
