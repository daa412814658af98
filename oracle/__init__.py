"""CPU oracle for NVFP4 quantization and the block-scaled products.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
never links, loads or calls it, and it shares no code with the library.

The arithmetic lives in ``nvfp4_oracle.c`` (plain C, built with gcc as
``liborc.so``); this module only marshals numpy arrays through ctypes.
Every function states the passage it follows in the C source.

Arrays: bf16 tensors are carried as ``numpy.uint16`` bit patterns; packed
E2M1 codes and E4M3 scale bytes as ``numpy.uint8``; products come back as
``numpy.float64``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liborc.so")
_LIB = None

CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
          "-std=c11", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile ``liborc.so`` with gcc (no GPU code involved)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        F = ctypes.c_float
        U32 = ctypes.c_uint32
        sig = {
            "orc_e2m1_value": (ctypes.c_double, [U32]),
            "orc_e4m3_value": (ctypes.c_double, [U32]),
            "orc_e4m3_encode": (U32, [F]),
            "orc_e2m1_encode_mag": (U32, [F]),
            "orc_e4m3_encode_array": (None, [P, I64, P]),
            "orc_e2m1_encode_mag_array": (None, [P, I64, P]),
            "orc_bf16_to_f32": (F, [ctypes.c_uint16]),
            "orc_f32_to_bf16": (ctypes.c_uint16, [F]),
            "orc_f64_to_bf16": (ctypes.c_uint16, [ctypes.c_double]),
            "orc_f32_to_bf16_array": (None, [P, I64, P]),
            "orc_global_scale": (F, [P, I64]),
            "orc_quantize": (None, [P, I64, I64, F, P, P]),
            "orc_dequantize": (None, [P, P, F, I64, I64, P, P]),
            "orc_gemv_w4a16": (None, [P, I64, I64, I64, P, P, F, P]),
            "orc_gemm_w4a4": (None, [P, F, I64, I64, I64, P, P, F, P]),
            "orc_moe": (None, [I64, I64, I64, I64, I64, ctypes.c_int32, P, P, P,
                               P, P, P, P, P, P, P, P, P, P]),
            "orc_moe_lora": (None, [I64, I64, I64, I64, I64, ctypes.c_int32, P, P, P,
                                    P, P, P, P, P, P, P, P, I64, F, P, P, P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


# ------------------------------------------------------------------ formats --

def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code (sign in bit 3)."""
    return _lib().orc_e2m1_value(code)


def e4m3_value(byte: int) -> float:
    """Value of an E4M3 ("fn") byte; NaN for 0x7F / 0xFF."""
    return _lib().orc_e4m3_value(byte)


def e4m3_encode(f: float) -> int:
    """Nearest E4M3 byte to a non-negative float (ties even, saturating)."""
    return _lib().orc_e4m3_encode(f)


def e2m1_encode_mag(v: float) -> int:
    """Nearest E2M1 magnitude code (0..7) to a non-negative float."""
    return _lib().orc_e2m1_encode_mag(v)


def e4m3_encode_array(f) -> np.ndarray:
    f = _c(f, np.float32)
    out = np.empty(f.shape, np.uint8)
    _lib().orc_e4m3_encode_array(_ptr(f), f.size, _ptr(out))
    return out


def e2m1_encode_mag_array(f) -> np.ndarray:
    f = _c(f, np.float32)
    out = np.empty(f.shape, np.uint8)
    _lib().orc_e2m1_encode_mag_array(_ptr(f), f.size, _ptr(out))
    return out


def f32_to_bf16(f) -> np.ndarray:
    f = _c(f, np.float32)
    out = np.empty(f.shape, np.uint16)
    _lib().orc_f32_to_bf16_array(_ptr(f), f.size, _ptr(out))
    return out


def f64_to_bf16_scalar(v: float) -> int:
    return _lib().orc_f64_to_bf16(v)


# --------------------------------------------------------- quantize / deq --

def global_scale(x_bf16) -> float:
    """fp32 amax(|x|) / (6 * 448)."""
    x = _c(x_bf16, np.uint16)
    return float(np.float32(_lib().orc_global_scale(_ptr(x), x.size)))


def quantize(x_bf16, global_scale_value=None):
    """Quantize bf16 [rows, cols] to (codes [rows, cols/2], scales [rows, cols/16], Sg).

    ``global_scale_value`` None = dynamic (Sg = amax / 2688); a float = static.
    """
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    if cols % 16:
        raise ValueError("cols must be a multiple of 16")
    sg = global_scale(x) if global_scale_value is None else float(np.float32(global_scale_value))
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 16), np.uint8)
    _lib().orc_quantize(_ptr(x), rows, cols, sg, _ptr(codes), _ptr(scales))
    return codes, scales, np.float32(sg)


def dequantize(codes, scales, sg, want_bf16: bool = False):
    """fp32 fl(fl(q*s)*Sg) [rows, cols]; with ``want_bf16`` also its RNE bf16."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    rows, half = codes.shape
    cols = half * 2
    out = np.empty((rows, cols), np.float32)
    outb = np.empty((rows, cols), np.uint16) if want_bf16 else None
    _lib().orc_dequantize(_ptr(codes), _ptr(scales), float(sg), rows, cols, _ptr(out), _ptr(outb))
    return (out, outb) if want_bf16 else out


# ---------------------------------------------------------------- products --

def gemv_w4a16(x_bf16, w_codes, w_scales, w_global) -> np.ndarray:
    """y[M, N] = x . deq(W)^T in fp64; x bf16 [M, K], W NVFP4 [N, K]."""
    x = _c(x_bf16, np.uint16)
    wc = _c(w_codes, np.uint8)
    ws = _c(w_scales, np.uint8)
    M, K = x.shape
    N = wc.shape[0]
    assert wc.shape == (N, K // 2) and ws.shape == (N, K // 16)
    y = np.empty((M, N), np.float64)
    _lib().orc_gemv_w4a16(_ptr(x), M, N, K, _ptr(wc), _ptr(ws), float(w_global), _ptr(y))
    return y


def gemm_w4a4(x_bf16, input_scale, w_codes, w_scales, w_global) -> np.ndarray:
    """y[M, N] = deq(quant(X, input_scale)) . deq(W)^T in fp64."""
    x = _c(x_bf16, np.uint16)
    wc = _c(w_codes, np.uint8)
    ws = _c(w_scales, np.uint8)
    M, K = x.shape
    N = wc.shape[0]
    assert wc.shape == (N, K // 2) and ws.shape == (N, K // 16)
    y = np.empty((M, N), np.float64)
    _lib().orc_gemm_w4a4(_ptr(x), float(np.float32(input_scale)), M, N, K, _ptr(wc), _ptr(ws),
                         float(w_global), _ptr(y))
    return y


def moe(x_bf16, topk_ids, topk_w, w13_codes, w13_scales, w13_global, w2_codes, w2_scales,
        w2_global, mode: int = 0, a13=None, a2=None, want_h: bool = False, lora=None):
    """Routed-expert MoE layer; returns out [T, H] fp64 (and h bf16 [T*k, I]).

    ``lora`` (optional) is a dict with ``scale`` (float) and the bf16 adapter
    tensors ``a13`` [r, H], ``b13`` [E, 2I, r], ``a2`` [r, I], ``b2`` [E, H, r];
    either pair may be ``None`` (no adapter on that projection).  The overlay
    follows ``orc_moe_lora`` in nvfp4_oracle.c.
    """
    x = _c(x_bf16, np.uint16)
    ids = _c(topk_ids, np.int32)
    w = _c(topk_w, np.float32)
    w13c = _c(w13_codes, np.uint8)
    w13s = _c(w13_scales, np.uint8)
    w13g = _c(w13_global, np.float32)
    w2c = _c(w2_codes, np.uint8)
    w2s = _c(w2_scales, np.uint8)
    w2g = _c(w2_global, np.float32)
    T, H = x.shape
    k = ids.shape[1]
    E, twoI, _ = w13c.shape
    I = twoI // 2
    assert w13c.shape == (E, 2 * I, H // 2) and w13s.shape == (E, 2 * I, H // 16)
    assert w2c.shape == (E, H, I // 2) and w2s.shape == (E, H, I // 16)
    if mode == 1:
        a13 = _c(a13, np.float32)
        a2 = _c(a2, np.float32)
    out = np.empty((T, H), np.float64)
    h = np.empty((T * k, I), np.uint16) if want_h else None
    rank, scale, la13, lb13, la2, lb2 = 0, 0.0, None, None, None, None
    if lora is not None:
        if lora.get("a13") is not None:
            la13 = _c(lora["a13"], np.uint16)
            lb13 = _c(lora["b13"], np.uint16)
            rank = la13.shape[0]
            assert la13.shape == (rank, H) and lb13.shape == (E, 2 * I, rank)
        if lora.get("a2") is not None:
            la2 = _c(lora["a2"], np.uint16)
            lb2 = _c(lora["b2"], np.uint16)
            assert rank in (0, la2.shape[0])
            rank = la2.shape[0]
            assert la2.shape == (rank, I) and lb2.shape == (E, H, rank)
        scale = float(np.float32(lora["scale"]))
    _lib().orc_moe_lora(T, E, k, H, I, mode, _ptr(x), _ptr(ids), _ptr(w), _ptr(w13c), _ptr(w13s),
                        _ptr(w13g), _ptr(w2c), _ptr(w2s), _ptr(w2g),
                        _ptr(a13) if mode == 1 else None, _ptr(a2) if mode == 1 else None,
                        rank, scale, _ptr(la13), _ptr(lb13), _ptr(la2), _ptr(lb2),
                        _ptr(out), _ptr(h))
    return (out, h) if want_h else out
