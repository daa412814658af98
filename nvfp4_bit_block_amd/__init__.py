"""Python binding of the gfx950 NVFP4 library (``libnvfp4.so``).

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
of ``include/nvfp4.h``.  torch supplies device memory and the current stream;
bf16 tensors are ``torch.bfloat16`` (or int16/uint16 bit patterns), packed codes
and E4M3 scale bytes ``torch.uint8``, global scales 1-element fp32 device
tensors.  If the library has not been built the import of any entry point
raises; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "nvfp4.h")

NVFP4_OK = 0
MODE_W4A16 = 0
MODE_W4A4 = 1

_LIB = None


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({_status_text(status)}): {detail}")
        self.status = status


class MoeProblem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("E", ctypes.c_int64), ("top_k", ctypes.c_int64),
                ("H", ctypes.c_int64), ("I", ctypes.c_int64), ("mode", ctypes.c_int32)]


class MoeTensors(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "x", "topk_ids", "topk_weights", "w13_codes", "w13_scales", "w13_global",
        "w2_codes", "w2_scales", "w2_global", "a13_scale", "a2_scale", "out")]


class MoeLora(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int64), ("scale", ctypes.c_float), ("a13", ctypes.c_void_p),
                ("b13", ctypes.c_void_p), ("a2", ctypes.c_void_p), ("b2", ctypes.c_void_p)]


def header_functions() -> list[str]:
    """Names of the entry points declared in include/nvfp4.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:size_t|int32_t|const char\*)\s+(nvfp4_\w+)\s*\(", text, re.M)))


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m nvfp4_bit_block_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, SZ, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int32
        sigs = {
            "nvfp4_version": (I32, []),
            "nvfp4_status_string": (ctypes.c_char_p, [I32]),
            "nvfp4_last_error": (ctypes.c_char_p, []),
            "nvfp4_quantize_workspace_size": (SZ, [I64, I64]),
            "nvfp4_quantize": (I32, [P, I64, I64, P, P, P, P, P, SZ, P]),
            "nvfp4_dequantize": (I32, [P, P, P, I64, I64, P, P]),
            "nvfp4_gemv_w4a16": (I32, [P, I64, I64, I64, P, P, P, P, P]),
            "nvfp4_gemm_w4a4_workspace_size": (SZ, [I64, I64, I64]),
            "nvfp4_gemm_w4a4": (I32, [P, P, I64, I64, I64, P, P, P, P, P, SZ, P]),
            "nvfp4_quantize_columnwise": (I32, [P, I64, I64, P, P, P, P, P, SZ, P]),
            "nvfp4_dequantize_transpose": (I32, [P, P, P, I64, I64, P, P]),
            "nvfp4_gemm_w4a4_packed_workspace_size": (SZ, [I64, I64, I64]),
            "nvfp4_gemm_w4a4_packed": (I32, [P, P, P, I64, I64, I64, P, P, P, P, P, SZ, P]),
            "nvfp4_gemm_w4a16_workspace_size": (SZ, [I64, I64, I64]),
            "nvfp4_gemm_w4a16": (I32, [P, I64, I64, I64, P, P, P, P, P, SZ, P]),
            "nvfp4_moe_workspace_size": (SZ, [ctypes.POINTER(MoeProblem)]),
            "nvfp4_moe_grouped_gemm": (I32, [ctypes.POINTER(MoeProblem), ctypes.POINTER(MoeTensors),
                                             P, SZ, P]),
            "nvfp4_moe_lora_workspace_size": (SZ, [ctypes.POINTER(MoeProblem), ctypes.POINTER(MoeLora)]),
            "nvfp4_moe_grouped_gemm_lora": (I32, [ctypes.POINTER(MoeProblem), ctypes.POINTER(MoeTensors),
                                                  ctypes.POINTER(MoeLora), P, SZ, P]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def _status_text(status: int) -> str:
    try:
        return lib().nvfp4_status_string(status).decode()
    except Exception:  # pragma: no cover - only while reporting another failure
        return "?"


def _check(status: int, where: str):
    if status != NVFP4_OK:
        raise Nvfp4Error(status, where, lib().nvfp4_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _bf16(t: torch.Tensor) -> torch.Tensor:
    if t.dtype in (torch.int16, torch.uint16):
        return t
    if t.dtype != torch.bfloat16:
        raise TypeError(f"expected bf16, got {t.dtype}")
    return t


def _dev_scalar(v, device) -> torch.Tensor:
    if isinstance(v, torch.Tensor):
        if v.dtype != torch.float32 or v.numel() < 1:
            raise TypeError("scales are fp32 device tensors")
        return v
    return torch.tensor([float(v)], dtype=torch.float32, device=device)


def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


# ------------------------------------------------------------------ sizes --

def quantize_workspace_size(rows: int, cols: int) -> int:
    return int(lib().nvfp4_quantize_workspace_size(rows, cols))


def gemm_w4a4_workspace_size(M: int, N: int, K: int) -> int:
    return int(lib().nvfp4_gemm_w4a4_workspace_size(M, N, K))


def gemm_w4a16_workspace_size(M: int, N: int, K: int) -> int:
    return int(lib().nvfp4_gemm_w4a16_workspace_size(M, N, K))


def moe_workspace_size(T, E, top_k, H, I, mode) -> int:
    p = MoeProblem(T, E, top_k, H, I, mode)
    return int(lib().nvfp4_moe_workspace_size(ctypes.byref(p)))


def _moe_lora(lora) -> MoeLora | None:
    """dict(scale=..., a13=, b13=, a2=, b2=) of bf16 device tensors (either
    pair may be None) -> the C struct; the rank is read off the A tensors."""
    if lora is None:
        return None
    rank = 0
    for name in ("a13", "a2"):
        if lora.get(name) is not None:
            rank = lora[name].shape[0]
    if lora.get("rank") is not None:
        rank = int(lora["rank"])
    return MoeLora(rank, float(lora["scale"]), *[None if lora.get(n) is None else _bf16(lora[n]).data_ptr()
                                                 for n in ("a13", "b13", "a2", "b2")])


def moe_lora_workspace_size(T, E, top_k, H, I, mode, lora) -> int:
    p = MoeProblem(T, E, top_k, H, I, mode)
    c = _moe_lora(lora)
    return int(lib().nvfp4_moe_lora_workspace_size(ctypes.byref(p), None if c is None else ctypes.byref(c)))


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------ entry points --

def quantize(x, static_scale=None, codes=None, scales=None, global_scale=None, ws=None, stream=None):
    """nvfp4_quantize: returns (codes [R, C/2], scales [R, C/16], global_scale [1])."""
    x = _bf16(x)
    rows, cols = x.shape
    dev = x.device
    codes = _empty((rows, cols // 2), torch.uint8, dev) if codes is None else codes
    scales = _empty((rows, cols // 16), torch.uint8, dev) if scales is None else scales
    global_scale = _empty((1,), torch.float32, dev) if global_scale is None else global_scale
    sst = None if static_scale is None else _dev_scalar(static_scale, dev)
    need = 0 if sst is not None else quantize_workspace_size(rows, cols)
    if ws is None and need:
        ws = workspace(need, dev)
    _check(lib().nvfp4_quantize(_ptr(x), rows, cols, _ptr(sst), _ptr(codes), _ptr(scales),
                                _ptr(global_scale), _ptr(ws), 0 if ws is None else ws.numel(),
                                _stream(stream)), "nvfp4_quantize")
    return codes, scales, global_scale


def quantize_columnwise(x, static_scale=None, codes=None, scales=None, global_scale=None, ws=None,
                        stream=None):
    """nvfp4_quantize_columnwise: NVFP4 of x^T; returns (codes [C, R/2], scales [C, R/16], global [1])."""
    x = _bf16(x)
    rows, cols = x.shape
    dev = x.device
    codes = _empty((cols, rows // 2), torch.uint8, dev) if codes is None else codes
    scales = _empty((cols, rows // 16), torch.uint8, dev) if scales is None else scales
    global_scale = _empty((1,), torch.float32, dev) if global_scale is None else global_scale
    sst = None if static_scale is None else _dev_scalar(static_scale, dev)
    need = 0 if sst is not None else quantize_workspace_size(rows, cols)
    if ws is None and need:
        ws = workspace(need, dev)
    _check(lib().nvfp4_quantize_columnwise(_ptr(x), rows, cols, _ptr(sst), _ptr(codes), _ptr(scales),
                                           _ptr(global_scale), _ptr(ws), 0 if ws is None else ws.numel(),
                                           _stream(stream)), "nvfp4_quantize_columnwise")
    return codes, scales, global_scale


def dequantize_transpose(codes, scales, global_scale, out=None, stream=None):
    """nvfp4_dequantize_transpose: bf16 [C, R] transpose of the dequantized [R, C] tensor."""
    rows, half = codes.shape
    out = _empty((half * 2, rows), torch.bfloat16, codes.device) if out is None else out
    _check(lib().nvfp4_dequantize_transpose(_ptr(codes), _ptr(scales), _ptr(global_scale), rows, half * 2,
                                            _ptr(out), _stream(stream)), "nvfp4_dequantize_transpose")
    return out


def dequantize(codes, scales, global_scale, out=None, stream=None):
    rows, half = codes.shape
    out = _empty((rows, half * 2), torch.bfloat16, codes.device) if out is None else out
    _check(lib().nvfp4_dequantize(_ptr(codes), _ptr(scales), _ptr(global_scale), rows, half * 2,
                                  _ptr(out), _stream(stream)), "nvfp4_dequantize")
    return out


def gemv_w4a16(x, w_codes, w_scales, w_global, out=None, stream=None):
    x = _bf16(x)
    M, K = x.shape
    N = w_codes.shape[0]
    out = _empty((M, N), torch.bfloat16, x.device) if out is None else out
    _check(lib().nvfp4_gemv_w4a16(_ptr(x), M, N, K, _ptr(w_codes), _ptr(w_scales), _ptr(w_global),
                                  _ptr(out), _stream(stream)), "nvfp4_gemv_w4a16")
    return out


def gemm_w4a4(x, input_scale, w_codes, w_scales, w_global, out=None, ws=None, stream=None):
    x = _bf16(x)
    M, K = x.shape
    N = w_codes.shape[0]
    dev = x.device
    isc = _dev_scalar(input_scale, dev)
    out = _empty((M, N), torch.bfloat16, dev) if out is None else out
    if ws is None:
        ws = workspace(gemm_w4a4_workspace_size(M, N, K), dev)
    _check(lib().nvfp4_gemm_w4a4(_ptr(x), _ptr(isc), M, N, K, _ptr(w_codes), _ptr(w_scales),
                                 _ptr(w_global), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)),
           "nvfp4_gemm_w4a4")
    return out


def gemm_w4a4_packed(a_codes, a_scales, a_global, w_codes, w_scales, w_global, out=None, ws=None,
                     stream=None):
    M, half = a_codes.shape
    K = half * 2
    N = w_codes.shape[0]
    dev = a_codes.device
    out = _empty((M, N), torch.bfloat16, dev) if out is None else out
    if ws is None:
        ws = workspace(int(lib().nvfp4_gemm_w4a4_packed_workspace_size(M, N, K)), dev)
    _check(lib().nvfp4_gemm_w4a4_packed(_ptr(a_codes), _ptr(a_scales), _ptr(a_global), M, N, K, _ptr(w_codes),
                                        _ptr(w_scales), _ptr(w_global), _ptr(out), _ptr(ws), ws.numel(),
                                        _stream(stream)),
           "nvfp4_gemm_w4a4_packed")
    return out


def gemm_w4a16(x, w_codes, w_scales, w_global, out=None, ws=None, stream=None):
    x = _bf16(x)
    M, K = x.shape
    N = w_codes.shape[0]
    dev = x.device
    out = _empty((M, N), torch.bfloat16, dev) if out is None else out
    if ws is None:
        ws = workspace(gemm_w4a16_workspace_size(M, N, K), dev)
    _check(lib().nvfp4_gemm_w4a16(_ptr(x), M, N, K, _ptr(w_codes), _ptr(w_scales), _ptr(w_global),
                                  _ptr(out), _ptr(ws), ws.numel(), _stream(stream)),
           "nvfp4_gemm_w4a16")
    return out


def moe_grouped_gemm(x, topk_ids, topk_weights, w13_codes, w13_scales, w13_global, w2_codes,
                     w2_scales, w2_global, mode=MODE_W4A16, a13_scale=None, a2_scale=None,
                     out=None, ws=None, stream=None, lora=None):
    """The routed-expert layer; ``lora`` (optional) is a dict with ``scale``
    and the bf16 adapter tensors ``a13``/``b13`` and ``a2``/``b2`` (either
    pair may be None) and runs nvfp4_moe_grouped_gemm_lora."""
    x = _bf16(x)
    T, H = x.shape
    k = topk_ids.shape[1]
    E, twoI, _ = w13_codes.shape
    I = twoI // 2
    dev = x.device
    out = _empty((T, H), torch.bfloat16, dev) if out is None else out
    p = MoeProblem(T, E, k, H, I, mode)
    c = _moe_lora(lora)
    if ws is None:
        n = (lib().nvfp4_moe_workspace_size(ctypes.byref(p)) if c is None else
             lib().nvfp4_moe_lora_workspace_size(ctypes.byref(p), ctypes.byref(c)))
        ws = workspace(n, dev)
    t = MoeTensors(*[None if v is None else v.data_ptr() for v in (
        x, topk_ids, topk_weights, w13_codes, w13_scales, w13_global, w2_codes, w2_scales,
        w2_global, a13_scale, a2_scale, out)])
    if c is None:
        _check(lib().nvfp4_moe_grouped_gemm(ctypes.byref(p), ctypes.byref(t), _ptr(ws), ws.numel(),
                                            _stream(stream)), "nvfp4_moe_grouped_gemm")
    else:
        _check(lib().nvfp4_moe_grouped_gemm_lora(ctypes.byref(p), ctypes.byref(t), ctypes.byref(c), _ptr(ws),
                                                 ws.numel(), _stream(stream)), "nvfp4_moe_grouped_gemm_lora")
    return out
