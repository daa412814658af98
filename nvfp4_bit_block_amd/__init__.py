"""Python binding of the gfx950 NVFP4 library (``libnvfp4.so``).

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
of ``include/nvfp4.h``.  torch supplies device memory and the current stream;
bf16 tensors are ``torch.bfloat16`` (or int16/uint16 bit patterns), packed codes
and E4M3 scale bytes ``torch.uint8``, global scales 1-element fp32 device
tensors.  If the library has not been built the import of any entry point
raises; there is no fallback implementation.
"""
from __future__ import annotations

import contextlib
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
            "nvfp4_quantize_noalloc": (I32, [P, I64, I64, P, P, P, P, P]),
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


@contextlib.contextmanager
def _on(stream):
    """Run a wrapper body with `stream` current, so that every temporary it
    allocates (outputs, workspace, device scalars) belongs to the stream the
    kernels run on and is not handed to other work while they still use it."""
    if stream is None:
        yield
    else:
        with torch.cuda.stream(stream):
            yield


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_U8 = (torch.uint8,)
_F32 = (torch.float32,)
_I32 = (torch.int32,)


def _req(t, name: str, dtypes, shape=None, device=None):
    """Check one tensor argument before its address is passed on: dtype, shape
    (None entries match any size), contiguity and, when `device` is given,
    that it lives there.  Raises TypeError or ValueError."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        want = " or ".join(str(d).replace("torch.", "") for d in dtypes)
        raise TypeError(f"{name}: expected dtype {want}, got {str(t.dtype).replace('torch.', '')}")
    if shape is not None:
        ok = t.dim() == len(shape) and all(w is None or w == g for w, g in zip(shape, t.shape))
        if not ok:
            want = "[" + ", ".join("*" if w is None else str(w) for w in shape) + "]"
            raise ValueError(f"{name}: expected shape {want}, got {list(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if device is not None:
        _cuda(t, name, device)
    return t


def _cuda(t, name: str, device=None):
    """t lives on a CUDA device (on `device` when given)."""
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be on a CUDA device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    return t


def _bf16(t: torch.Tensor, name: str = "x", shape=None, device=None) -> torch.Tensor:
    return _req(t, name, _BF16, shape, device)


def _dev_scalar(v, device, name="scale") -> torch.Tensor:
    if isinstance(v, torch.Tensor):
        _req(v, name, _F32, device=device)
        if v.numel() < 1:
            raise ValueError(f"{name}: needs at least one element")
        return v
    return torch.tensor([float(v)], dtype=torch.float32, device=device)


def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


def _weights(w_codes, w_scales, w_global, K, device):
    """NVFP4 weight [N, K]: codes uint8 [N, K/2], scales uint8 [N, K/16],
    global fp32 [>= 1]; returns N."""
    _req(w_codes, "w_codes", _U8, (None, K // 2), device)
    N = w_codes.shape[0]
    _req(w_scales, "w_scales", _U8, (N, K // 16), device)
    _dev_scalar(w_global, device, "w_global")
    return N


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


def _moe_lora(lora, E=None, H=None, I=None, device=None) -> MoeLora | None:
    """dict(scale=..., a13=, b13=, a2=, b2=) of bf16 device tensors (either
    pair may be None) -> the C struct; the rank is read off the A tensors.
    With the layer's E, H, I the adapter shapes are checked: a13 [R, H], b13
    [E, 2I, R], a2 [R, I], b2 [E, H, R]."""
    if lora is None:
        return None
    rank = 0
    for name in ("a13", "a2"):
        if lora.get(name) is not None:
            rank = lora[name].shape[0]
    if lora.get("rank") is not None:
        rank = int(lora["rank"])
    shapes = {"a13": (rank, H), "b13": (E, None if I is None else 2 * I, rank), "a2": (rank, I), "b2": (E, H, rank)}
    ptrs = []
    for n in ("a13", "b13", "a2", "b2"):
        t = lora.get(n)
        if t is not None:
            _bf16(t, "lora " + n, shapes[n] if E is not None else None, device)
        ptrs.append(None if t is None else t.data_ptr())
    return MoeLora(rank, float(lora["scale"]), *ptrs)


def moe_lora_workspace_size(T, E, top_k, H, I, mode, lora) -> int:
    p = MoeProblem(T, E, top_k, H, I, mode)
    c = _moe_lora(lora)
    return int(lib().nvfp4_moe_lora_workspace_size(ctypes.byref(p), None if c is None else ctypes.byref(c)))


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------ entry points --
#
# Every wrapper checks its tensor arguments (dtype, shape, contiguity, one
# CUDA device) before any address reaches the library, and allocates its
# temporaries with the launch stream current.

def quantize(x, static_scale=None, codes=None, scales=None, global_scale=None, ws=None, stream=None):
    """nvfp4_quantize: returns (codes [R, C/2], scales [R, C/16], global_scale [1])."""
    _cuda(_bf16(x, "x", (None, None)), "x")
    rows, cols = x.shape
    dev = x.device
    with _on(stream):
        codes = _empty((rows, cols // 2), torch.uint8, dev) if codes is None else _req(codes, "codes", _U8, (rows, cols // 2), dev)
        scales = _empty((rows, cols // 16), torch.uint8, dev) if scales is None else _req(scales, "scales", _U8, (rows, cols // 16), dev)
        global_scale = _empty((1,), torch.float32, dev) if global_scale is None else _dev_scalar(global_scale, dev, "global_scale")
        sst = None if static_scale is None else _dev_scalar(static_scale, dev, "static_scale")
        need = 0 if sst is not None else quantize_workspace_size(rows, cols)
        if ws is None and need:
            ws = workspace(need, dev)
        elif ws is not None:
            _req(ws, "ws", _U8, device=dev)
        _check(lib().nvfp4_quantize(_ptr(x), rows, cols, _ptr(sst), _ptr(codes), _ptr(scales),
                                    _ptr(global_scale), _ptr(ws), 0 if ws is None else ws.numel(),
                                    _stream(stream)), "nvfp4_quantize")
    return codes, scales, global_scale


def quantize_columnwise(x, static_scale=None, codes=None, scales=None, global_scale=None, ws=None,
                        stream=None):
    """nvfp4_quantize_columnwise: NVFP4 of x^T; returns (codes [C, R/2], scales [C, R/16], global [1])."""
    _cuda(_bf16(x, "x", (None, None)), "x")
    rows, cols = x.shape
    dev = x.device
    with _on(stream):
        codes = _empty((cols, rows // 2), torch.uint8, dev) if codes is None else _req(codes, "codes", _U8, (cols, rows // 2), dev)
        scales = _empty((cols, rows // 16), torch.uint8, dev) if scales is None else _req(scales, "scales", _U8, (cols, rows // 16), dev)
        global_scale = _empty((1,), torch.float32, dev) if global_scale is None else _dev_scalar(global_scale, dev, "global_scale")
        sst = None if static_scale is None else _dev_scalar(static_scale, dev, "static_scale")
        need = 0 if sst is not None else quantize_workspace_size(rows, cols)
        if ws is None and need:
            ws = workspace(need, dev)
        elif ws is not None:
            _req(ws, "ws", _U8, device=dev)
        _check(lib().nvfp4_quantize_columnwise(_ptr(x), rows, cols, _ptr(sst), _ptr(codes), _ptr(scales),
                                               _ptr(global_scale), _ptr(ws), 0 if ws is None else ws.numel(),
                                               _stream(stream)), "nvfp4_quantize_columnwise")
    return codes, scales, global_scale


def _nvfp4_tensor(codes, scales, global_scale):
    """A packed NVFP4 tensor [R, C]: codes uint8 [R, C/2], scales uint8
    [R, C/16], global fp32; returns (R, C)."""
    _cuda(_req(codes, "codes", _U8, (None, None)), "codes")
    rows, half = codes.shape
    _req(scales, "scales", _U8, (rows, half * 2 // 16), codes.device)
    _dev_scalar(global_scale, codes.device, "global_scale")
    return rows, half * 2


def dequantize_transpose(codes, scales, global_scale, out=None, stream=None):
    """nvfp4_dequantize_transpose: bf16 [C, R] transpose of the dequantized [R, C] tensor."""
    rows, cols = _nvfp4_tensor(codes, scales, global_scale)
    with _on(stream):
        out = _empty((cols, rows), torch.bfloat16, codes.device) if out is None else _bf16(out, "out", (cols, rows), codes.device)
        _check(lib().nvfp4_dequantize_transpose(_ptr(codes), _ptr(scales), _ptr(global_scale), rows, cols,
                                                _ptr(out), _stream(stream)), "nvfp4_dequantize_transpose")
    return out


def dequantize(codes, scales, global_scale, out=None, stream=None):
    rows, cols = _nvfp4_tensor(codes, scales, global_scale)
    with _on(stream):
        out = _empty((rows, cols), torch.bfloat16, codes.device) if out is None else _bf16(out, "out", (rows, cols), codes.device)
        _check(lib().nvfp4_dequantize(_ptr(codes), _ptr(scales), _ptr(global_scale), rows, cols,
                                      _ptr(out), _stream(stream)), "nvfp4_dequantize")
    return out


def gemv_w4a16(x, w_codes, w_scales, w_global, out=None, stream=None):
    _cuda(_bf16(x, "x", (None, None)), "x")
    M, K = x.shape
    N = _weights(w_codes, w_scales, w_global, K, x.device)
    with _on(stream):
        out = _empty((M, N), torch.bfloat16, x.device) if out is None else _bf16(out, "out", (M, N), x.device)
        _check(lib().nvfp4_gemv_w4a16(_ptr(x), M, N, K, _ptr(w_codes), _ptr(w_scales), _ptr(w_global),
                                      _ptr(out), _stream(stream)), "nvfp4_gemv_w4a16")
    return out


def gemm_w4a4(x, input_scale, w_codes, w_scales, w_global, out=None, ws=None, stream=None):
    _cuda(_bf16(x, "x", (None, None)), "x")
    M, K = x.shape
    dev = x.device
    N = _weights(w_codes, w_scales, w_global, K, dev)
    with _on(stream):
        isc = _dev_scalar(input_scale, dev, "input_scale")
        out = _empty((M, N), torch.bfloat16, dev) if out is None else _bf16(out, "out", (M, N), dev)
        if ws is None:
            ws = workspace(gemm_w4a4_workspace_size(M, N, K), dev)
        _req(ws, "ws", _U8, device=dev)
        _check(lib().nvfp4_gemm_w4a4(_ptr(x), _ptr(isc), M, N, K, _ptr(w_codes), _ptr(w_scales),
                                     _ptr(w_global), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)),
               "nvfp4_gemm_w4a4")
    return out


def gemm_w4a4_packed(a_codes, a_scales, a_global, w_codes, w_scales, w_global, out=None, ws=None,
                     stream=None):
    M, K = _nvfp4_tensor(a_codes, a_scales, a_global)
    dev = a_codes.device
    N = _weights(w_codes, w_scales, w_global, K, dev)
    with _on(stream):
        out = _empty((M, N), torch.bfloat16, dev) if out is None else _bf16(out, "out", (M, N), dev)
        if ws is None:
            ws = workspace(int(lib().nvfp4_gemm_w4a4_packed_workspace_size(M, N, K)), dev)
        _req(ws, "ws", _U8, device=dev)
        _check(lib().nvfp4_gemm_w4a4_packed(_ptr(a_codes), _ptr(a_scales), _ptr(a_global), M, N, K, _ptr(w_codes),
                                            _ptr(w_scales), _ptr(w_global), _ptr(out), _ptr(ws), ws.numel(),
                                            _stream(stream)),
               "nvfp4_gemm_w4a4_packed")
    return out


def gemm_w4a16(x, w_codes, w_scales, w_global, out=None, ws=None, stream=None):
    _cuda(_bf16(x, "x", (None, None)), "x")
    M, K = x.shape
    dev = x.device
    N = _weights(w_codes, w_scales, w_global, K, dev)
    with _on(stream):
        out = _empty((M, N), torch.bfloat16, dev) if out is None else _bf16(out, "out", (M, N), dev)
        if ws is None:
            ws = workspace(gemm_w4a16_workspace_size(M, N, K), dev)
        _req(ws, "ws", _U8, device=dev)
        _check(lib().nvfp4_gemm_w4a16(_ptr(x), M, N, K, _ptr(w_codes), _ptr(w_scales), _ptr(w_global),
                                      _ptr(out), _ptr(ws), ws.numel(), _stream(stream)),
               "nvfp4_gemm_w4a16")
    return out


def moe_grouped_gemm(x, topk_ids, topk_weights, w13_codes, w13_scales, w13_global, w2_codes,
                     w2_scales, w2_global, mode=MODE_W4A16, a13_scale=None, a2_scale=None,
                     out=None, ws=None, stream=None, lora=None):
    """The routed-expert layer; ``lora`` (optional) is a dict with ``scale``
    and the bf16 adapter tensors ``a13``/``b13`` and ``a2``/``b2`` (either
    pair may be None) and runs nvfp4_moe_grouped_gemm_lora.

    topk_ids must be int32 [T, k] (torch.topk returns int64: convert it) and
    topk_weights fp32 [T, k]."""
    # every dtype and shape first, then the devices
    _bf16(x, "x", (None, None))
    T, H = x.shape
    _req(topk_ids, "topk_ids", _I32, (T, None))
    k = topk_ids.shape[1]
    _req(topk_weights, "topk_weights", _F32, (T, k))
    _req(w13_codes, "w13_codes", _U8, (None, None, H // 2))
    E, twoI, _ = w13_codes.shape
    I = twoI // 2
    _req(w13_scales, "w13_scales", _U8, (E, 2 * I, H // 16))
    _req(w13_global, "w13_global", _F32, (E,))
    _req(w2_codes, "w2_codes", _U8, (E, H, I // 2))
    _req(w2_scales, "w2_scales", _U8, (E, H, I // 16))
    _req(w2_global, "w2_global", _F32, (E,))
    if mode not in (MODE_W4A16, MODE_W4A4):
        raise ValueError(f"mode must be MODE_W4A16 or MODE_W4A4, got {mode!r}")
    scales = []
    if mode == MODE_W4A4:
        if a13_scale is None or a2_scale is None:
            raise ValueError("W4A4 mode needs a13_scale and a2_scale")
        scales = [_req(a13_scale, "a13_scale", _F32, (E,)), _req(a2_scale, "a2_scale", _F32, (E,))]
    dev = _cuda(x, "x").device
    for t, n in zip((topk_ids, topk_weights, w13_codes, w13_scales, w13_global, w2_codes, w2_scales, w2_global,
                     *scales), ("topk_ids", "topk_weights", "w13_codes", "w13_scales", "w13_global", "w2_codes",
                                "w2_scales", "w2_global", "a13_scale", "a2_scale")):
        _cuda(t, n, dev)
    c = _moe_lora(lora, E, H, I, dev)
    with _on(stream):
        out = _empty((T, H), torch.bfloat16, dev) if out is None else _bf16(out, "out", (T, H), dev)
        p = MoeProblem(T, E, k, H, I, mode)
        if ws is None:
            n = (lib().nvfp4_moe_workspace_size(ctypes.byref(p)) if c is None else
                 lib().nvfp4_moe_lora_workspace_size(ctypes.byref(p), ctypes.byref(c)))
            ws = workspace(n, dev)
        _req(ws, "ws", _U8, device=dev)
        t = MoeTensors(*[None if v is None else v.data_ptr() for v in (
            x, topk_ids, topk_weights, w13_codes, w13_scales, w13_global, w2_codes, w2_scales,
            w2_global, a13_scale if mode == MODE_W4A4 else None, a2_scale if mode == MODE_W4A4 else None, out)])
        if c is None:
            _check(lib().nvfp4_moe_grouped_gemm(ctypes.byref(p), ctypes.byref(t), _ptr(ws), ws.numel(),
                                                _stream(stream)), "nvfp4_moe_grouped_gemm")
        else:
            _check(lib().nvfp4_moe_grouped_gemm_lora(ctypes.byref(p), ctypes.byref(t), ctypes.byref(c), _ptr(ws),
                                                     ws.numel(), _stream(stream)), "nvfp4_moe_grouped_gemm_lora")
    return out
