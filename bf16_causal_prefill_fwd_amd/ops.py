"""Thin ctypes binding of libattn_prefill.so (include/attn_prefill.h).

Argument marshalling only: every computation runs in the library's HIP
kernels. torch supplies device memory and the current HIP stream. The
library is loaded on first use; if it has not been built this raises -- there
is no fallback path.
"""

from __future__ import annotations

import ctypes
import math
import os
import re

import torch

from .build import LIB_PATH, INCLUDE

ATTN_OK = 0
ATTN_DTYPE_FP8_E4M3 = 0
ATTN_DTYPE_BF16 = 1

_lib = None

_c_void_p = ctypes.c_void_p
_c_int = ctypes.c_int
_c_float = ctypes.c_float
_c_int64 = ctypes.c_int64

_SIGNATURES = {
    "attn_prefill_fwd": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                  _c_float, _c_float, _c_float,
                                  _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                  _c_void_p]),
    "attn_prefill_fwd_ex": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                     _c_float, _c_float, _c_float, _c_void_p, _c_float,
                                     _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                     _c_void_p]),
    "attn_quantize_fp8": (_c_int, [_c_void_p, _c_int, _c_int64, _c_void_p, _c_void_p, _c_void_p]),
    "attn_quantize_fp8_q": (_c_int, [_c_void_p, _c_int, _c_int64, _c_void_p, _c_void_p, _c_void_p, _c_float,
                                     _c_void_p]),
    "attn_quantize_fp8_hadamard": (_c_int, [_c_void_p, _c_int, _c_int64, _c_int, _c_void_p, _c_void_p, _c_void_p,
                                            _c_float, _c_void_p]),
    "attn_quantize_fp8_qkv": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_int, _c_int64, _c_int64, _c_int64,
                                       _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_float, _c_void_p]),
    "attn_cast_bf16": (_c_int, [_c_void_p, _c_int64, _c_void_p, _c_void_p]),
    "attn_strerror": (ctypes.c_char_p, [_c_int]),
    "attn_abi_version": (_c_int, []),
}


class AttnError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {code} ({strerror(code)})")
        self.code = code


def header_functions() -> list[str]:
    """Names of the functions declared in include/attn_prefill.h."""
    text = open(os.path.join(INCLUDE, "attn_prefill.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(attn_\w+)\s*\(", text, flags=re.M)


def lib() -> ctypes.CDLL:
    """Load the library (once) and declare every exported signature."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m bf16_causal_prefill_fwd_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().attn_strerror(code).decode()


def _check(fn: str, code: int):
    if code != ATTN_OK:
        raise AttnError(fn, code)


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def attn_quantize_fp8(x: torch.Tensor, out: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                      stream=None, k_scale: torch.Tensor | None = None, softmax_scale: float | None = None,
                      hadamard: bool = False):
    """Per-tensor e4m3fn quantization on the device.

    With ``k_scale`` (the key tensor's device scale) and ``softmax_scale``
    this is the query form (attn_quantize_fp8_q): the scale is folded so that
    q_scale * k_scale * softmax_scale * log2(e) is a power of two.
    With ``hadamard`` the head vectors (last axis) are first rotated by
    Hadamard blocks (attn_quantize_fp8_hadamard): for Q and K only.
    Returns (codes uint8 tensor shaped like x, scale float32 device tensor [1]).
    """
    _need(x, "x")
    if x.dtype == torch.float32:
        xdt = 0
    elif x.dtype == torch.bfloat16:
        xdt = 1
    else:
        raise ValueError("x must be float32 or bfloat16")
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if out is None else out
    scale = torch.empty(1, dtype=torch.float32, device=x.device) if scale is None else scale
    _need(out, "out")
    if hadamard:
        if k_scale is not None:
            _need(k_scale, "k_scale")
            if softmax_scale is None:
                raise ValueError("the folded query scale needs softmax_scale")
        _check("attn_quantize_fp8_hadamard",
               lib().attn_quantize_fp8_hadamard(x.data_ptr(), xdt, x.numel(), x.shape[-1], out.data_ptr(),
                                                scale.data_ptr(), _ptr(k_scale),
                                                float(softmax_scale) if softmax_scale is not None else 0.0,
                                                _stream(stream)))
    elif k_scale is None:
        _check("attn_quantize_fp8",
               lib().attn_quantize_fp8(x.data_ptr(), xdt, x.numel(), out.data_ptr(), scale.data_ptr(),
                                       _stream(stream)))
    else:
        _need(k_scale, "k_scale")
        if softmax_scale is None:
            raise ValueError("the folded query scale needs softmax_scale")
        _check("attn_quantize_fp8_q",
               lib().attn_quantize_fp8_q(x.data_ptr(), xdt, x.numel(), out.data_ptr(), scale.data_ptr(),
                                         k_scale.data_ptr(), float(softmax_scale), _stream(stream)))
    return out, scale


def attn_quantize_fp8_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, softmax_scale: float,
                          out=None, scales: torch.Tensor | None = None, stream=None):
    """The FP8 input step of one attention call in one pass per kind of work
    (attn_quantize_fp8_qkv): K and V with plain scales, Q with the folded one.
    Returns ((q8, k8, v8) uint8 tensors shaped like the inputs, scales float32
    device tensor [3] = {q_scale, k_scale, v_scale})."""
    xs = (q, k, v)
    dts = {t.dtype for t in xs}
    if dts == {torch.float32}:
        xdt = 0
    elif dts == {torch.bfloat16}:
        xdt = 1
    else:
        raise ValueError("q, k, v must all be float32 or all bfloat16")
    for name, t in zip("qkv", xs):
        _need(t, name)
    out = tuple(torch.empty(t.shape, dtype=torch.uint8, device=t.device) for t in xs) if out is None else out
    scales = torch.empty(3, dtype=torch.float32, device=q.device) if scales is None else scales
    for t in (*out, scales):
        _need(t, "output")
    _check("attn_quantize_fp8_qkv",
           lib().attn_quantize_fp8_qkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), xdt, q.numel(), k.numel(),
                                       v.numel(), out[0].data_ptr(), out[1].data_ptr(), out[2].data_ptr(),
                                       scales.data_ptr(), float(softmax_scale), _stream(stream)))
    return out, scales


def attn_cast_bf16(x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """float32 -> bfloat16 (round to nearest even) on the device."""
    _need(x, "x")
    if x.dtype != torch.float32:
        raise ValueError("x must be float32")
    out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device) if out is None else out
    _need(out, "out")
    _check("attn_cast_bf16", lib().attn_cast_bf16(x.data_ptr(), x.numel(), out.data_ptr(), _stream(stream)))
    return out


def _dtype_code(q: torch.Tensor) -> int:
    if q.dtype in (torch.uint8, torch.float8_e4m3fn):
        return ATTN_DTYPE_FP8_E4M3
    if q.dtype == torch.bfloat16:
        return ATTN_DTYPE_BF16
    raise ValueError("q/k/v must be uint8 / float8_e4m3fn codes or bfloat16")


def attn_prefill_fwd(q, k, v, q_scale=1.0, k_scale=1.0, v_scale=1.0, causal=True, out=None, lse=None,
                     return_lse=True, softmax_scale=None, d_scales=None, stream=None):
    """Causal prefill attention forward through the C ABI.

    q [B,S,Hq,d_qk], k [B,S,Hkv,d_qk], v [B,S,Hkv,d_v] device tensors (FP8
    codes as uint8/float8_e4m3fn, or bfloat16). Returns (o bf16 [B,S,Hq,d_v],
    lse fp32 [B,Hq,S] or None). ``d_scales`` (device float32[3]) or an
    explicit ``softmax_scale`` route through attn_prefill_fwd_ex.
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n)
    B, S, Hq, dqk = q.shape
    Hkv, dv = k.shape[2], v.shape[3]
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise ValueError("q, k, v must share one dtype")
    out = torch.empty((B, S, Hq, dv), dtype=torch.bfloat16, device=q.device) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _need(out, "out")
    if lse is not None:
        _need(lse, "lse")
    L = lib()
    if d_scales is None and softmax_scale is None:
        code = L.attn_prefill_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _ptr(lse),
                                  float(q_scale), float(k_scale), float(v_scale),
                                  B, S, Hq, Hkv, dqk, dv, int(bool(causal)), dt, _stream(stream))
        _check("attn_prefill_fwd", code)
    else:
        sm = 1.0 / math.sqrt(dqk) if softmax_scale is None else float(softmax_scale)
        if d_scales is not None:
            _need(d_scales, "d_scales")
            if d_scales.dtype != torch.float32 or d_scales.numel() != 3:
                raise ValueError("d_scales must be float32[3] on the device")
        code = L.attn_prefill_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _ptr(lse),
                                     float(q_scale), float(k_scale), float(v_scale), _ptr(d_scales), sm,
                                     B, S, Hq, Hkv, dqk, dv, int(bool(causal)), dt, _stream(stream))
        _check("attn_prefill_fwd_ex", code)
    return out, lse


def prefill(q32: torch.Tensor, k32: torch.Tensor, v32: torch.Tensor, dtype: str = "fp8", causal=True,
            stream=None, fold_q: bool = True, hadamard: bool = False):
    """The whole path on float32 device inputs: input step, then attention.

    dtype "fp8": per-tensor quantization (scales stay on the device and are
    read by the kernel, so no host synchronisation); with ``fold_q`` the query
    takes the folded scale (see attn_quantize_fp8). With ``hadamard`` (fp8
    only; implies ``fold_q``) Q and K are rotated before the cast.
    "bf16": RNE cast.
    Returns (o, lse, extras) where extras holds the codes and the scale tensor.
    """
    if hadamard and dtype != "fp8":
        raise ValueError("the Hadamard rotation applies to the fp8 path")
    if dtype == "fp8" and fold_q and not hadamard:
        (q8, k8, v8), scales = attn_quantize_fp8_qkv(q32, k32, v32, 1.0 / math.sqrt(q32.shape[-1]), stream=stream)
        o, lse = attn_prefill_fwd(q8, k8, v8, causal=causal, d_scales=scales, stream=stream)
        return o, lse, dict(q=q8, k=k8, v=v8, scales=scales)
    if dtype == "fp8":
        scales = torch.empty(3, dtype=torch.float32, device=q32.device)
        k8, _ = attn_quantize_fp8(k32, scale=scales[1:2], stream=stream, hadamard=hadamard)
        v8, _ = attn_quantize_fp8(v32, scale=scales[2:3], stream=stream)
        if hadamard:
            q8, _ = attn_quantize_fp8(q32, scale=scales[0:1], stream=stream, k_scale=scales[1:2],
                                      softmax_scale=1.0 / math.sqrt(q32.shape[-1]), hadamard=True)
        elif fold_q:
            q8, _ = attn_quantize_fp8(q32, scale=scales[0:1], stream=stream, k_scale=scales[1:2],
                                      softmax_scale=1.0 / math.sqrt(q32.shape[-1]))
        else:
            q8, _ = attn_quantize_fp8(q32, scale=scales[0:1], stream=stream)
        o, lse = attn_prefill_fwd(q8, k8, v8, causal=causal, d_scales=scales, stream=stream)
        return o, lse, dict(q=q8, k=k8, v=v8, scales=scales)
    if dtype == "bf16":
        qb, kb, vb = (attn_cast_bf16(t, stream=stream) for t in (q32, k32, v32))
        o, lse = attn_prefill_fwd(qb, kb, vb, causal=causal, stream=stream)
        return o, lse, dict(q=qb, k=kb, v=vb, scales=None)
    raise ValueError("dtype must be 'fp8' or 'bf16'")
