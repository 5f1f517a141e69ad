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
ATTN_FLAG_P_BLOCK_SCALE = 1
ATTN_FLAG_LEAN_P = 2
ATTN_FLAG_P_ROUNDED_SUM = 4

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
                                     _c_int, _c_void_p]),
    "attn_quantize_fp8": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_void_p, _c_int64, _c_void_p]),
    "attn_quantize_fp8_q": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_void_p, _c_int64, _c_void_p, _c_float,
                                     _c_void_p]),
    "attn_quantize_fp8_hadamard": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_void_p, _c_int64, _c_int, _c_void_p,
                                            _c_float, _c_void_p]),
    "attn_quantize_fp8_qkv": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_int, _c_int64, _c_int64, _c_int64,
                                       _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_float, _c_void_p]),
    "attn_quantize_fp8_qkv_hadamard": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_int, _c_int64, _c_int64,
                                                _c_int64, _c_int, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                                _c_float, _c_void_p]),
    "attn_cast_bf16": (_c_int, [_c_void_p, _c_void_p, _c_int64, _c_void_p]),
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


def _tensor(t, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")


def _need(t: torch.Tensor, name: str, device: torch.device | None = None):
    """A contiguous device tensor (on ``device`` when given)."""
    _tensor(t, name)
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _need_current(t: torch.Tensor, name: str):
    """The library launches on the current device: the tensor must live there."""
    cur = torch.cuda.current_device()
    if t.device.index != cur:
        raise ValueError(f"{name} is on {t.device} but the current device is cuda:{cur}")


_CODE_DTYPES = (torch.uint8, torch.float8_e4m3fn)


def _form(t: torch.Tensor, name: str, numel: int | None = None, shape=None, dtypes=None):
    """Structural check of a buffer: exact shape or element count, and dtype."""
    _tensor(t, name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} must be of dtype {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")


def _x_dtype(x: torch.Tensor, name: str) -> int:
    if x.dtype == torch.float32:
        return 0
    if x.dtype == torch.bfloat16:
        return 1
    raise ValueError(f"{name} must be float32 or bfloat16")


def check_quantize_args(x, out=None, scale=None, k_scale=None, softmax_scale=None, hadamard=False) -> int:
    """Host checks of one single-tensor quantize call; returns the x dtype
    code. Structure (dtype, element counts) is checked before placement (a
    contiguous tensor on x's device), so every mismatch raises ValueError."""
    _tensor(x, "x")
    xdt = _x_dtype(x, "x")
    if x.numel() == 0:
        raise ValueError("x is empty")
    if out is not None:
        _form(out, "out", numel=x.numel(), dtypes=_CODE_DTYPES)
    if scale is not None:
        _form(scale, "scale", numel=1, dtypes=(torch.float32,))
    if k_scale is not None:
        _form(k_scale, "k_scale", numel=1, dtypes=(torch.float32,))
        if softmax_scale is None:
            raise ValueError("the folded query scale needs softmax_scale")
    if hadamard and x.dim() < 1:
        raise ValueError("x must have a head-dim axis")
    _need(x, "x")
    for t, n in ((out, "out"), (scale, "scale"), (k_scale, "k_scale")):
        if t is not None:
            _need(t, n, x.device)
    return xdt


def attn_quantize_fp8(x: torch.Tensor, out: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                      stream=None, k_scale: torch.Tensor | None = None, softmax_scale: float | None = None,
                      hadamard: bool = False):
    """Per-tensor e4m3fn quantization on the device (attn_quantize_fp8).

    With ``k_scale`` (the key tensor's device scale) and ``softmax_scale``
    this is the query form (attn_quantize_fp8_q): the scale is folded so that
    q_scale * k_scale * softmax_scale * log2(e) is a power of two.
    With ``hadamard`` the head vectors (last axis) are first rotated by
    Hadamard blocks (attn_quantize_fp8_hadamard): for Q and K only.
    Returns (codes uint8 tensor shaped like x, scale float32 device tensor [1]).
    """
    xdt = check_quantize_args(x, out, scale, k_scale, softmax_scale, hadamard)
    _need_current(x, "x")
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if out is None else out
    scale = torch.empty(1, dtype=torch.float32, device=x.device) if scale is None else scale
    if hadamard:
        _check("attn_quantize_fp8_hadamard",
               lib().attn_quantize_fp8_hadamard(x.data_ptr(), xdt, out.data_ptr(), scale.data_ptr(), x.numel(),
                                                x.shape[-1], _ptr(k_scale),
                                                float(softmax_scale) if softmax_scale is not None else 0.0,
                                                _stream(stream)))
    elif k_scale is None:
        _check("attn_quantize_fp8",
               lib().attn_quantize_fp8(x.data_ptr(), xdt, out.data_ptr(), scale.data_ptr(), x.numel(),
                                       _stream(stream)))
    else:
        _check("attn_quantize_fp8_q",
               lib().attn_quantize_fp8_q(x.data_ptr(), xdt, out.data_ptr(), scale.data_ptr(), x.numel(),
                                         k_scale.data_ptr(), float(softmax_scale), _stream(stream)))
    return out, scale


def check_quantize_qkv_args(q, k, v, out=None, scales=None) -> int:
    """Host checks of the fused Q/K/V quantize call; returns the x dtype code."""
    xs = (q, k, v)
    for name, t in zip("qkv", xs):
        _tensor(t, name)
        if t.numel() == 0:
            raise ValueError(f"{name} is empty")
    dts = {_x_dtype(t, n) for n, t in zip("qkv", xs)}
    if len(dts) != 1:
        raise ValueError("q, k, v must all be float32 or all bfloat16")
    if out is not None:
        if len(out) != 3:
            raise ValueError("out must be three code tensors (q8, k8, v8)")
        for name, t, x in zip(("q8", "k8", "v8"), out, xs):
            _form(t, name, numel=x.numel(), dtypes=_CODE_DTYPES)
    if scales is not None:
        _form(scales, "scales", numel=3, dtypes=(torch.float32,))
    _need(q, "q")
    for name, t in zip("kv", (k, v)):
        _need(t, name, q.device)
    for name, t in zip(("q8", "k8", "v8", "scales"), (*(out or (None,) * 3), scales)):
        if t is not None:
            _need(t, name, q.device)
    return dts.pop()


def attn_quantize_fp8_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, softmax_scale: float,
                          out=None, scales: torch.Tensor | None = None, stream=None, hadamard: bool = False):
    """The FP8 input step of one attention call in one pass per kind of work
    (attn_quantize_fp8_qkv): K and V with plain scales, Q with the folded one.
    With ``hadamard`` Q and K are rotated first (attn_quantize_fp8_qkv_hadamard;
    the head dim is the last axis of q and k).
    Returns ((q8, k8, v8) uint8 tensors shaped like the inputs, scales float32
    device tensor [3] = {q_scale, k_scale, v_scale})."""
    out = tuple(out) if out is not None else None
    xdt = check_quantize_qkv_args(q, k, v, out, scales)
    if hadamard and (q.dim() < 1 or k.dim() < 1 or q.shape[-1] != k.shape[-1]):
        raise ValueError("the rotation needs q and k with the same head dim (last axis)")
    _need_current(q, "q")
    out = tuple(torch.empty(t.shape, dtype=torch.uint8, device=t.device) for t in (q, k, v)) if out is None else out
    scales = torch.empty(3, dtype=torch.float32, device=q.device) if scales is None else scales
    if hadamard:
        _check("attn_quantize_fp8_qkv_hadamard",
               lib().attn_quantize_fp8_qkv_hadamard(q.data_ptr(), k.data_ptr(), v.data_ptr(), xdt, q.numel(),
                                                    k.numel(), v.numel(), q.shape[-1], out[0].data_ptr(),
                                                    out[1].data_ptr(), out[2].data_ptr(), scales.data_ptr(),
                                                    float(softmax_scale), _stream(stream)))
    else:
        _check("attn_quantize_fp8_qkv",
               lib().attn_quantize_fp8_qkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), xdt, q.numel(), k.numel(),
                                           v.numel(), out[0].data_ptr(), out[1].data_ptr(), out[2].data_ptr(),
                                           scales.data_ptr(), float(softmax_scale), _stream(stream)))
    return out, scales


def attn_cast_bf16(x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """float32 -> bfloat16 (round to nearest even) on the device (attn_cast_bf16)."""
    _tensor(x, "x")
    if x.dtype != torch.float32:
        raise ValueError("x must be float32")
    if x.numel() == 0:
        raise ValueError("x is empty")
    if out is not None:
        _form(out, "out", numel=x.numel(), dtypes=(torch.bfloat16,))
    _need(x, "x")
    if out is not None:
        _need(out, "out", x.device)
    _need_current(x, "x")
    out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device) if out is None else out
    _check("attn_cast_bf16", lib().attn_cast_bf16(x.data_ptr(), out.data_ptr(), x.numel(), _stream(stream)))
    return out


def _dtype_code(q: torch.Tensor) -> int:
    if q.dtype in _CODE_DTYPES:
        return ATTN_DTYPE_FP8_E4M3
    if q.dtype == torch.bfloat16:
        return ATTN_DTYPE_BF16
    raise ValueError("q/k/v must be uint8 / float8_e4m3fn codes or bfloat16")


def check_attention_args(q, k, v, out=None, lse=None, d_scales=None):
    """Shape, dtype and device checks of one attention call (host only).

    Returns (B, S, Hq, Hkv, d_qk, d_v, dtype code). Raises ValueError on any
    mismatch: the kernels trust these sizes, so a short k, a narrow v or an
    undersized out / lse would be read or written out of bounds. Structure
    is checked before placement (contiguous tensors on q's device).
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _tensor(t, n)
        if t.dim() != 4:
            raise ValueError(f"{n} must be 4-D [B, S, H, d], got shape {tuple(t.shape)}")
    B, S, Hq, dqk = q.shape
    Hkv, dv = k.shape[2], v.shape[3]
    if tuple(k.shape) != (B, S, Hkv, dqk):
        raise ValueError(f"k must have shape {(B, S, Hkv, dqk)} (q's B, S and d_qk), got {tuple(k.shape)}")
    if tuple(v.shape[:3]) != (B, S, Hkv):
        raise ValueError(f"v must have shape {(B, S, Hkv)} + (d_v,), got {tuple(v.shape)}")
    if min(B, S, Hq, Hkv, dqk, dv) == 0:
        raise ValueError("empty attention input")
    if Hq % Hkv != 0:
        raise ValueError(f"Hq ({Hq}) must be a multiple of Hkv ({Hkv})")
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise ValueError("q, k, v must share one dtype")
    if out is not None:
        _form(out, "out", shape=(B, S, Hq, dv), dtypes=(torch.bfloat16,))
    if lse is not None:
        _form(lse, "lse", shape=(B, Hq, S), dtypes=(torch.float32,))
    if d_scales is not None:
        _form(d_scales, "d_scales", numel=3, dtypes=(torch.float32,))
    _need(q, "q")
    for t, n in ((k, "k"), (v, "v"), (out, "out"), (lse, "lse"), (d_scales, "d_scales")):
        if t is not None:
            _need(t, n, q.device)
    return B, S, Hq, Hkv, dqk, dv, dt


def attn_prefill_fwd(q, k, v, q_scale=1.0, k_scale=1.0, v_scale=1.0, causal=True, out=None, lse=None,
                     return_lse=True, softmax_scale=None, d_scales=None, stream=None, flags: int = 0):
    """Causal prefill attention forward through the C ABI (attn_prefill_fwd,
    or attn_prefill_fwd_ex when ``d_scales``, ``softmax_scale`` or ``flags``
    is given; ``flags``: ATTN_FLAG_* bits).

    q [B,S,Hq,d_qk], k [B,S,Hkv,d_qk], v [B,S,Hkv,d_v] device tensors (FP8
    codes as uint8/float8_e4m3fn, or bfloat16). Returns (o bf16 [B,S,Hq,d_v],
    lse fp32 [B,Hq,S] or None). ``d_scales`` is a device float32[3]
    {q_scale, k_scale, v_scale}; ``out`` / ``lse`` are optional preallocated
    outputs.
    """
    B, S, Hq, Hkv, dqk, dv, dt = check_attention_args(q, k, v, out, lse, d_scales)
    _need_current(q, "q")
    out = torch.empty((B, S, Hq, dv), dtype=torch.bfloat16, device=q.device) if out is None else out
    if flags & ATTN_FLAG_LEAN_P:
        if lse is not None:
            raise ValueError("Lean P computes O only: pass lse=None")
        return_lse = False
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    L = lib()
    if d_scales is None and softmax_scale is None and not flags:
        code = L.attn_prefill_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _ptr(lse),
                                  float(q_scale), float(k_scale), float(v_scale),
                                  B, S, Hq, Hkv, dqk, dv, int(bool(causal)), dt, _stream(stream))
        _check("attn_prefill_fwd", code)
    else:
        sm = 1.0 / math.sqrt(dqk) if softmax_scale is None else float(softmax_scale)
        code = L.attn_prefill_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _ptr(lse),
                                     float(q_scale), float(k_scale), float(v_scale), _ptr(d_scales), sm,
                                     B, S, Hq, Hkv, dqk, dv, int(bool(causal)), dt, int(flags), _stream(stream))
        _check("attn_prefill_fwd_ex", code)
    return out, lse


def attn_prefill(q, k, v, q_scale=1.0, k_scale=1.0, v_scale=1.0, causal=True):
    """The boundary's Python form: attention on FP8 codes (with their
    per-tensor scales) or BF16 inputs, softmax scale 1/sqrt(d_qk).
    Allocates and returns (o bf16 [B,S,Hq,d_v], lse fp32 [B,Hq,S]); runs on
    the current stream."""
    return attn_prefill_fwd(q, k, v, q_scale, k_scale, v_scale, causal=causal)


def prefill(q32: torch.Tensor, k32: torch.Tensor, v32: torch.Tensor, dtype: str = "fp8", causal=True,
            stream=None, fold_q: bool = True, hadamard: bool | None = None, flags: int = 0):
    """The whole path on float32 device inputs: input step, then attention.

    dtype "fp8": per-tensor quantization (scales stay on the device and are
    read by the kernel, so no host synchronisation). By default Q and K are
    rotated by Hadamard blocks before the cast and the query takes the folded
    scale (attn_quantize_fp8_qkv_hadamard): on heavy-tailed activations the
    rotation spreads outlier channels over the head dim, which keeps the FP8
    matrix core's summing error on a row's largest scores, and so the LSE,
    within its bar (aicronaca.it, "Perché l'FP8 non basta da solo"). With
    ``hadamard=False`` the unrotated tensors are quantized, with the folded
    query scale when ``fold_q``; ``fold_q=False`` gives the plain per-tensor
    absmax scales, unrotated (the rotated step always folds the query scale).
    "bf16": RNE cast. ``flags`` (ATTN_FLAG_* bits) go to the attention call.
    Returns (o, lse, extras) where extras holds the codes and the scale tensor.
    """
    if hadamard is None:
        hadamard = dtype == "fp8" and fold_q
    if hadamard and dtype != "fp8":
        raise ValueError("the Hadamard rotation applies to the fp8 path")
    if hadamard and not fold_q:
        raise ValueError("the rotated input step folds the query scale: hadamard needs fold_q")
    if dtype == "fp8" and (fold_q or hadamard):
        (q8, k8, v8), scales = attn_quantize_fp8_qkv(q32, k32, v32, 1.0 / math.sqrt(q32.shape[-1]), stream=stream,
                                                     hadamard=hadamard)
        o, lse = attn_prefill_fwd(q8, k8, v8, causal=causal, d_scales=scales, stream=stream, flags=flags)
        return o, lse, dict(q=q8, k=k8, v=v8, scales=scales)
    if dtype == "fp8":
        scales = torch.empty(3, dtype=torch.float32, device=q32.device)
        k8, _ = attn_quantize_fp8(k32, scale=scales[1:2], stream=stream)
        v8, _ = attn_quantize_fp8(v32, scale=scales[2:3], stream=stream)
        q8, _ = attn_quantize_fp8(q32, scale=scales[0:1], stream=stream)
        o, lse = attn_prefill_fwd(q8, k8, v8, causal=causal, d_scales=scales, stream=stream, flags=flags)
        return o, lse, dict(q=q8, k=k8, v=v8, scales=scales)
    if dtype == "bf16":
        qb, kb, vb = (attn_cast_bf16(t, stream=stream) for t in (q32, k32, v32))
        o, lse = attn_prefill_fwd(qb, kb, vb, causal=causal, stream=stream, flags=flags)
        return o, lse, dict(q=qb, k=kb, v=vb, scales=None)
    raise ValueError("dtype must be 'fp8' or 'bf16'")
