"""Number formats of the attention inputs, written from their definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

FP8 is OCP e4m3fn, the 8-bit format the pages name ("FP8 e4m3": ai4bro.com,
"TL;DR"; Le Fil IA, context paragraph). Its definition:

* bit 7 sign, bits 6..3 exponent field E (bias 7), bits 2..0 mantissa M;
* E = 0: subnormal, value M/8 * 2^-6;
* E > 0: value (1 + M/8) * 2^(E-7);
* S.1111.111 is NaN; there are no infinities, so the largest finite
  magnitude is 1.75 * 2^8 = 448 (code 0x7E).

The pages' one fact about the codes (Le Fil IA, context paragraph;
aicronaca.it, "Perché l'FP8 non basta da solo"): read as an integer, a
positive code grows by 8 each time the value doubles. That holds for every
normal value because the exponent field starts at bit 3.

Quantization (not specified by the pages; the reading used here): one fp32
scale per tensor, scale = absmax / 448 computed in fp32, and code = the e4m3fn
value nearest to x / scale (the division in fp32, correctly rounded), ties to
the even code. A tensor of zeros gets scale 1. The dequantized value is
decode(code) * scale, exact in float64.

Folded query scale (a reading of the quantize step, also not on the pages):
a query tensor may take, instead of absmax / 448, the smallest scale of the
form 2^j / (k_scale * softmax_scale * log2 e), j an integer, that is at least
absmax / 448. It is evaluated in float64 with each operation correctly
rounded -- g = (k_scale * softmax_scale) * log2e, t = (absmax / 448) * g,
j = ceil(log2 t) exactly, scale = 2^j / g -- and rounded once to fp32; a
tensor of zeros gets scale 1. It is then at most twice absmax / 448, codes
are formed as above, and q_scale * k_scale * softmax_scale * log2 e is a
power of two.

bfloat16 is the top 16 bits of an IEEE binary32: 1 sign, 8 exponent, 7
mantissa bits. Encoding from fp32 rounds to the nearest bfloat16, ties to the
even mantissa.
"""

from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
# log2(e) rounded to float64
LOG2E = 1.4426950408889634


def e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each e4m3fn code as float64 (NaN for the two NaN codes)."""
    c = np.asarray(codes).astype(np.int64)
    if np.any((c < 0) | (c > 255)):
        raise ValueError("e4m3fn codes are bytes")
    sign = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = (m / 8.0) * 2.0**-6
    nrm = (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64))
    mag = np.where(e == 0, sub, nrm)
    val = np.where(sign == 1, -mag, mag)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return val.astype(np.float64)


# The 127 non-negative finite e4m3fn values, indexed by their code 0x00..0x7E.
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = e4m3fn_decode(_POS_CODES)
# Midpoints between neighbouring values (exact in float64: dyadic, few bits).
_MIDPOINTS = (_POS_VALUES[:-1] + _POS_VALUES[1:]) / 2.0


def e4m3fn_encode(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest e4m3fn code, ties to even.

    Magnitudes in (448, 464] round to 448 (464 is the tie point between 448
    and the next step, 480, which the format does not have; the even code
    0x7E wins). Larger magnitudes and non-finite inputs are outside this
    oracle's contract and raise ``ValueError``. The sign bit is kept on
    values that round to zero (-0 encodes as 0x80).
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x.astype(np.float64))
    if not np.all(np.isfinite(a)) or np.any(a > 464.0):
        raise ValueError("e4m3fn_encode: input outside [-464, 464]")
    a = np.minimum(a, E4M3_MAX)
    # lower neighbour index i: values[i] <= a < values[i+1]
    i = np.searchsorted(_POS_VALUES, a, side="right") - 1
    i = np.clip(i, 0, len(_POS_VALUES) - 1)
    top = i == len(_POS_VALUES) - 1
    ii = np.where(top, i - 1, i)
    mid = _MIDPOINTS[ii]
    up = np.where(a > mid, True, np.where(a < mid, False, (ii % 2) == 1))
    code = np.where(top, i, np.where(up, ii + 1, ii))
    signbit = np.signbit(x)
    code = code | np.where(signbit, 0x80, 0)
    return code.astype(np.uint8)


def quantize_fp8_per_tensor(x: np.ndarray) -> tuple[np.ndarray, np.float32]:
    """Per-tensor absmax quantization of a float32 tensor to e4m3fn codes.

    Returns (codes uint8 with the shape of x, scale float32) with
    x ~= decode(codes) * scale.
    """
    x = np.asarray(x, dtype=np.float32)
    scale = per_tensor_scale(x)
    return encode_with_scale(x, scale), scale


def per_tensor_scale(x: np.ndarray) -> np.float32:
    """absmax(|x|) / 448 in fp32 (1.0 for an all-zero tensor)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / np.float32(E4M3_MAX))


def per_tensor_scale_folded(x: np.ndarray, k_scale, softmax_scale) -> np.float32:
    """The folded query scale: smallest 2^j / (k_scale*softmax_scale*log2 e) >= absmax/448."""
    x = np.asarray(x, dtype=np.float32)
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    if amax == 0.0:
        return np.float32(1.0)
    g = float(np.float64(np.float32(k_scale)) * np.float64(np.float32(softmax_scale))) * LOG2E
    t = (amax / E4M3_MAX) * g
    f, e = math.frexp(t)  # t = f * 2^e, 0.5 <= f < 1
    j = e - 1 if f == 0.5 else e
    return np.float32(math.ldexp(1.0, j) / g)


def encode_with_scale(x: np.ndarray, scale) -> np.ndarray:
    """e4m3fn codes of x / scale (fp32 division, then round to nearest even)."""
    x = np.asarray(x, dtype=np.float32)
    y = (x / np.float32(scale)).astype(np.float32)
    return e4m3fn_encode(y)


def dequantize_fp8(codes: np.ndarray, scale) -> np.ndarray:
    """decode(code) * scale in float64 (exact: both factors are dyadic)."""
    return e4m3fn_decode(codes) * np.float64(np.float32(scale))


def bf16_encode(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (returned as uint16 bit patterns).

    Nearest bfloat16 value, ties to the even mantissa; finite inputs only
    (inputs whose rounding would overflow are outside the contract).
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16_encode: finite inputs only")
    bits = x.view(np.uint32).astype(np.uint64)
    low = bits & 0xFFFF
    trunc = bits >> 16  # rounds the magnitude toward zero
    half = 0x8000
    odd = trunc & 1
    up = (low > half) | ((low == half) & (odd == 1))
    out = trunc + up.astype(np.uint64)
    if np.any((out & 0x7F80) == 0x7F80):
        raise ValueError("bf16_encode: rounding overflowed")
    return out.astype(np.uint16)


def bf16_decode(u: np.ndarray) -> np.ndarray:
    """Value of each bfloat16 bit pattern as float64."""
    u = np.ascontiguousarray(np.asarray(u, dtype=np.uint16))
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
