"""Hadamard rotation of Q and K ahead of the FP8 quantization.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path imports this module.

Source: aicronaca.it, section "Perché l'FP8 non basta da solo". Rotating Q
and K by a Hadamard matrix before the FP8 cast roughly halves the input
quantization error. It costs about 0.1 % of the attention time on a
Mistral-7B layer. The page gives no construction, block size or scale
convention. The readings taken here:

* Sylvester Hadamard matrices, unnormalized: H_1 = [1] and
  H_2m = [[H_m, H_m], [H_m, -H_m]]. Entries are +-1 and H_m H_m^T = m I.
  Entry (i, j) is (-1)^popcount(i & j).
* Block size b = the largest power of two dividing the head dim, capped at
  128: d = 128 gives one 128 block; d = 192 (the MLA query/key dim) gives three
  64 blocks (dims 0-63, 64-127, 128-191). Each head vector x (one row of the
  last axis) becomes y = x H_b blockwise. Then (q H)(k H)^T = b q.k^T, so the
  scores change only by the factor b, which the query's scale absorbs.
* The rotated values are formed in float64. They are the exact sums up to
  float64 rounding, so both sides take the code decision in the same
  precision. Their absmax is rounded once to float32. The per-tensor scale
  follows the unrotated quantizer's rule on that absmax: plain absmax/448 for
  a key, or the folded query scale. Codes are e4m3fn(fp32(y * r)) with
  r = fp64(1 / scale): the reciprocal and the product are each rounded once
  in float64, then the product is rounded to float32 and to e4m3 with ties
  to even. One multiply per element replaces a division.
* The query's stored scale is that scale divided by b. The division is exact
  because b is a power of two. code * stored_scale then dequantizes to y_q / b,
  and dequantized Q.K^T products equal the unrotated q.k^T up to the
  quantization error. The key keeps its plain scale.
* V is not rotated: rotating it would need an inverse rotation of O.
* Only the FP8 path is rotated: the page ties the rotation to the FP8 input
  error.
"""

from __future__ import annotations

import numpy as np

from .formats import e4m3fn_encode, per_tensor_scale, per_tensor_scale_folded


def sylvester_hadamard(m: int) -> np.ndarray:
    """Unnormalized Sylvester Hadamard matrix of order m (a power of two), int64."""
    if m < 1 or m & (m - 1):
        raise ValueError("order must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < m:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_block(d: int) -> int:
    """Block size for head dim d: largest power of two dividing d, at most 128."""
    if d < 1:
        raise ValueError("head dim must be positive")
    return min(d & -d, 128)


def rotate_rows(x: np.ndarray) -> np.ndarray:
    """y = x H_b on each b-wide block of the last axis, in float64."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    b = hadamard_block(d)
    h = sylvester_hadamard(b).astype(np.float64)
    blocks = x.reshape(x.shape[:-1] + (d // b, b))
    return (blocks @ h).reshape(x.shape)


def rotated_absmax(x: np.ndarray, chunk_rows: int = 1 << 16) -> np.float32:
    """max |x H| over the tensor, rounded once to float32 (chunked over rows)."""
    x = np.asarray(x)
    d = x.shape[-1]
    flat = x.reshape(-1, d)
    m = 0.0
    for r0 in range(0, flat.shape[0], chunk_rows):
        y = rotate_rows(flat[r0:r0 + chunk_rows])
        if y.size:
            m = max(m, float(np.max(np.abs(y))))
    return np.float32(m)


def _scale_from_absmax(a: np.float32, k_scale=None, softmax_scale=None) -> np.float32:
    """The unrotated quantizer's scale rules applied to the absmax a (float32).

    A one-element tensor holding a has absmax a, so the plain and folded scale
    functions of the unrotated quantizer give the scales directly.
    """
    one = np.array([a], dtype=np.float32)
    if k_scale is None:
        return per_tensor_scale(one)
    return per_tensor_scale_folded(one, k_scale, softmax_scale)


def hadamard_scales(x: np.ndarray, k_scale=None, softmax_scale=None):
    """(scale the codes are taken with, scale stored for dequantization).

    Key (k_scale None): both are the plain scale of the rotated tensor.
    Query (k_scale and softmax_scale given): the codes use the folded scale;
    the stored scale is that divided by the block size b.
    """
    a = rotated_absmax(x)
    s = _scale_from_absmax(a, k_scale, softmax_scale)
    if k_scale is None:
        return s, s
    b = hadamard_block(np.shape(x)[-1])
    return s, np.float32(float(s) / b)


def hadamard_encode(x: np.ndarray, code_scale) -> np.ndarray:
    """e4m3fn codes of fp32(y * fp64(1 / code_scale)) for the rotated rows y of x."""
    y = rotate_rows(x)
    r = 1.0 / float(np.float32(code_scale))
    return e4m3fn_encode((y * np.float64(r)).astype(np.float32))


def hadamard_quantize(x: np.ndarray, k_scale=None, softmax_scale=None):
    """Rotate, then quantize per tensor: returns (codes uint8, stored scale)."""
    code_scale, stored = hadamard_scales(x, k_scale, softmax_scale)
    return hadamard_encode(x, code_scale), stored
