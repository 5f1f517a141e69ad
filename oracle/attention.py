"""Exact causal softmax attention in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What is computed (the causal forward/prefill attention pass of the pages:
Le Fil IA summary paragraph; aicronaca.it "Che cosa ha annunciato Zyphra";
ai4bro.com "TL;DR"). The pages describe the tiled method -- Q.K^T, a row
softmax, P.V -- whose exact result is plain softmax attention, so the oracle is
that definition written out, with no tiling and no online rescaling:

    for batch b, query head h, kv head g = floor(h / G), G = Hq / Hkv:
      s[i, j]  = softmax_scale * dot(Q[b, i, h, :], K[b, j, g, :])   for j <= i
      m[i]     = max_j s[i, j]
      l[i]     = sum_j exp(s[i, j] - m[i])
      O[b,i,h] = sum_j exp(s[i, j] - m[i]) * V[b, j, g, :] / l[i]
      LSE[b,h,i] = m[i] + ln l[i]

Readings where the pages are silent (each listed in the design notes):

* tensor layout is that of ``flash_attn_func`` (the pages call the library a
  drop-in for it): q [B,S,Hq,d_qk], k [B,S,Hkv,d_qk], v [B,S,Hkv,d_v];
* grouped-query heads map contiguously, kv head = floor(h / G);
* the softmax scale is 1/sqrt(d_qk) (1/sqrt(192) for the MLA shape);
* causal alignment is square (S_q = S_k): key j is visible to query i iff
  j <= i, so no row is empty;
* LSE is the natural logarithm and includes every scale.

Subtracting the row maximum is an exact identity (it cancels between the
numerator and l); it only keeps exp() in range.
"""

from __future__ import annotations

import math

import numpy as np

from .rotation import hadamard_encode, hadamard_scales
from .formats import (bf16_decode, bf16_encode, dequantize_fp8, encode_with_scale, per_tensor_scale,
                      per_tensor_scale_folded)


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, S, H, d]")
    B, S, Hq, dqk = q.shape
    if k.shape[:2] != (B, S) or v.shape[:2] != (B, S):
        raise ValueError("q, k, v must share B and S")
    Hkv = k.shape[2]
    if v.shape[2] != Hkv or k.shape[3] != dqk:
        raise ValueError("k/v head count or k head dim mismatch")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, S, Hq, Hkv, dqk, v.shape[3]


def _rows_softmax_attention(qrows, K, V, ends, scale):
    """Exact attention for a set of query rows against keys [0, end_r).

    qrows [R, d_qk]; K [S, d_qk]; V [S, d_v]; ends[r] = number of visible keys.
    Returns (O [R, d_v], LSE [R]) in float64.
    """
    R = qrows.shape[0]
    n = int(max(ends)) if R else 0
    s = (qrows @ K[:n].T) * scale  # [R, n]
    visible = np.arange(n)[None, :] < np.asarray(ends)[:, None]
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])  # exp(-inf) = 0 for hidden keys
    l = p.sum(axis=1)
    o = (p @ V[:n]) / l[:, None]
    return o, m + np.log(l)


def causal_attention(q, k, v, causal: bool = True, softmax_scale: float | None = None,
                     row_block: int = 512):
    """Softmax attention of float64 tensors in the flash_attn_func layout.

    Returns (O [B,S,Hq,d_v] float64, LSE [B,Hq,S] float64). Rows are processed
    ``row_block`` at a time only to bound memory; each row is computed by the
    definition above.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, S, Hq, Hkv, dqk, dv = _check_shapes(q, k, v)
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(dqk) if softmax_scale is None else float(softmax_scale)
    O = np.zeros((B, S, Hq, dv), dtype=np.float64)
    L = np.zeros((B, Hq, S), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            K = np.ascontiguousarray(k[b, :, g, :])
            V = np.ascontiguousarray(v[b, :, g, :])
            for i0 in range(0, S, row_block):
                i1 = min(S, i0 + row_block)
                rows = np.arange(i0, i1)
                ends = rows + 1 if causal else np.full(i1 - i0, S)
                o, lse = _rows_softmax_attention(q[b, i0:i1, h, :], K, V, ends, scale)
                O[b, i0:i1, h, :] = o
                L[b, h, i0:i1] = lse
    return O, L


def attention_rows(q, k, v, rows, causal: bool = True, softmax_scale: float | None = None):
    """Exact attention for selected (b, h, i) rows only.

    ``q``, ``k``, ``v`` may be any array-likes indexable as [b, :, h, :]
    (for example the dequantizing views made by ``prefill_reference``);
    only the heads the rows touch are materialised in float64.
    Returns (O [R, d_v], LSE [R]).
    """
    Hq = q.shape[2]
    Hkv = k.shape[2]
    S = q.shape[1]
    G = Hq // Hkv
    dqk = q.shape[3]
    scale = 1.0 / math.sqrt(dqk) if softmax_scale is None else float(softmax_scale)
    rows = [tuple(int(t) for t in r) for r in rows]
    outs = [None] * len(rows)
    lses = np.zeros(len(rows))
    by_head: dict[tuple[int, int], list[int]] = {}
    for idx, (b, h, i) in enumerate(rows):
        by_head.setdefault((b, h), []).append(idx)
    for (b, h), idxs in by_head.items():
        g = h // G
        K = np.asarray(k[b, :, g, :], dtype=np.float64)
        V = np.asarray(v[b, :, g, :], dtype=np.float64)
        Q = np.asarray(q[b, :, h, :], dtype=np.float64)
        ii = np.array([rows[t][2] for t in idxs])
        ends = ii + 1 if causal else np.full(len(ii), S)
        o, lse = _rows_softmax_attention(Q[ii], K, V, ends, scale)
        for t, idx in enumerate(idxs):
            outs[idx] = o[t]
            lses[idx] = lse[t]
    return np.stack(outs), lses


class _QuantizedView:
    """Array-like view of a float32 tensor after the input step.

    Indexing returns the dequantized float64 values of the selected elements:
    fp8 -> decode(e4m3fn(x / scale)) * scale with the per-tensor scale of the
    WHOLE tensor; bf16 -> the bf16-rounded values. Only the requested slice is
    encoded, so rows of very long sequences stay cheap.
    """

    def __init__(self, x32, kind, scale=None):
        self.x32 = np.asarray(x32, dtype=np.float32)
        self.kind = kind
        self.shape = self.x32.shape
        if kind != "fp8":
            self.scale = np.float32(1.0)
        else:
            self.scale = per_tensor_scale(self.x32) if scale is None else np.float32(scale)

    def codes(self, idx=slice(None)):
        if self.kind == "fp8":
            return encode_with_scale(self.x32[idx], self.scale)
        return bf16_encode(self.x32[idx])

    def __getitem__(self, idx):
        c = self.codes(idx)
        if self.kind == "fp8":
            return dequantize_fp8(c, self.scale)
        return bf16_decode(c)


class _RotatedView(_QuantizedView):
    """As _QuantizedView for a Hadamard-rotated FP8 tensor (oracle/rotation.py).

    Codes come from the rotated rows with the code scale; indexing returns
    decode(code) * stored scale. Indices must keep the last axis whole (rows
    are rotated one head vector at a time).
    """

    def __init__(self, x32, code_scale, stored_scale):
        self.x32 = np.asarray(x32, dtype=np.float32)
        self.kind = "fp8"
        self.shape = self.x32.shape
        self.code_scale = np.float32(code_scale)
        self.scale = np.float32(stored_scale)

    def codes(self, idx=slice(None)):
        return hadamard_encode(self.x32[idx], self.code_scale)


def prefill_reference(q32, k32, v32, dtype: str, causal: bool = True, rows=None,
                      softmax_scale: float | None = None, fold_q: bool = False, hadamard: bool = False):
    """The whole path on float32 inputs: the input step, then attention.

    dtype "fp8": per-tensor absmax e4m3fn codes and scales (with ``fold_q``
    the query takes the folded scale for the key scale and softmax scale);
    "bf16": bf16 RNE.
    With ``hadamard`` (fp8 only, implies ``fold_q``) Q and K are rotated
    before quantization (oracle/rotation.py); the key keeps its plain scale
    and the query's stored scale is its folded scale over the block size.
    Attention runs in float64 on the dequantized values. Without ``rows``:
    returns the codes (uint8 for fp8, uint16 bit patterns for bf16), the
    scales (1.0 for bf16) and the full O / LSE. With ``rows`` (a list of
    (b, h, i)): only those rows are computed (o_rows, lse_rows), together with
    the scales; codes are then available per slice through ``views``.
    """
    if dtype not in ("fp8", "bf16"):
        raise ValueError("dtype must be 'fp8' or 'bf16'")
    sm = 1.0 / math.sqrt(np.shape(q32)[-1]) if softmax_scale is None else softmax_scale
    if hadamard:
        if dtype != "fp8":
            raise ValueError("the Hadamard rotation applies to the fp8 path")
        kcs, ks = hadamard_scales(k32)
        qcs, qs = hadamard_scales(q32, k_scale=ks, softmax_scale=sm)
        views = [_RotatedView(q32, qcs, qs), _RotatedView(k32, kcs, ks), _QuantizedView(v32, dtype)]
    else:
        kv = [_QuantizedView(t, dtype) for t in (k32, v32)]
        q_scale = None
        if dtype == "fp8" and fold_q:
            q_scale = per_tensor_scale_folded(q32, kv[0].scale, sm)
        views = [_QuantizedView(q32, dtype, q_scale)] + kv
    out = dict(q_scale=views[0].scale, k_scale=views[1].scale, v_scale=views[2].scale, views=views)
    if rows is None:
        qc, kc, vc = (vw.codes() for vw in views)
        out.update(q_codes=qc, k_codes=kc, v_codes=vc)
        if dtype == "fp8":
            qd, kd, vd = (dequantize_fp8(c, vw.scale) for c, vw in zip((qc, kc, vc), views))
        else:
            qd, kd, vd = (bf16_decode(c) for c in (qc, kc, vc))
        O, L = causal_attention(qd, kd, vd, causal=causal, softmax_scale=softmax_scale)
        out.update(o=O, lse=L)
    else:
        O, L = attention_rows(*views, rows=rows, causal=causal, softmax_scale=softmax_scale)
        out.update(o_rows=O, lse_rows=L)
    return out
