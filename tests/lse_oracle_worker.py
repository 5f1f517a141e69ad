"""Per-head oracle work for tests/test_gpu_lse_full_tensor.py, run in worker
processes (numpy and oracle/ only: no torch, no device).

For one (query head, kv head) pair of float32 inputs, with the per-tensor
scales the oracle chose for the whole tensors, it returns the oracle's e4m3
codes of both head slices, the oracle's log-sum-exp of every query row, and a
bound on how far an FP8 matrix core that sums each 64-product block to 2^-14
of its largest terms can move each row's log-sum-exp: 2^-13 (twice that) times
the softmax scale times the largest sum of absolute products over the keys
the row sees.
"""

import math

import numpy as np

from oracle.attention import causal_attention
from oracle.formats import dequantize_fp8, encode_with_scale
from oracle.rotation import hadamard_encode


def head_lse(args):
    q32, k32, rotated, q_code_scale, q_scale, k_code_scale, k_scale, causal = args
    if rotated:
        qc = hadamard_encode(q32, q_code_scale)
        kc = hadamard_encode(k32, k_code_scale)
    else:
        qc = encode_with_scale(q32, q_code_scale)
        kc = encode_with_scale(k32, k_code_scale)
    qd = dequantize_fp8(qc, q_scale)
    kd = dequantize_fp8(kc, k_scale)
    S, d = qd.shape
    _, lse = causal_attention(qd[None, :, None, :], kd[None, :, None, :], np.zeros((1, S, 1, 1)), causal=causal)
    # largest sum of |q_d k_d| over the visible keys of each row
    aq, ak = np.abs(qd), np.abs(kd)
    worst = np.empty(S)
    for i0 in range(0, S, 1024):
        i1 = min(S, i0 + 1024)
        n = i1 if causal else S
        a = aq[i0:i1] @ ak[:n].T
        if causal:
            a = np.where(np.arange(n)[None, :] <= np.arange(i0, i1)[:, None], a, 0.0)
        worst[i0:i1] = a.max(axis=1)
    bound = 2.0 ** -11 * worst / math.sqrt(d)
    return qc, kc, lse[0, 0], bound
