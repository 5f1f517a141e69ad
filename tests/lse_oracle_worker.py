"""Per-head oracle work for tests/test_gpu_lse_full_tensor.py, run in worker
processes (numpy and oracle/ only: no torch, no device).

For one (query head, kv head) pair of float32 inputs, with the per-tensor
scales the oracle chose for the whole tensors, it returns the oracle's e4m3
codes of the head slices, the oracle's log-sum-exp of every query row, and a
bound on how far the FP8 matrix core's summing error (within 2^-11 of the sum
of |products| of a dot product, pinned in test_gpu_mfma_precision) can move
each row's log-sum-exp: 2^-11 times the softmax scale times the largest sum
of absolute products over the keys the row sees. Given V and the GPU's O for
the head, it also returns the oracle's O error of every row (relative L2)
and the two sums of the whole-tensor relative L2.
"""

import math

import numpy as np

from oracle.attention import causal_attention
from oracle.formats import dequantize_fp8, encode_with_scale
from oracle.rotation import hadamard_encode


def head_lse(args):
    q32, k32, rotated, q_code_scale, q_scale, k_code_scale, k_scale, causal, v32, v_scale, o_gpu = args
    if rotated:
        qc = hadamard_encode(q32, q_code_scale)
        kc = hadamard_encode(k32, k_code_scale)
    else:
        qc = encode_with_scale(q32, q_code_scale)
        kc = encode_with_scale(k32, k_code_scale)
    qd = dequantize_fp8(qc, q_scale)
    kd = dequantize_fp8(kc, k_scale)
    S, d = qd.shape
    vc = None
    if v32 is None:
        vd = np.zeros((S, 1))
    else:
        vc = encode_with_scale(v32, v_scale)
        vd = dequantize_fp8(vc, v_scale)
    o, lse = causal_attention(qd[None, :, None, :], kd[None, :, None, :], vd[None, :, None, :], causal=causal)
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
    out = dict(q_codes=qc, k_codes=kc, v_codes=vc, lse=lse[0, 0], bound=bound)
    if o_gpu is not None:
        ref = o[0, :, 0, :]
        diff = np.asarray(o_gpu, dtype=np.float64) - ref
        out["o_row_err"] = np.linalg.norm(diff, axis=1) / np.linalg.norm(ref, axis=1)
        out["o_sums"] = (float(np.sum(diff * diff)), float(np.sum(ref * ref)))
    return out
