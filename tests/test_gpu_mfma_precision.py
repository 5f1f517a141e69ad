"""How exactly the FP8 matrix core sums a Q.K dot product, read through the
attention kernel itself.

With one key per row (S = 1) the softmax has a single term: p = 1, l = 1,
and the kernel's LSE is ln 2 * t, where t is the row's score in log2 units as
the scaled FP8 MFMA hands it over. Codes are passed directly (no input step)
with q_scale = k_scale = 1 and softmax_scale = fp32(ln 2), so the score factor
q_scale * k_scale * softmax_scale * log2(e) rounds to 1 and the kernel takes
its folded form with an operand scale of 2^0: t is the MFMA's sum of the
e4m3 products, chained over the 64-deep contraction steps in fp32. Every
product of two e4m3 values is exact in fp32, so a correctly rounded fp32
accumulation would be off by at most a few units of 2^-24 of the sum of the
absolute products. The test measures the actual error against the exact
(fp64) dot product of the same codes, for Gaussian operands, for operands
where one product (448 * 448) dominates, and for operands shaped like the
heavy-tailed layer's rows whose Q and K outlier channels meet: four x8
channels in both.

What it pins, for the LSE error of the heavy-tailed layer: the matrix core
does not accumulate in full fp32 (errors far above the few units of 2^-24 an
fp32 sum would leave; measured 2^-16.7 of the sum of |products| for Gaussian
operands, 2^-14.1 with one dominant product and about 2^-12 with four large
products), and the error stays within 2^-11 of that sum. With logits of
50-80 on such rows, that moves a row's largest score, and with it the LSE,
by up to about 2e-2 (test_gpu_lse_full_tensor); the input step's Hadamard
rotation spreads the outlier channels over every column and removes it.
"""

import math

import numpy as np
import pytest
import torch

from bf16_causal_prefill_fwd_amd import ops
from oracle import e4m3fn_decode, e4m3fn_encode

pytestmark = pytest.mark.gpu

LN2_F32 = float(np.float32(math.log(2.0)))


def _codes(rng, shape, scale):
    return e4m3fn_encode(np.float32(rng.standard_normal(shape) * scale))


def _case(d_qk: int, kind: str, seed: int, H: int = 2048):
    rng = np.random.default_rng(seed)
    if kind == "outliers":
        # four channels per head x8 in both q and k (clipped to the e4m3 range)
        qf = rng.standard_normal((1, 1, H, d_qk)) * 40.0
        kf = rng.standard_normal((1, 1, H, d_qk)) * 40.0
        for h in range(H):
            ch = rng.choice(d_qk, 4, replace=False)
            qf[0, 0, h, ch] *= 8.0
            kf[0, 0, h, ch] *= 8.0
        return (e4m3fn_encode(np.float32(np.clip(qf, -448, 448))),
                e4m3fn_encode(np.float32(np.clip(kf, -448, 448))))
    q = _codes(rng, (1, 1, H, d_qk), 48.0)
    k = _codes(rng, (1, 1, H, d_qk), 48.0)
    if kind == "dominant":
        # one channel per head holds the largest e4m3 value in both q and k
        ch = rng.integers(0, d_qk, H)
        big = e4m3fn_encode(np.float32([448.0]))[0]
        q[0, 0, np.arange(H), ch] = big
        k[0, 0, np.arange(H), ch] = big
    return q, k


@pytest.mark.parametrize("d_qk", [128, 192])
def test_fp8_mfma_dot_product_error(d_qk):
    worst = {}
    for i, kind in enumerate(("gauss", "dominant", "outliers")):
        q, k = _case(d_qk, kind, seed=7 + d_qk + i)
        H = q.shape[2]
        v = np.full((1, 1, H, 128), e4m3fn_encode(np.float32([1.0]))[0], dtype=np.uint8)
        print(f"case mfma precision d_qk={d_qk} {kind} H={H}", flush=True)
        qd, kd, vd = (torch.from_numpy(x).to("cuda") for x in (q, k, v))
        o, lse = ops.attn_prefill_fwd(qd, kd, vd, 1.0, 1.0, 1.0, causal=True, softmax_scale=LN2_F32)
        torch.cuda.synchronize()
        t = lse.cpu().numpy().astype(np.float64)[0, :, 0] / LN2_F32
        prod = e4m3fn_decode(q[0, 0]) * e4m3fn_decode(k[0, 0])  # [H, d_qk], exact in fp64
        exact = prod.sum(axis=1)
        mag = np.abs(prod).sum(axis=1)
        # the LSE's own fp32 rounding (ln 2 * t, then / ln 2 here) is 2^-24 of |t|
        rel = np.abs(t - exact) / mag
        worst[kind] = float(rel.max())
        print(f"  max |t - exact| / sum|products| = 2^{math.log2(max(worst[kind], 1e-30)):.2f} "
              f"(median 2^{math.log2(max(float(np.median(rel)), 1e-30)):.2f})", flush=True)
        assert np.all(np.isfinite(t))
        # O of a single key is that key's V row (1.0) exactly
        assert torch.all(o == 1.0).item()
    assert worst["gauss"] <= 2.0 ** -15 and worst["dominant"] <= 2.0 ** -13.5, worst
    assert worst["outliers"] <= 2.0 ** -11, worst
    # a correctly rounded fp32 accumulation of exact products, chained over
    # two or three MFMAs, is off by at most ~3 * 2^-24 of the sum of |products|
    assert worst["dominant"] >= 2.0 ** -20 and worst["outliers"] >= 2.0 ** -20, worst
