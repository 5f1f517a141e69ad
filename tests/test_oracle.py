"""Pins of the CPU oracle against facts that do not come from the oracle.

Format pins: torch's own float8_e4m3fn / bfloat16 casts (an independent
library routine) and the pages' +8-codes-per-doubling fact.
Attention pins: brute force with math.fsum on tiny inputs (a different
computation: no max subtraction, log-domain normalisation), closed forms
(Q = 0 gives running means and LSE = ln(i+1); a hand-worked 2-row case),
invariants (rows of P sum to 1, row 0 copies V row 0, the causal mask hides
future keys), and library reductions (GQA = MHA with repeated K/V heads, the
last causal row = the unmasked row via scipy's softmax).
"""

import math
import os

import numpy as np
import pytest
import torch
from scipy.special import softmax as scipy_softmax

from oracle import (
    attention_rows,
    bf16_decode,
    bf16_encode,
    causal_attention,
    e4m3fn_decode,
    e4m3fn_encode,
    per_tensor_scale,
    per_tensor_scale_folded,
    prefill_reference,
    quantize_fp8_per_tensor,
    encode_with_scale,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_e4m3_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


# ----------------------------------------------------------------------------- formats

def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3fn_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0


def test_e4m3_plus_8_per_doubling_golden():
    rows = np.loadtxt(os.path.join(GOLDEN, "e4m3_powers_of_two.txt"), dtype=np.int64)
    for n, code in rows:
        assert e4m3fn_decode(np.array([code]))[0] == 2.0 ** n
        assert int(e4m3fn_encode(np.array([2.0 ** n], np.float32))[0]) == code
    # the fact itself, over every normal positive code that has a doubled partner
    c = np.arange(8, 0x7E - 8 + 1)
    assert np.array_equal(e4m3fn_decode(c + 8), 2.0 * e4m3fn_decode(c))


def test_e4m3_encode_matches_torch_random_and_ties():
    rng = np.random.default_rng(7)
    mags = np.exp2(rng.uniform(-14, 8.8, 200_000)).astype(np.float32)
    signs = np.where(rng.random(mags.size) < 0.5, -1, 1).astype(np.float32)
    x = mags * signs
    # exact midpoints between neighbouring codes: ties must go to the even code
    pos = e4m3fn_decode(np.arange(0x7F))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, np.float32([0.0, -0.0, 448.0, -448.0, 460.0, 464.0])])
    got = e4m3fn_encode(x)
    ref = torch_e4m3_bits(x)
    assert np.array_equal(got, ref)


def test_e4m3_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        e4m3fn_encode(np.float32([465.0]))
    with pytest.raises(ValueError):
        e4m3fn_encode(np.float32([np.nan]))


def test_quantizer_matches_torch_cast():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 33, 3, 16), dtype=np.float32)
    x[1, 2, 0, 5] = 9.5  # the absmax element
    codes, scale = quantize_fp8_per_tensor(x)
    assert scale.dtype == np.float32
    assert scale == np.float32(np.float32(9.5) / np.float32(448.0))
    ref = torch_e4m3_bits((x / scale).astype(np.float32))
    assert np.array_equal(codes, ref)
    assert codes[1, 2, 0, 5] == 0x7E  # the absmax lands on 448


def test_quantizer_zero_tensor():
    codes, scale = quantize_fp8_per_tensor(np.zeros((3, 5), np.float32))
    assert scale == 1.0 and not codes.any()


def _folded_cases():
    rng = np.random.default_rng(41)
    for i in range(300):
        x = (rng.standard_normal(257) * 10.0 ** rng.uniform(-6, 6)).astype(np.float32)
        ks = np.float32(10.0 ** rng.uniform(-8, 2))
        sm = np.float32(1.0 / math.sqrt([64, 128, 192, 256][i % 4]))
        yield x, ks, sm


def test_folded_scale_by_search_and_bounds():
    # j found by a plain search over integers (not frexp), the bounds of the
    # definition, and the power-of-two product, checked in exact rationals
    from fractions import Fraction
    for x, ks, sm in _folded_cases():
        a = float(np.max(np.abs(x)))
        g = (float(ks) * float(sm)) * math.log2(math.e)
        t = (a / 448.0) * g
        j = next(jj for jj in range(-300, 300) if 2.0 ** jj >= t)
        assert 2.0 ** (j - 1) < t
        sc = per_tensor_scale_folded(x, ks, sm)
        assert sc == np.float32(2.0 ** j / g)
        base = Fraction(a) / 448
        assert Fraction(float(sc)) >= base * (1 - Fraction(1, 2 ** 23))
        assert Fraction(float(sc)) < 2 * base * (1 + Fraction(1, 2 ** 22))
        prod = Fraction(float(sc)) * Fraction(float(ks)) * Fraction(float(sm)) * Fraction(math.log2(math.e))
        assert abs(prod / Fraction(2) ** j - 1) < Fraction(1, 2 ** 22)
        # codes stay in range: nothing overflows to NaN and |value| <= 448
        dec = e4m3fn_decode(encode_with_scale(x, sc))
        assert np.all(np.isfinite(dec)) and np.abs(dec).max() <= 448.0
        # never below the plain scale's precision: at most one binade coarser
        assert sc >= per_tensor_scale(x) * np.float32(1 - 2 ** -22)


def test_folded_scale_zero_tensor_and_exact_power():
    assert per_tensor_scale_folded(np.zeros(9, np.float32), np.float32(0.5), np.float32(0.125)) == 1.0
    # absmax/448 * g exactly a power of two: the plain scale is already folded.
    # k_scale * sm * log2(e) is rounded in fp64, so pick absmax so that
    # (absmax/448) * g is 2^-3 up to that rounding and check the result lands
    # on 2^-3 / g itself.
    ks, sm = np.float32(2.0 ** -4), np.float32(2.0 ** -3)
    g = (float(ks) * float(sm)) * math.log2(math.e)
    a = np.float32(448.0 * 2.0 ** -3 / g)
    x = np.array([a, -a / 2, 1.0], np.float32)
    sc = per_tensor_scale_folded(x, ks, sm)
    j = math.ceil(math.log2((float(a) / 448.0) * g))
    assert sc == np.float32(2.0 ** j / g) and j in (-3, -2)


def test_bf16_encode_matches_torch():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(300_000) * np.exp2(rng.uniform(-30, 30, 300_000))).astype(np.float32)
    # ties: low 16 bits exactly 0x8000, with both parities of the kept part
    t = rng.integers(0x00800000, 0x7E000000, 4096, dtype=np.uint32) & np.uint32(0xFFFF0000)
    ties = (t | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.float32([0.0, -0.0, 1.0])])
    got = bf16_encode(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.uint16).numpy()
    assert np.array_equal(got, ref)
    assert np.array_equal(bf16_decode(got), torch.from_numpy(x).to(torch.bfloat16).double().numpy())


# ----------------------------------------------------------------------------- attention

def brute_force(q, k, v, causal=True, scale=None):
    """Per-row pure Python: logits by fsum, LSE = log(fsum(exp)), no max shift."""
    B, S, Hq, dqk = q.shape
    Hkv, dv = k.shape[2], v.shape[3]
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(dqk) if scale is None else scale
    O = np.zeros((B, S, Hq, dv))
    L = np.zeros((B, Hq, S))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(S):
                js = range(i + 1) if causal else range(S)
                logit = [math.fsum(float(q[b, i, h, c]) * float(k[b, j, g, c]) for c in range(dqk)) * sc
                         for j in js]
                lse = math.log(math.fsum(math.exp(x) for x in logit))
                w = [math.exp(x - lse) for x in logit]
                for c in range(dv):
                    O[b, i, h, c] = math.fsum(wj * float(v[b, j, g, c]) for wj, j in zip(w, js))
                L[b, h, i] = lse
    return O, L


@pytest.mark.parametrize("S,Hq,Hkv,dqk,dv,causal", [
    (1, 1, 1, 16, 16, True),
    (2, 2, 1, 16, 16, True),
    (17, 4, 1, 24, 16, True),
    (17, 2, 2, 16, 16, False),
    (64, 4, 2, 16, 16, True),
    (130, 1, 1, 24, 16, True),
])
def test_attention_vs_brute_force(S, Hq, Hkv, dqk, dv, causal):
    rng = np.random.default_rng(S * 100 + Hq * 10 + Hkv)
    q = rng.standard_normal((1, S, Hq, dqk))
    k = rng.standard_normal((1, S, Hkv, dqk))
    v = rng.standard_normal((1, S, Hkv, dv))
    O, L = causal_attention(q, k, v, causal=causal)
    Ob, Lb = brute_force(q, k, v, causal=causal)
    assert np.max(np.abs(O - Ob)) <= 1e-12 * max(1.0, np.max(np.abs(Ob)))
    assert np.max(np.abs(L - Lb)) <= 1e-12 * max(1.0, np.max(np.abs(Lb)))


def test_attention_mla_shape_vs_brute_force():
    rng = np.random.default_rng(192)
    q = rng.standard_normal((1, 9, 2, 192))
    k = rng.standard_normal((1, 9, 2, 192))
    v = rng.standard_normal((1, 9, 2, 128))
    O, L = causal_attention(q, k, v)
    Ob, Lb = brute_force(q, k, v)
    assert np.allclose(O, Ob, rtol=0, atol=1e-12) and np.allclose(L, Lb, rtol=0, atol=1e-12)
    # the 192-dim logit is the sum of the no-rope (128) and rope (64) parts
    s_split = (q[0, :, 0, :128] @ k[0, :, 0, :128].T + q[0, :, 0, 128:] @ k[0, :, 0, 128:].T) / math.sqrt(192)
    s_split = np.where(np.tril(np.ones((9, 9), bool)), s_split, -np.inf)
    assert np.allclose(L[0, 0], np.log(np.exp(s_split).sum(1)), rtol=0, atol=1e-12)


def test_hand_worked_two_rows():
    # d = 4 -> softmax scale 1/2. Row 0 sees key 0 only; row 1 sees keys 0, 1.
    q = np.zeros((1, 2, 1, 4)); k = np.zeros((1, 2, 1, 4)); v = np.zeros((1, 2, 1, 4))
    q[0, 1, 0, 0] = 2.0          # q1 = (2,0,0,0)
    k[0, 0, 0, 0] = 1.0          # k0 = (1,0,0,0), k1 = 0  ->  s10 = 2*1/2 = 1, s11 = 0, s00 = 0
    v[0, 0, 0] = [1.0, 0.0, 3.0, -1.0]
    v[0, 1, 0] = [0.0, 1.0, 5.0, 1.0]
    O, L = causal_attention(q, k, v)
    e = math.e
    assert L[0, 0, 0] == 0.0
    assert abs(L[0, 0, 1] - 1.3132616875182228) < 1e-15       # ln(1 + e)
    assert np.allclose(O[0, 0, 0], v[0, 0, 0], rtol=0, atol=0)
    want = (e * v[0, 0, 0] + v[0, 1, 0]) / (e + 1.0)
    assert np.allclose(O[0, 1, 0], want, rtol=0, atol=1e-15)


def test_invariants_rows_sum_to_one_and_row0():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 40, 4, 16)) * 3
    k = rng.standard_normal((2, 40, 2, 16)) * 3
    v = np.full((2, 40, 2, 8), 2.5)
    O, _ = causal_attention(q, k, v)
    assert np.allclose(O, 2.5, rtol=0, atol=1e-13)        # softmax rows sum to 1
    v = rng.standard_normal((2, 40, 2, 8))
    O, L = causal_attention(q, k, v)
    for h in range(4):
        assert np.array_equal(O[:, 0, h], v[:, 0, h // 2])  # row 0 sees only key 0 (weight exactly 1)
        # LSE of row 0 is its single logit q0.k0 / sqrt(16)
        assert np.allclose(L[:, h, 0], np.sum(q[:, 0, h] * k[:, 0, h // 2], axis=1) / 4.0, atol=1e-13)


def test_constant_logits_running_mean():
    rng = np.random.default_rng(9)
    S = 70
    v = rng.standard_normal((1, S, 1, 8))
    means = np.cumsum(v[0, :, 0], axis=0) / np.arange(1, S + 1)[:, None]
    # Q = 0: every logit is 0
    O, L = causal_attention(np.zeros((1, S, 1, 16)), rng.standard_normal((1, S, 1, 16)), v)
    assert np.allclose(O[0, :, 0], means, rtol=0, atol=1e-13)
    assert np.allclose(L[0, 0], np.log(np.arange(1, S + 1)), rtol=0, atol=1e-13)
    # all K rows equal: logit of row i is the constant c_i = q_i.k / 4
    kk = np.tile(rng.standard_normal(16), (1, S, 1, 1))
    q = rng.standard_normal((1, S, 1, 16))
    O, L = causal_attention(q, kk, v)
    c = q[0, :, 0] @ kk[0, 0, 0] / 4.0
    assert np.allclose(O[0, :, 0], means, rtol=0, atol=1e-12)
    assert np.allclose(L[0, 0], c + np.log(np.arange(1, S + 1)), rtol=0, atol=1e-12)


def test_lse_direct_logsumexp_and_unmasked_last_row():
    rng = np.random.default_rng(13)
    S, d = 50, 16
    q = rng.standard_normal((1, S, 1, d)); k = rng.standard_normal((1, S, 1, d))
    v = rng.standard_normal((1, S, 1, d))
    O, L = causal_attention(q, k, v)
    s = q[0, :, 0] @ k[0, :, 0].T / 4.0
    for i in (0, 1, 17, S - 1):
        assert abs(L[0, 0, i] - math.log(np.exp(s[i, :i + 1]).sum())) < 1e-12
    # last causal row sees every key: equals the unmasked softmax (scipy)
    P = scipy_softmax(s, axis=1)
    assert np.allclose(O[0, S - 1, 0], P[S - 1] @ v[0, :, 0], rtol=0, atol=1e-13)
    On, _ = causal_attention(q, k, v, causal=False)
    assert np.allclose(On[0, :, 0], P @ v[0, :, 0], rtol=0, atol=1e-13)


def test_causal_mask_hides_future_keys():
    rng = np.random.default_rng(17)
    q = rng.standard_normal((1, 30, 2, 16)); k = rng.standard_normal((1, 30, 2, 16))
    v = rng.standard_normal((1, 30, 2, 8))
    O, L = causal_attention(q, k, v)
    k2, v2 = k.copy(), v.copy()
    k2[0, 20:] *= 50.0
    v2[0, 20:] += 7.0
    O2, L2 = causal_attention(q, k2, v2)
    assert np.array_equal(O[0, :20], O2[0, :20]) and np.array_equal(L[0, :, :20], L2[0, :, :20])
    assert not np.allclose(O[0, 20:], O2[0, 20:])


def test_gqa_equals_mha_with_repeated_heads():
    rng = np.random.default_rng(21)
    q = rng.standard_normal((2, 33, 8, 16)); k = rng.standard_normal((2, 33, 2, 16))
    v = rng.standard_normal((2, 33, 2, 8))
    O, L = causal_attention(q, k, v)
    Om, Lm = causal_attention(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2))
    assert np.array_equal(O, Om) and np.array_equal(L, Lm)


def test_attention_rows_matches_full():
    rng = np.random.default_rng(23)
    q = rng.standard_normal((2, 77, 4, 16)); k = rng.standard_normal((2, 77, 2, 16))
    v = rng.standard_normal((2, 77, 2, 8))
    O, L = causal_attention(q, k, v, row_block=16)
    rows = [(0, 0, 0), (1, 3, 76), (0, 2, 31), (1, 1, 40)]
    Or, Lr = attention_rows(q, k, v, rows)
    for t, (b, h, i) in enumerate(rows):
        assert np.allclose(Or[t], O[b, i, h], rtol=0, atol=1e-14)
        assert abs(Lr[t] - L[b, h, i]) < 1e-14


def test_prefill_reference_fp8_and_bf16_paths():
    rng = np.random.default_rng(29)
    q = rng.standard_normal((1, 40, 2, 16), dtype=np.float32)
    k = rng.standard_normal((1, 40, 1, 16), dtype=np.float32)
    v = rng.standard_normal((1, 40, 1, 16), dtype=np.float32)
    r = prefill_reference(q, k, v, "fp8")
    for name, x in (("q", q), ("k", k), ("v", v)):
        codes, scale = quantize_fp8_per_tensor(x)
        assert np.array_equal(r[name + "_codes"], codes) and r[name + "_scale"] == scale
    qd = e4m3fn_decode(r["q_codes"]) * float(r["q_scale"])
    kd = e4m3fn_decode(r["k_codes"]) * float(r["k_scale"])
    vd = e4m3fn_decode(r["v_codes"]) * float(r["v_scale"])
    O, L = causal_attention(qd, kd, vd)
    assert np.array_equal(r["o"], O) and np.array_equal(r["lse"], L)
    # fp8 inputs are close to the fp32 ones (quantization error only)
    O32, _ = causal_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64))
    assert np.linalg.norm(O - O32) / np.linalg.norm(O32) < 0.1
    rows = prefill_reference(q, k, v, "fp8", rows=[(0, 1, 39), (0, 0, 5)])
    assert np.allclose(rows["o_rows"][0], O[0, 39, 1], atol=1e-14)
    assert abs(rows["lse_rows"][1] - L[0, 0, 5]) < 1e-14
    rb = prefill_reference(q, k, v, "bf16")
    assert np.array_equal(rb["q_codes"], bf16_encode(q))
    Ob, _ = causal_attention(bf16_decode(rb["q_codes"]), bf16_decode(rb["k_codes"]), bf16_decode(rb["v_codes"]))
    assert np.array_equal(rb["o"], Ob)


def test_workload_generator_is_seeded_and_shaped():
    from bf16_causal_prefill_fwd_amd.workloads import WORKLOADS, make_inputs
    q, k, v = make_inputs("gqa_fp8_outlier_16k", seed=1, S=64)
    assert q.shape == (1, 64, 32, 128) and k.shape == (1, 64, 8, 128) and v.shape == (1, 64, 8, 128)
    q2, _, _ = make_inputs("gqa_fp8_outlier_16k", seed=1, S=64)
    assert np.array_equal(q, q2)
    # 4 outlier channels per head: their per-channel std is ~8x the others
    std = q[0].std(axis=0)  # [H, d]
    assert np.all(np.sort(std, axis=1)[:, -4:].min(axis=1) > 4.0)
    assert np.all(np.sort(std, axis=1)[:, :-4].max(axis=1) < 2.0)
    qm, km, _ = make_inputs("mla_fp8_16k", seed=0, S=256)
    assert qm.shape[-1] == 192 and abs(qm[..., 128:].std() / qm[..., :128].std() - math.sqrt(2)) < 0.05
    assert WORKLOADS["mha_fp8_32k"].causal_flops == pytest.approx(8.796093022208e12)
