"""The input step on seeded random sizes and value ranges, bit-exact.

Every entry point of the input step (per-tensor e4m3 codes with the plain or
the folded query scale, Hadamard-rotated Q or K, the fused Q/K/V step with and
without the rotation, the BF16 cast) on float32 or bfloat16 inputs of random
length (ragged tails of the 16-byte vectors and of the grid's trips), random
magnitude (1e-6 to 1e4) and a few x1000 outliers, against the oracle's codes
and scales (e4m3fn: ai4bro.com, "TL;DR"; the rotation: aicronaca.it, "Perché
l'FP8 non basta da solo"). Codes and scales must match bit for bit.
"""

import math
import os

import numpy as np
import pytest
import torch

from bf16_causal_prefill_fwd_amd import ops
from oracle.formats import bf16_encode, encode_with_scale, per_tensor_scale_folded, quantize_fp8_per_tensor
from oracle.rotation import hadamard_quantize

pytestmark = pytest.mark.gpu

KINDS = ["plain", "folded", "rotated_k", "rotated_q", "qkv", "qkv_rotated", "cast_bf16"]


def _values(rng, n):
    x = rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 4)
    if n > 8:
        idx = rng.choice(n, int(rng.integers(1, 5)), replace=False)
        x[idx] *= 1000.0
    return x.astype(np.float32)


def _tensor(rng, shape, xdt):
    x = _values(rng, int(np.prod(shape))).reshape(shape)
    t = torch.from_numpy(x).to("cuda")
    if xdt == "bf16":
        t = t.to(torch.bfloat16)
    return t, t.float().cpu().numpy()


def _draw(n, seed=2025):
    cases = []
    for i in range(n):
        rng = np.random.default_rng([seed, i])
        kind = KINDS[i % len(KINDS)]
        xdt = "fp32" if kind == "cast_bf16" else str(rng.choice(["fp32", "bf16"]))
        d = int(rng.choice([128, 192]))
        rows = int(rng.integers(1, 2500))
        cases.append((f"{kind}_{xdt}_{i}", kind, xdt, d, rows, i))
    return cases


# (a longer sweep: ATTN_INPUT_STEP_CASES=700 python -m pytest -m gpu <this file>)
CASES = _draw(int(os.environ.get("ATTN_INPUT_STEP_CASES", "28")))


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_input_step_random_bit_exact(case):
    name, kind, xdt, d, rows, i = case
    rng = np.random.default_rng([7, i])
    print(f"case {name} d={d} rows={rows}", flush=True)
    sm = 1.0 / math.sqrt(d)
    if kind in ("plain", "folded", "cast_bf16"):
        # flat lengths: any tail of the 16-byte vectors and of the trips
        n = int(rng.integers(1, 300000))
        x, x32 = _tensor(rng, (n,), xdt)
    else:
        x, x32 = _tensor(rng, (1, rows, 2, d), xdt)
    if kind == "plain":
        codes, scale = ops.attn_quantize_fp8(x)
        rc, rs = quantize_fp8_per_tensor(x32)
        assert np.array_equal(codes.cpu().numpy(), rc) and scale.item() == rs
    elif kind == "folded":
        ks = np.float32(10.0 ** rng.uniform(-4, 1))
        codes, scale = ops.attn_quantize_fp8(x, k_scale=torch.tensor([ks], device="cuda"), softmax_scale=sm)
        rs = per_tensor_scale_folded(x32, ks, sm)
        assert scale.item() == rs
        assert np.array_equal(codes.cpu().numpy(), encode_with_scale(x32, rs))
    elif kind == "rotated_k":
        codes, scale = ops.attn_quantize_fp8(x, hadamard=True)
        rc, rs = hadamard_quantize(x32)
        assert np.array_equal(codes.cpu().numpy(), rc) and scale.item() == rs
    elif kind == "rotated_q":
        ks = np.float32(10.0 ** rng.uniform(-4, 1))
        codes, scale = ops.attn_quantize_fp8(x, k_scale=torch.tensor([ks], device="cuda"), softmax_scale=sm,
                                             hadamard=True)
        rc, rs = hadamard_quantize(x32, k_scale=ks, softmax_scale=sm)
        assert np.array_equal(codes.cpu().numpy(), rc) and scale.item() == rs
    elif kind in ("qkv", "qkv_rotated"):
        rot = kind == "qkv_rotated"
        hkv = int(rng.integers(1, 3))
        k, k32 = _tensor(rng, (1, rows, hkv, d), xdt)
        v, v32 = _tensor(rng, (1, rows, hkv, 128), xdt)
        (q8, k8, v8), sc = ops.attn_quantize_fp8_qkv(x, k, v, sm, hadamard=rot)
        if rot:
            kc, ksr = hadamard_quantize(k32)
            qc, qsr = hadamard_quantize(x32, k_scale=ksr, softmax_scale=sm)
        else:
            kc, ksr = quantize_fp8_per_tensor(k32)
            qsr = per_tensor_scale_folded(x32, ksr, sm)
            qc = encode_with_scale(x32, qsr)
        vc, vsr = quantize_fp8_per_tensor(v32)
        for got, want in ((q8, qc), (k8, kc), (v8, vc)):
            assert np.array_equal(got.cpu().numpy(), want)
        assert np.array_equal(sc.cpu().numpy(), np.float32([qsr, ksr, vsr]))
    else:
        out = ops.attn_cast_bf16(x)
        assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), bf16_encode(x32))
