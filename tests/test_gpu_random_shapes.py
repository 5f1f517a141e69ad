"""GPU parity on seeded random shapes, against the full fp64 oracle.

Besides the hand-picked cases of test_gpu_parity.py, 96 shapes drawn from a
fixed seed mix what those keep apart: batch 1-3, lengths 1-700 (any ragged
tail of the 64-key steps and 128-row tiles), 1-3 kv heads with 1, 2, 3, 4, 6
or 8 query heads each (so both work orders), d_qk 128 or 192, FP8 or BF16,
causal or not, Gaussian, heavy-tailed or MLA-shaped inputs, and for FP8 the
default input step (Q and K rotated, folded query scale), the unrotated one
with the folded query scale, or the plain per-tensor one, and each P mode
(exact, block-scaled, and block-scaled with the rounded-sum normalizer).
Every case must meet the same bars as the other parity tests: whole-tensor
and per-row O, LSE max-abs, bit-exact codes and scales, and a bit-identical
second launch. One reading applies to the LSE of heavy-tailed inputs
quantized without the rotation: there the gfx950 FP8 matrix core's summing
precision (pinned in test_gpu_mfma_precision.py) can move a row's LSE past
1e-2 where its query's and a key's outlier channels meet (aicronaca.it,
"Perché l'FP8 non basta da solo", on outlier channels and FP8), so a row may
exceed 1e-2 only by as much as that precision allows.
"""

import math
import os


import numpy as np
import pytest
import torch

from bf16_causal_prefill_fwd_amd import ops
from bf16_causal_prefill_fwd_amd.workloads import Workload, make_inputs
from oracle import prefill_reference
from oracle.formats import dequantize_fp8

from .parity_util import LSE_TOL, check_o
from .test_gpu_parity import codes_np, dev

pytestmark = pytest.mark.gpu

PS = ops.ATTN_FLAG_P_BLOCK_SCALE
RS = ops.ATTN_FLAG_P_ROUNDED_SUM


def _draw(n: int, seed: int = 2024):
    rng = np.random.default_rng(seed)
    # (a stream of its own, so that adding the unrotated folded step left the
    # other draws as they were)
    rng_rot = np.random.default_rng([seed, 1])
    cases = []
    for i in range(n):
        dtype = "fp8" if rng.random() < 0.65 else "bf16"
        dqk = 192 if rng.random() < 0.35 else 128
        B = int(rng.integers(1, 4))
        S = int(rng.choice([1, 2, 63, 64, 65, 127, 128, 129])) if rng.random() < 0.25 else int(rng.integers(1, 701))
        Hkv = int(rng.integers(1, 4))
        G = int(rng.choice([1, 2, 3, 4, 6, 8]))
        causal = bool(rng.random() < 0.75)
        dist = "mla" if dqk == 192 else str(rng.choice(["gauss", "outlier"]))
        fold_q = bool(rng.random() < 0.6) if dtype == "fp8" else True
        flags = int(rng.choice([0, 0, PS, RS | PS])) if dtype == "fp8" else 0
        rotated = dtype == "fp8" and fold_q and bool(rng_rot.random() < 0.75)
        w = Workload(f"rand{i}_{dtype}_d{dqk}_B{B}_S{S}_G{G}x{Hkv}", B, S, G * Hkv, Hkv, dqk, 128, dtype, dist,
                     causal=causal)
        cases.append((w, fold_q, rotated, flags, 1000 + i))
    return cases


# (a longer sweep: ATTN_RANDOM_SHAPES=1000 ATTN_RANDOM_SEED=79 python -m pytest -m gpu <this file>)
CASES = _draw(int(os.environ.get("ATTN_RANDOM_SHAPES", "96")), int(os.environ.get("ATTN_RANDOM_SEED", "2024")))


def _id(c):
    w, fold_q, rotated, flags, _ = c
    step = "" if w.dtype == "bf16" or rotated else ("_unrotated" if fold_q else "_plain_q")
    return f"{w.name}{'' if w.causal else '_noncausal'}{step}_f{flags}"


def _summing_bound(ref, w):
    """[B, Hq, S]: how far the FP8 matrix core's summing precision (within
    2^-11 of a dot product's sum of |products|) can move each row's LSE:
    2^-11 times the softmax scale times the row's largest sum of |products|
    over the keys it sees, on the oracle's dequantized codes."""
    qa = np.abs(dequantize_fp8(ref["q_codes"], ref["q_scale"]))
    ka = np.abs(dequantize_fp8(ref["k_codes"], ref["k_scale"]))
    G = w.Hq // w.Hkv
    seen = np.tril(np.ones((w.S, w.S), dtype=bool)) if w.causal else np.ones((w.S, w.S), dtype=bool)
    worst = np.empty((w.B, w.Hq, w.S))
    for b in range(w.B):
        for h in range(w.Hq):
            worst[b, h] = np.where(seen, qa[b, :, h, :] @ ka[b, :, h // G, :].T, 0.0).max(axis=1)
    return 2.0 ** -11 * worst / math.sqrt(w.d_qk)


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_random_shape_full_oracle(case):
    w, fold_q, rotated, flags, seed = case
    q, k, v = make_inputs(w, seed)
    print(f"case {_id(case)} seed={seed}", flush=True)
    o, lse, ex = ops.prefill(dev(q), dev(k), dev(v), w.dtype, causal=w.causal, fold_q=fold_q, hadamard=rotated,
                             flags=flags)
    torch.cuda.synchronize()
    ref = prefill_reference(q, k, v, w.dtype, causal=w.causal, fold_q=fold_q, hadamard=rotated)
    for name in ("q", "k", "v"):
        assert np.array_equal(codes_np(ex[name]), ref[name + "_codes"]), f"{name} codes differ"
    if w.dtype == "fp8":
        sc = ex["scales"].cpu().numpy()
        assert np.array_equal(sc, np.float32([ref["q_scale"], ref["k_scale"], ref["v_scale"]]))
    og = o.float().cpu().numpy().astype(np.float64)
    lg = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    check_o(og, ref["o"], w.dtype)
    lerr_rows = np.abs(lg - ref["lse"])
    lerr = float(np.max(lerr_rows))
    print(f"  LSE max-abs {lerr:.3e}", flush=True)
    if w.dtype == "fp8" and not rotated and w.dist == "outlier":
        bound = _summing_bound(ref, w)
        over = int(np.sum(lerr_rows > LSE_TOL))
        print(f"  unrotated heavy-tailed: {over} rows past {LSE_TOL}, largest error / summing bound "
              f"{np.max(lerr_rows / (bound + 2e-5)):.3f}", flush=True)
        assert np.all(lerr_rows <= np.maximum(LSE_TOL, bound + 2e-5))
    else:
        assert lerr <= LSE_TOL
    o2, l2 = ops.attn_prefill_fwd(ex["q"], ex["k"], ex["v"], causal=w.causal, d_scales=ex["scales"], flags=flags)
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16)) and torch.equal(l2, lse)
