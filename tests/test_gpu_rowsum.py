"""GPU parity of the rounded-P row-sum normalizer (ATTN_FLAG_P_ROUNDED_SUM) against the fp64 oracle.

With the flag (valid together with block-scaled P, ATTN_FLAG_P_BLOCK_SCALE),
O is divided by the row sum of the rounded probabilities that the P.V MFMAs
take, accumulated by one more MFMA per step (P times an operand of e4m3
ones), instead of by the fp32 sum of the exact exponentials (aicronaca.it,
"Perché l'FP8 non basta da solo"; ai4bro.com, "How does ZYFA work?"); LSE
still comes from the exact sum. The oracle's result is the same
exact attention: only the rounding of O's normalizer changes, so the same
bars apply (whole tensor, per row, LSE), codes stay bit-exact and launches
bit-identical.

Cases: the small FP8 cases of the main parity file, closed-form Q = 0 (every
p is 1, so the rounded sum is exact), scores that rise every tile (the exact
path rescales the rounded sum with O on nearly every step), the three
full-size FP8 layers on sampled rows, and heavy-tailed inputs on which the
normalizer must lower the O error: rounding a row's largest probabilities
then cancels between O and the sum that divides it.
"""

import numpy as np
import pytest
import torch

from bf16_causal_prefill_fwd_amd import ops
from bf16_causal_prefill_fwd_amd.workloads import WORKLOADS, Workload, make_inputs
from oracle import prefill_reference

from .parity_util import LSE_TOL, check_o, rel_l2
from .test_gpu_parity import SMALL, codes_np, dev, sample_rows
from .test_gpu_pscale import _ramp_inputs

pytestmark = pytest.mark.gpu

RS = ops.ATTN_FLAG_P_ROUNDED_SUM
PS = ops.ATTN_FLAG_P_BLOCK_SCALE
MODES = [RS | PS]
MODE_IDS = ["rounded_sum_block_scaled"]
FP8_SMALL = [w for w in SMALL if w.dtype == "fp8"]


def _run(q, k, v, flags, causal=True, fold_q=True, hadamard=None):
    o, lse, ex = ops.prefill(dev(q), dev(k), dev(v), "fp8", causal=causal, fold_q=fold_q, hadamard=hadamard,
                             flags=flags)
    torch.cuda.synchronize()
    return o, lse, ex


def _lse_err(lse, ref):
    return float(np.max(np.abs(lse.cpu().numpy().astype(np.float64) - ref)))


@pytest.mark.parametrize("flags", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("w", FP8_SMALL, ids=[w.name for w in FP8_SMALL])
def test_small_rounded_sum(w, flags):
    q, k, v = make_inputs(w, seed=1)
    print(f"case {w.name} S={w.S} Hq={w.Hq} Hkv={w.Hkv} d={w.d_qk} causal={w.causal} flags={flags}", flush=True)
    o, lse, ex = _run(q, k, v, flags, w.causal)
    ref = prefill_reference(q, k, v, "fp8", causal=w.causal, fold_q=True, hadamard=True)
    for name in ("q", "k", "v"):
        assert np.array_equal(codes_np(ex[name]), ref[name + "_codes"])
    og = o.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(og))
    err, _ = check_o(og, ref["o"], "fp8")
    lerr = _lse_err(lse, ref["lse"])
    o0, _, _ = _run(q, k, v, 0, w.causal)
    err0 = rel_l2(o0.float().cpu().numpy().astype(np.float64), ref["o"])
    print(f"  LSE max-abs {lerr:.3e}; O rel-L2 exact sum {err0:.4e} -> rounded sum {err:.4e}", flush=True)
    assert lerr <= LSE_TOL
    o2, l2 = ops.attn_prefill_fwd(ex["q"], ex["k"], ex["v"], causal=w.causal, d_scales=ex["scales"], flags=flags)
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16)) and torch.equal(l2, lse)


@pytest.mark.parametrize("flags", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("dqk", [128, 192])
def test_zero_query_rounded_sum(dqk, flags):
    # Q = 0: every p is 1, exact in e4m3, so the rounded sum is i + 1 exactly
    B, S, Hq, Hkv = 2, 1087, 16, 4
    w = Workload("zero_q", B, S, Hq, Hkv, dqk, 128, "fp8", "gauss")
    q, k, v = make_inputs(w, seed=3)
    q[:] = 0
    print(f"case zero_q rounded sum d_qk={dqk} flags={flags}", flush=True)
    o, lse, ex = _run(q, k, v, flags)
    ref = prefill_reference(q, k, v, "fp8", rows=[(0, 0, 0)])
    vd = np.asarray(ref["views"][2][:])
    mean = np.repeat(np.cumsum(vd, axis=1) / np.arange(1, S + 1)[None, :, None, None], Hq // Hkv, axis=2)
    assert np.allclose(o.float().cpu().numpy(), mean, rtol=2 ** -8, atol=1e-5 * np.abs(vd).max())
    assert np.allclose(lse.cpu().numpy(), np.log(np.arange(1, S + 1))[None, None, :], rtol=0, atol=1e-5)


@pytest.mark.parametrize("flags", MODES, ids=MODE_IDS)
def test_rising_scores_rounded_sum(flags):
    # each tile holds the row's largest score: the exact path rescales O and
    # the rounded sum together on nearly every step
    q, k, v = _ramp_inputs(700, 2, True, seed=21)
    print(f"case rising scores, rounded sum, flags={flags}", flush=True)
    o, lse, ex = _run(q, k, v, flags)
    ref = prefill_reference(q, k, v, "fp8", fold_q=True, hadamard=True)
    check_o(o.float().cpu().numpy().astype(np.float64), ref["o"], "fp8")
    assert _lse_err(lse, ref["lse"]) <= LSE_TOL


# heavy-tailed inputs, unrotated (the default input step's rotation would
# spread the outlier channels this test is about): independent outlier
# channels (the GQA layer's distribution) and outlier channels shared by Q
# and K, whose rows are carried by a few keys. Their logits reach tens of
# units, where the FP8 MFMA's own summing error on a row's largest scores
# (pinned in test_gpu_mfma_precision) can move LSE past its bar in every P
# mode: the shared case does, so only O is compared there; this seed of the
# independent case stays under it (test_gpu_lse_full_tensor checks every row
# of the 16K layer).
HEAVY = [Workload("heavy_gqa_777", 1, 777, 8, 2, 128, 128, "fp8", "outlier"),
         Workload("shared_outlier_1024", 1, 1024, 4, 2, 128, 128, "fp8", "outlier_shared")]


@pytest.mark.parametrize("w", HEAVY, ids=[w.name for w in HEAVY])
def test_rounded_sum_lowers_heavy_tailed_error(w):
    q, k, v = make_inputs(w, seed=1)
    ref = prefill_reference(q, k, v, "fp8", fold_q=True)
    errs = {}
    for flags in (0, PS, RS | PS):
        print(f"case {w.name} flags={flags} unrotated", flush=True)
        o, lse, _ = _run(q, k, v, flags, hadamard=False)
        errs[flags], _ = check_o(o.float().cpu().numpy().astype(np.float64), ref["o"], "fp8", f"flags={flags}: ")
        lerr = _lse_err(lse, ref["lse"])
        print(f"  LSE max-abs {lerr:.3e}", flush=True)
        if w.dist == "outlier":
            assert lerr <= LSE_TOL
    print(f"  O rel-L2 exact P {errs[0]:.4e}, block-scaled P {errs[PS]:.4e}, "
          f"block-scaled with the rounded sum {errs[RS | PS]:.4e}", flush=True)
    assert errs[RS | PS] < errs[0] and errs[RS | PS] < errs[PS]


FULL = ["gqa_fp8_outlier_16k", "mha_fp8_32k", "mla_fp8_16k"]


@pytest.mark.parametrize("flags", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("name", FULL)
def test_full_size_rounded_sum(name, flags):
    w = WORKLOADS[name]
    q, k, v = make_inputs(w, seed=0)
    print(f"case {name} full size, flags={flags}", flush=True)
    o, lse, ex = _run(q, k, v, flags)
    rows = sample_rows(w, np.random.default_rng(12345))
    ref = prefill_reference(q, k, v, "fp8", rows=rows, fold_q=True, hadamard=True)
    bi = torch.tensor([r[0] for r in rows]); hi = torch.tensor([r[1] for r in rows])
    ii = torch.tensor([r[2] for r in rows])
    og = o[bi, ii, hi].float().cpu().numpy().astype(np.float64)
    err, _ = check_o(og, ref["o_rows"], "fp8", f"{len(rows)} rows: ")
    lerr = float(np.max(np.abs(lse[bi, hi, ii].cpu().numpy().astype(np.float64) - ref["lse_rows"])))
    print(f"  LSE max-abs {lerr:.3e}", flush=True)
    assert lerr <= LSE_TOL
    o2 = torch.empty_like(o); l2 = torch.empty_like(lse)
    bad = torch.zeros((), dtype=torch.int64, device="cuda")
    for _ in range(10):
        ops.attn_prefill_fwd(ex["q"], ex["k"], ex["v"], out=o2, lse=l2, d_scales=ex["scales"], flags=flags)
        bad += (o2.view(torch.int16) != o.view(torch.int16)).sum() + (l2 != lse).sum()
    torch.cuda.synchronize()
    assert bad.item() == 0
