"""GPU parity of block-scaled P (ATTN_FLAG_P_BLOCK_SCALE) against the fp64 oracle.

With the flag, every (query row, 64-key block) of probabilities is rounded to
e4m3 as p * 2^k and the P.V MFMA takes 2^-k back through the power-of-two
scale of its P operand (aicronaca.it, "Perché l'FP8 non basta da solo";
ai4bro.com, "How does ZYFA work?"). The oracle's result is the same exact
attention: only the rounding of P changes, so the same bars apply (whole
tensor, per row, LSE), codes stay bit-exact and launches bit-identical.

Cases: the small FP8 cases of the main parity file with both query-scale
forms, closed-form Q = 0, scores that rise every tile (the exact path sets
the shift from the block maximum) and scores that fall every tile (the shift
of later blocks is lifted), and the three full-size FP8 layers on sampled
rows. The error of the heavy-tailed layers with and without the flag is
printed side by side.
"""

import numpy as np
import pytest
import torch

from bf16_causal_prefill_fwd_amd import ops
from bf16_causal_prefill_fwd_amd.workloads import WORKLOADS, Workload, make_inputs
from oracle import prefill_reference

from .parity_util import LSE_TOL, check_o
from .test_gpu_parity import SMALL, codes_np, dev, sample_rows

pytestmark = pytest.mark.gpu

PS = ops.ATTN_FLAG_P_BLOCK_SCALE
FP8_SMALL = [w for w in SMALL if w.dtype == "fp8"]
RUNS = [(w, f) for w in FP8_SMALL for f in (True, False)]


def _run(q, k, v, causal=True, fold_q=True, flags=PS):
    o, lse, ex = ops.prefill(dev(q), dev(k), dev(v), "fp8", causal=causal, fold_q=fold_q, flags=flags)
    torch.cuda.synchronize()
    return o, lse, ex


def _lse_err(lse, ref):
    return float(np.max(np.abs(lse.cpu().numpy().astype(np.float64) - ref)))


@pytest.mark.parametrize("w,fold_q", RUNS, ids=[w.name + ("" if f else "_plain_q") for w, f in RUNS])
def test_small_block_scaled(w, fold_q):
    q, k, v = make_inputs(w, seed=1)
    print(f"case {w.name} S={w.S} Hq={w.Hq} Hkv={w.Hkv} d={w.d_qk} causal={w.causal} fold_q={fold_q} "
          f"block-scaled P", flush=True)
    o, lse, ex = _run(q, k, v, w.causal, fold_q)
    ref = prefill_reference(q, k, v, "fp8", causal=w.causal, fold_q=fold_q, hadamard=fold_q)
    for name in ("q", "k", "v"):
        assert np.array_equal(codes_np(ex[name]), ref[name + "_codes"])
    og = o.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(og))
    err, _ = check_o(og, ref["o"], "fp8")
    lerr = _lse_err(lse, ref["lse"])
    o0, _, _ = _run(q, k, v, w.causal, fold_q, flags=0)
    err0 = float(np.linalg.norm(o0.float().cpu().numpy() - ref["o"]) / np.linalg.norm(ref["o"]))
    print(f"  LSE max-abs {lerr:.3e}; O rel-L2 exact-P {err0:.4e} -> block-scaled {err:.4e}", flush=True)
    assert lerr <= LSE_TOL
    o2, l2 = ops.attn_prefill_fwd(ex["q"], ex["k"], ex["v"], causal=w.causal, d_scales=ex["scales"], flags=PS)
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16)) and torch.equal(l2, lse)


@pytest.mark.parametrize("dqk", [128, 192])
def test_zero_query_block_scaled(dqk):
    # Q = 0: every p is 1, exact under any power-of-two scaling
    B, S, Hq, Hkv = 2, 1087, 16, 4
    w = Workload("zero_q", B, S, Hq, Hkv, dqk, 128, "fp8", "gauss")
    q, k, v = make_inputs(w, seed=3)
    q[:] = 0
    print(f"case zero_q block-scaled d_qk={dqk}", flush=True)
    o, lse, ex = _run(q, k, v)
    ref = prefill_reference(q, k, v, "fp8", rows=[(0, 0, 0)])
    vd = np.asarray(ref["views"][2][:])
    mean = np.repeat(np.cumsum(vd, axis=1) / np.arange(1, S + 1)[None, :, None, None], Hq // Hkv, axis=2)
    assert np.allclose(o.float().cpu().numpy(), mean, rtol=2 ** -8, atol=1e-5 * np.abs(vd).max())
    assert np.allclose(lse.cpu().numpy(), np.log(np.arange(1, S + 1))[None, None, :], rtol=0, atol=1e-5)


def _ramp_inputs(S, H, rising: bool, seed: int):
    # k_j = ramp(j) * u, q_i = 4 u: the scores rise (or fall) with the key index
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(128).astype(np.float32)
    u /= np.float32(np.linalg.norm(u) / np.sqrt(128))
    j = np.arange(S, dtype=np.float32) / S
    ramp = (0.5 + 2.0 * j) if rising else (2.5 - 2.0 * j)
    k = np.ascontiguousarray(np.broadcast_to(ramp[None, :, None, None] * u, (1, S, H, 128))).astype(np.float32)
    k += 0.05 * rng.standard_normal(k.shape).astype(np.float32)
    q = np.ascontiguousarray(np.broadcast_to(4.0 * u, (1, S, H, 128))).astype(np.float32)
    v = rng.standard_normal((1, S, H, 128)).astype(np.float32)
    return q, k, v


@pytest.mark.parametrize("rising", [True, False], ids=["rising", "falling"])
@pytest.mark.parametrize("fold_q", [True, False], ids=["folded", "plain_q"])
def test_monotone_scores_block_scaled(rising, fold_q):
    # rising: each tile holds the row's largest score, so the exact path (and
    # its shift from the block maximum) runs on nearly every step; falling:
    # each tile's probabilities are far below the running maximum, so later
    # blocks are lifted by ever larger shifts
    q, k, v = _ramp_inputs(700, 2, rising, seed=21 if rising else 22)
    print(f"case {'rising' if rising else 'falling'} scores, block-scaled P, fold_q={fold_q}", flush=True)
    o, lse, ex = _run(q, k, v, fold_q=fold_q)
    ref = prefill_reference(q, k, v, "fp8", fold_q=fold_q, hadamard=fold_q)
    err, _ = check_o(o.float().cpu().numpy().astype(np.float64), ref["o"], "fp8")
    lerr = _lse_err(lse, ref["lse"])
    o0, _, _ = _run(q, k, v, fold_q=fold_q, flags=0)
    err0 = float(np.linalg.norm(o0.float().cpu().numpy() - ref["o"]) / np.linalg.norm(ref["o"]))
    print(f"  LSE max-abs {lerr:.3e}; O rel-L2 exact-P {err0:.4e} -> block-scaled {err:.4e}", flush=True)
    assert lerr <= LSE_TOL
    o2, l2 = ops.attn_prefill_fwd(ex["q"], ex["k"], ex["v"], d_scales=ex["scales"], flags=PS)
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16)) and torch.equal(l2, lse)


FULL = ["gqa_fp8_outlier_16k", "mha_fp8_32k", "mla_fp8_16k"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_block_scaled(name):
    w = WORKLOADS[name]
    q, k, v = make_inputs(w, seed=0)
    print(f"case {name} full size, block-scaled P", flush=True)
    o, lse, ex = _run(q, k, v)
    rows = sample_rows(w, np.random.default_rng(12345))
    ref = prefill_reference(q, k, v, "fp8", rows=rows, fold_q=True, hadamard=True)
    bi = torch.tensor([r[0] for r in rows]); hi = torch.tensor([r[1] for r in rows])
    ii = torch.tensor([r[2] for r in rows])
    og = o[bi, ii, hi].float().cpu().numpy().astype(np.float64)
    err, _ = check_o(og, ref["o_rows"], "fp8", f"{len(rows)} rows: ")
    lerr = float(np.max(np.abs(lse[bi, hi, ii].cpu().numpy().astype(np.float64) - ref["lse_rows"])))
    o0, _ = ops.attn_prefill_fwd(ex["q"], ex["k"], ex["v"], d_scales=ex["scales"])
    torch.cuda.synchronize()
    og0 = o0[bi, ii, hi].float().cpu().numpy().astype(np.float64)
    err0 = float(np.linalg.norm(og0 - ref["o_rows"]) / np.linalg.norm(ref["o_rows"]))
    print(f"  LSE max-abs {lerr:.3e}; O rel-L2 exact-P {err0:.4e} -> block-scaled {err:.4e}", flush=True)
    assert lerr <= LSE_TOL
    o2 = torch.empty_like(o); l2 = torch.empty_like(lse)
    bad = torch.zeros((), dtype=torch.int64, device="cuda")
    for _ in range(10):
        ops.attn_prefill_fwd(ex["q"], ex["k"], ex["v"], out=o2, lse=l2, d_scales=ex["scales"], flags=PS)
        bad += (o2.view(torch.int16) != o.view(torch.int16)).sum() + (l2 != lse).sum()
    torch.cuda.synchronize()
    assert bad.item() == 0
