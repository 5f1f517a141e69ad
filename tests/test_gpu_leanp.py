"""Lean P (ATTN_FLAG_LEAN_P): O-only FP8 attention without exponentials.

The code of each probability is round(8 x + 56 + 8 kb) for p = 2^x (an e4m3
code read as an integer grows by 8 per doubling: Le Fil IA, context
paragraph; aicronaca.it, "Perché l'FP8 non basta da solo"; ai4bro.com,
"How does ZYFA work?"), and O is divided by the sum of those rounded
probabilities. It approximates 2^x by straight lines between powers of two,
so its result is compared with the oracle's exact attention on the bars of
the exact path: O relative L2 <= 3e-2 on every FP8 workload. The per-row
error is reported beside it.

Closed form: with Q = 0 every code is the same, so O is exactly the mean of
the visible V rows (only the bf16 output rounding remains).

These tests ran once with the mode enabled: every case passed except the
non-causal one (O rel-L2 0.0315), so the library now rejects the flag and
they are skipped. test_abi.py checks the rejection on the host.
"""

import numpy as np
import pytest
import torch

from bf16_causal_prefill_fwd_amd import ops
from bf16_causal_prefill_fwd_amd.workloads import WORKLOADS, Workload, make_inputs
from oracle import prefill_reference

from .parity_util import O_TOL, rel_l2, row_rel_l2
from .test_gpu_parity import dev, sample_rows

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skip(reason="Lean P is switched off in the library (ATTN_ERR_UNSUPPORTED): its O error missed the "
                            "3e-2 bar on the non-causal case (0.0315) and it ran no faster than the exact path"),
]

LEAN = ops.ATTN_FLAG_LEAN_P

GATE_SMALL = [
    Workload("tiny_mha_fp8", 1, 512, 2, 2, 128, 128, "fp8", "gauss"),
    Workload("ragged_gqa_fp8_outlier", 1, 777, 8, 2, 128, 128, "fp8", "outlier"),
    Workload("mla_fp8_1087", 1, 1087, 4, 2, 192, 128, "fp8", "mla"),
    Workload("gauss_2048", 1, 2048, 2, 2, 128, 128, "fp8", "gauss"),
    Workload("noncausal_fp8", 1, 300, 4, 2, 128, 128, "fp8", "gauss", causal=False),
]
GATE_FULL = ["gqa_fp8_outlier_16k", "mha_fp8_32k", "mla_fp8_16k"]


def _lean(q, k, v, causal=True):
    o, lse, ex = ops.prefill(dev(q), dev(k), dev(v), "fp8", causal=causal, hadamard=False, flags=LEAN)
    torch.cuda.synchronize()
    assert lse is None
    return o, ex


@pytest.mark.parametrize("w", GATE_SMALL, ids=[w.name for w in GATE_SMALL])
def test_lean_p_small(w):
    q, k, v = make_inputs(w, seed=1)
    print(f"case lean P {w.name} S={w.S} Hq={w.Hq} Hkv={w.Hkv} d={w.d_qk} causal={w.causal}", flush=True)
    o, ex = _lean(q, k, v, w.causal)
    ref = prefill_reference(q, k, v, "fp8", causal=w.causal, fold_q=True)
    og = o.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(og))
    err, rows = rel_l2(og, ref["o"]), row_rel_l2(og, ref["o"])
    print(f"  O rel-L2 {err:.4e}  rows: max {rows.max():.4e}", flush=True)
    o2, _ = ops.attn_prefill_fwd(ex["q"], ex["k"], ex["v"], causal=w.causal, d_scales=ex["scales"], flags=LEAN,
                                 return_lse=False)
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16))
    assert err <= O_TOL["fp8"], err


@pytest.mark.parametrize("name", GATE_FULL)
def test_lean_p_full_size(name):
    w = WORKLOADS[name]
    q, k, v = make_inputs(w, seed=0)
    print(f"case lean P {name} full size", flush=True)
    o, ex = _lean(q, k, v)
    rows = sample_rows(w, np.random.default_rng(12345))
    ref = prefill_reference(q, k, v, "fp8", rows=rows, fold_q=True)
    bi = torch.tensor([r[0] for r in rows]); hi = torch.tensor([r[1] for r in rows])
    ii = torch.tensor([r[2] for r in rows])
    og = o[bi, ii, hi].float().cpu().numpy().astype(np.float64)
    err, rr = rel_l2(og, ref["o_rows"]), row_rel_l2(og, ref["o_rows"])
    print(f"  {len(rows)} rows: O rel-L2 {err:.4e}  rows: max {rr.max():.4e}", flush=True)
    assert err <= O_TOL["fp8"], err


def test_lean_p_zero_query_closed_form():
    B, S, Hq, Hkv = 2, 1087, 16, 4
    w = Workload("zero_q", B, S, Hq, Hkv, 128, 128, "fp8", "gauss")
    q, k, v = make_inputs(w, seed=3)
    q[:] = 0
    print("case lean P zero_q", flush=True)
    o, ex = _lean(q, k, v)
    ref = prefill_reference(q, k, v, "fp8", rows=[(0, 0, 0)])
    vd = np.asarray(ref["views"][2][:])
    mean = np.repeat(np.cumsum(vd, axis=1) / np.arange(1, S + 1)[None, :, None, None], Hq // Hkv, axis=2)
    assert np.allclose(o.float().cpu().numpy(), mean, rtol=2 ** -8, atol=1e-5 * np.abs(vd).max())


def test_lean_p_rejects_lse_and_bf16():
    w = Workload("x", 1, 64, 2, 2, 128, 128, "fp8", "gauss")
    q, k, v = make_inputs(w, seed=1)
    _, _, ex = ops.prefill(dev(q), dev(k), dev(v), "fp8", hadamard=False)
    lse = torch.empty((1, 2, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        ops.attn_prefill_fwd(ex["q"], ex["k"], ex["v"], d_scales=ex["scales"], flags=LEAN, lse=lse)
    L = ops.lib()
    o = torch.empty((1, 64, 2, 128), dtype=torch.bfloat16, device="cuda")
    code = L.attn_prefill_fwd_ex(ex["q"].data_ptr(), ex["k"].data_ptr(), ex["v"].data_ptr(), o.data_ptr(),
                                 lse.data_ptr(), 1.0, 1.0, 1.0, None, 0.1, 1, 64, 2, 2, 128, 128, 1, 0, LEAN, None)
    assert code == -1  # an LSE output with Lean P
