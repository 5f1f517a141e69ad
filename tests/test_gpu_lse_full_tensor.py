"""LSE on EVERY row of the heavy-tailed FP8 GQA layer (B=1, S=16K, 32/8 heads).

The sampled-row tests check a few hundred rows. On this layer's inputs (four
x8 outlier channels per head in Q and K, drawn independently) a row whose Q
and K outlier channels meet reaches logits of 50-80, and the gfx950 FP8 matrix
core sums such a dot product only to within about 2^-12 of its sum of
|products| (pinned in test_gpu_mfma_precision.py). So a few dozen of the
524,288 rows land past the 1e-2 LSE bar on the unrotated input step (up to
about 2e-2), while the Hadamard-rotated input step (aicronaca.it, "Perché
l'FP8 non basta da solo": rotating Q and K before the FP8 cast) spreads the
outlier channels over every column and keeps every row far inside it. This
test computes the oracle's LSE for all rows (head by head, in worker processes
that run numpy and oracle/ only) and checks:

* rotated input step (the pipeline's default): every row's LSE within the
  1e-2 bar, and O within its bars over the whole tensor and on every row;
* unrotated input step, folded and plain query scale: every row within the
  bound that the matrix core's pinned summing error allows (2^-11 times the
  softmax scale times the row's largest sum of |products|), and the count of
  rows past 1e-2 is printed.

The e4m3 codes of every head slice are compared with the oracle's, bit for bit.
"""

import multiprocessing
import os

import numpy as np
import pytest
import torch

from bf16_causal_prefill_fwd_amd import ops
from bf16_causal_prefill_fwd_amd.workloads import WORKLOADS, make_inputs
from oracle import prefill_reference

from .lse_oracle_worker import head_lse
from .parity_util import LSE_TOL, O_TOL, ROW_TOL
from .test_gpu_parity import dev

pytestmark = pytest.mark.gpu

W = WORKLOADS["gqa_fp8_outlier_16k"]
PIPES = [("rotated", dict(hadamard=True)), ("folded", dict(hadamard=False)), ("plain_q", dict(fold_q=False))]
# worker processes for the oracle: at most the 16 cores a single-GPU host gives a job
WORKERS = min(16, os.cpu_count() or 1)


@pytest.fixture(scope="module")
def inputs():
    return make_inputs(W, seed=0)


@pytest.mark.parametrize("label,kw", PIPES, ids=[p[0] for p in PIPES])
def test_heavy_tailed_layer_lse_on_every_row(inputs, label, kw):
    q, k, v = inputs
    rotated = kw.get("hadamard", False)
    fold_q = kw.get("fold_q", True)
    print(f"case {W.name} full tensor, input step {label}", flush=True)
    o, lse, ex = ops.prefill(dev(q), dev(k), dev(v), "fp8", **kw)
    torch.cuda.synchronize()
    lse_gpu = lse[0].cpu().numpy().astype(np.float64)
    q8, k8, v8 = (ex[n][0].cpu().numpy() for n in ("q", "k", "v"))
    o_gpu = o[0].float().cpu().numpy() if rotated else None
    del o, lse, ex
    # the oracle's per-tensor scales (whole tensors), then every head in workers
    ref = prefill_reference(q, k, v, "fp8", rows=[(0, 0, 0)], fold_q=fold_q, hadamard=rotated)
    vq, vk, vv = ref["views"]
    qcs = vq.code_scale if rotated else vq.scale
    kcs = vk.code_scale if rotated else vk.scale
    G = W.Hq // W.Hkv
    tasks = [(np.ascontiguousarray(q[0, :, h, :]), np.ascontiguousarray(k[0, :, h // G, :]), rotated,
              qcs, vq.scale, kcs, vk.scale, True,
              np.ascontiguousarray(v[0, :, h // G, :]) if rotated else None, vv.scale,
              o_gpu[:, h, :] if rotated else None) for h in range(W.Hq)]
    with multiprocessing.get_context("spawn").Pool(WORKERS) as pool:
        results = pool.map(head_lse, tasks)
    err = np.empty((W.Hq, W.S))
    bound = np.empty((W.Hq, W.S))
    o_rows, o_sums = [], np.zeros(2)
    for h, r in enumerate(results):
        assert np.array_equal(q8[:, h, :], r["q_codes"]), f"q codes of head {h} differ"
        assert np.array_equal(k8[:, h // G, :], r["k_codes"]), f"k codes of kv head {h // G} differ"
        if r["v_codes"] is not None:
            assert np.array_equal(v8[:, h // G, :], r["v_codes"]), f"v codes of kv head {h // G} differ"
        err[h] = np.abs(lse_gpu[h] - r["lse"])
        bound[h] = r["bound"]
        if "o_row_err" in r:
            o_rows.append(r["o_row_err"])
            o_sums += r["o_sums"]
    over = int((err > LSE_TOL).sum())
    print(f"  LSE max-abs {err.max():.3e} over {err.size} rows, median {np.median(err):.2e}; "
          f"rows past {LSE_TOL}: {over}; largest error / matrix-core bound {np.max(err / (bound + 2e-5)):.3f}",
          flush=True)
    if rotated:
        o_rows = np.concatenate(o_rows)
        o_err = float(np.sqrt(o_sums[0] / o_sums[1]))
        print(f"  O rel-L2 {o_err:.3e}; rows: max {o_rows.max():.3e} p99.9 {np.quantile(o_rows, 0.999):.3e} "
              f"over {o_rows.size}", flush=True)
        assert o_err <= O_TOL["fp8"] and o_rows.max() <= ROW_TOL["fp8"]
        assert err.max() <= LSE_TOL
    else:
        assert np.all(err <= bound + 2e-5)
