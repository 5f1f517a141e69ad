"""GPU parity of the Hadamard-rotated FP8 input step against the fp64 oracle.

attn_quantize_fp8_hadamard (through the C ABI) against oracle/rotation.py:
codes and stored scales bit-exact (both sides decide the codes from fp64
rotated values), for keys and folded queries, fp32 and bf16 inputs, head dims
128 and 192, ragged row counts, a single row, an all-zero tensor and a
one-hot row. Then the whole path with the rotation against the oracle on the
same rotated inputs (O rel-L2 <= 3e-2 over the tensor and the per-row bar of
parity_util.py, LSE max-abs <= 1e-2, repeat launches bit-identical). The end-to-end error against fp64 attention on the
unquantized inputs must drop on inputs whose large channels Q and K share,
which is the effect the pages report (aicronaca.it, section "Perché l'FP8 non
basta da solo"). Last, the full-size GQA layer: whole Q and K code tensors
bit-exact and sampled rows of the attention.
"""

import math

import numpy as np
import pytest
import torch

from bf16_causal_prefill_fwd_amd import ops
from bf16_causal_prefill_fwd_amd.workloads import WORKLOADS, Workload, make_inputs
from oracle import causal_attention, prefill_reference
from oracle.rotation import hadamard_quantize

pytestmark = pytest.mark.gpu

from .parity_util import LSE_TOL, check_o, rel_l2  # noqa: E402


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def _input(shape, xdtype, seed):
    """(device tensor, the float32 values the oracle sees)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32)
    x[..., rng.choice(shape[-1], 3, replace=False)] *= 8.0
    t = torch.from_numpy(x)
    if xdtype == "bf16":
        t = t.to(torch.bfloat16)
        x = t.float().numpy()
    return t.to("cuda"), x


CODE_CASES = [
    (128, "fp32", "k", (1, 777, 3)),
    (128, "bf16", "q", (2, 301, 4)),
    (192, "fp32", "q", (1, 500, 3)),
    (192, "bf16", "k", (1, 123, 5)),
    (128, "fp32", "q", (1, 1, 1)),
    (192, "fp32", "k", (1, 1, 1)),
    (128, "bf16", "k", (1, 2048, 8)),
]


@pytest.mark.parametrize("d,xdtype,role,shape", CODE_CASES,
                         ids=[f"d{c[0]}_{c[1]}_{c[2]}_{'x'.join(map(str, c[3]))}" for c in CODE_CASES])
def test_rotated_codes_and_scale_bit_exact(d, xdtype, role, shape):
    print(f"case rotated codes d={d} {xdtype} {role} shape={shape}", flush=True)
    t, x = _input(shape + (d,), xdtype, seed=d + len(shape) + shape[1])
    if role == "k":
        codes, scale = ops.attn_quantize_fp8(t, hadamard=True)
        rc, rs = hadamard_quantize(x)
    else:
        ks = np.float32(0.0123)
        sm = 1.0 / math.sqrt(d)
        codes, scale = ops.attn_quantize_fp8(t, hadamard=True, k_scale=torch.tensor([ks], device="cuda"),
                                             softmax_scale=sm)
        rc, rs = hadamard_quantize(x, k_scale=ks, softmax_scale=sm)
    torch.cuda.synchronize()
    got = codes.cpu().numpy()
    assert np.array_equal(got, rc), f"{int((got != rc).sum())} codes differ"
    assert scale.cpu().numpy()[0] == rs


def test_rotated_zero_and_one_hot():
    print("case rotated zero / one-hot", flush=True)
    z = torch.zeros(3, 5, 2, 192, device="cuda")
    c, s = ops.attn_quantize_fp8(z, hadamard=True)
    assert s.item() == 1.0 and not c.any().item()
    c, s = ops.attn_quantize_fp8(z, hadamard=True, k_scale=torch.tensor([0.5], device="cuda"), softmax_scale=0.1)
    assert s.item() == 1.0 / 64 and not c.any().item()
    x = torch.zeros(1, 1, 1, 128, device="cuda")
    x[..., 3] = 5.0
    c, s = ops.attn_quantize_fp8(x, hadamard=True)
    signs = np.array([bin(3 & j).count("1") & 1 for j in range(128)])
    assert np.array_equal(c.cpu().numpy().reshape(-1), np.where(signs == 1, 0xFE, 0x7E).astype(np.uint8))
    assert s.item() == float(np.float32(np.float32(5.0) / np.float32(448.0)))


ROT_CASES = [
    Workload("rot_gqa_shared_outliers", 1, 777, 8, 2, 128, 128, "fp8", "outlier_shared"),
    Workload("rot_mla", 1, 333, 4, 4, 192, 128, "fp8", "mla"),
    Workload("rot_batch2_gauss", 2, 300, 4, 1, 128, 128, "fp8", "gauss"),
    Workload("rot_noncausal", 1, 200, 2, 2, 128, 128, "fp8", "outlier_shared", causal=False),
]


@pytest.mark.parametrize("w", ROT_CASES, ids=[w.name for w in ROT_CASES])
def test_rotated_path_matches_oracle(w):
    q, k, v = make_inputs(w, seed=2)
    print(f"case {w.name} B={w.B} S={w.S} Hq={w.Hq} Hkv={w.Hkv} d={w.d_qk} causal={w.causal} hadamard", flush=True)
    o, lse, ex = ops.prefill(dev(q), dev(k), dev(v), "fp8", causal=w.causal, hadamard=True)
    torch.cuda.synchronize()
    ref = prefill_reference(q, k, v, "fp8", causal=w.causal, hadamard=True)
    for name in ("q", "k", "v"):
        assert np.array_equal(ex[name].cpu().numpy(), ref[name + "_codes"]), f"{name} codes differ"
    sc = ex["scales"].cpu().numpy()
    assert np.array_equal(sc, np.float32([ref["q_scale"], ref["k_scale"], ref["v_scale"]]))
    og = o.float().cpu().numpy().astype(np.float64)
    lg = lse.cpu().numpy().astype(np.float64)
    check_o(og, ref["o"], "fp8")
    lerr = float(np.max(np.abs(lg - ref["lse"])))
    print(f"  LSE max-abs {lerr:.3e}", flush=True)
    assert lerr <= LSE_TOL
    o2, l2 = ops.attn_prefill_fwd(ex["q"], ex["k"], ex["v"], causal=w.causal, d_scales=ex["scales"])
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16)) and torch.equal(l2, lse)


def test_rotation_reduces_error_against_unquantized_inputs():
    w = Workload("rot_error", 1, 1024, 4, 2, 128, 128, "fp8", "outlier_shared")
    q, k, v = make_inputs(w, seed=4)
    print("case rotation error vs unquantized fp64, outlier_shared S=1024", flush=True)
    O, _ = causal_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64))
    errs = {}
    for rot in (False, True):
        o, _, _ = ops.prefill(dev(q), dev(k), dev(v), "fp8", hadamard=rot)
        errs[rot] = rel_l2(o.float().cpu().numpy().astype(np.float64), O)
    print(f"  O rel-L2 vs unquantized: plain {errs[False]:.4f}  rotated {errs[True]:.4f}", flush=True)
    assert errs[True] < 0.6 * errs[False]


def test_full_size_gqa_rotated():
    w = WORKLOADS["gqa_fp8_outlier_16k"]
    q, k, v = make_inputs(w, seed=0, dist="outlier_shared")
    print("case full-size GQA 16K outlier_shared, hadamard", flush=True)
    o, lse, ex = ops.prefill(dev(q), dev(k), dev(v), "fp8", hadamard=True)
    torch.cuda.synchronize()
    kc, ks = hadamard_quantize(k)
    assert np.array_equal(ex["k"].cpu().numpy(), kc)
    sm = 1.0 / math.sqrt(w.d_qk)
    qc, qs = hadamard_quantize(q, k_scale=ks, softmax_scale=sm)
    assert np.array_equal(ex["q"].cpu().numpy(), qc)
    del qc, kc
    sc = ex["scales"].cpu().numpy()
    assert sc[0] == qs and sc[1] == ks
    rng = np.random.default_rng(99)
    rows = [(0, int(h), int(i)) for h in (0, 13, 31) for i in sorted(set([0, 1, 4095, 8191, w.S - 1]
                                                                          + list(rng.integers(0, w.S, 3))))]
    ref = prefill_reference(q, k, v, "fp8", rows=rows, hadamard=True)
    assert np.array_equal(sc, np.float32([ref["q_scale"], ref["k_scale"], ref["v_scale"]]))
    bi = torch.tensor([r[0] for r in rows]); hi = torch.tensor([r[1] for r in rows])
    ii = torch.tensor([r[2] for r in rows])
    og = o[bi, ii, hi].float().cpu().numpy().astype(np.float64)
    lg = lse[bi, hi, ii].cpu().numpy().astype(np.float64)
    check_o(og, ref["o_rows"], "fp8", f"{len(rows)} rows: ")
    lerr = float(np.max(np.abs(lg - ref["lse_rows"])))
    print(f"  LSE max-abs {lerr:.3e}", flush=True)
    assert lerr <= LSE_TOL


@pytest.mark.parametrize("xdt", ["fp32", "bf16"])
@pytest.mark.parametrize("dqk", [128, 192])
def test_fused_rotated_input_step_matches_separate_calls(xdt, dqk):
    # one absmax and one encode launch for rotated Q and K and plain V give
    # the codes and scales of the three separate calls, and the oracle's
    rng = np.random.default_rng(40 + dqk)
    shapes = ((1, 333, 4, dqk), (1, 333, 2, dqk), (1, 333, 2, 128))
    xs = []
    for sh in shapes:
        t, _ = _input(sh, xdt, int(rng.integers(1 << 30)))
        xs.append(t)
    print(f"case fused rotated input step {xdt} d_qk={dqk}", flush=True)
    sm = 1.0 / math.sqrt(dqk)
    (q8, k8, v8), sc = ops.attn_quantize_fp8_qkv(*xs, sm, hadamard=True)
    k8s, ks = ops.attn_quantize_fp8(xs[1], hadamard=True)
    v8s, vs = ops.attn_quantize_fp8(xs[2])
    q8s, qs = ops.attn_quantize_fp8(xs[0], k_scale=ks, softmax_scale=sm, hadamard=True)
    torch.cuda.synchronize()
    assert torch.equal(q8, q8s) and torch.equal(k8, k8s) and torch.equal(v8, v8s)
    assert torch.equal(sc, torch.cat([qs, ks, vs]))
    x32 = [t.float().cpu().numpy() for t in xs]
    kc, ksr = hadamard_quantize(x32[1])
    qc, qsr = hadamard_quantize(x32[0], k_scale=ksr, softmax_scale=sm)
    assert np.array_equal(k8.cpu().numpy(), kc) and np.array_equal(q8.cpu().numpy(), qc)
    assert sc[0].item() == qsr and sc[1].item() == ksr
