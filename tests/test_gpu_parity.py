"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Bars: O relative L2 <= 3e-2 (FP8) / 5e-3 (BF16) over the
compared outputs, and the same measure taken row by row (each query row's
d_v outputs) <= ROW_TOL; LSE max-abs error <= 1e-2, quantized codes and
scales bit-exact, repeated launches bit-identical.
The bars and the reasoning behind the per-row one are in parity_util.py.

Small cases run the full oracle (several tiles, ragged tails, GQA, MLA, BF16,
non-causal, B > 1, S = 1). The five full-size workloads run in the same launch
configuration as bench.py and are compared on sampled rows, which the oracle
computes one by one.
"""

import hashlib
import math

import numpy as np
import pytest
import torch

from bf16_causal_prefill_fwd_amd import ops
from bf16_causal_prefill_fwd_amd.workloads import WORKLOADS, Workload, make_inputs
from oracle import prefill_reference

pytestmark = pytest.mark.gpu

from .parity_util import LSE_TOL, O_TOL, ROW_TOL, check_o, rel_l2, row_rel_l2  # noqa: F401


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def codes_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def rot(dtype: str, fold_q: bool) -> bool:
    """Whether the pipeline's default FP8 input step rotates Q and K: it does
    with the folded query scale; the plain-scale step is the unrotated one."""
    return dtype == "fp8" and fold_q


def run_case(w: Workload, seed: int, fold_q: bool = True):
    q, k, v = make_inputs(w, seed)
    print(f"case {w.name} B={w.B} S={w.S} Hq={w.Hq} Hkv={w.Hkv} d={w.d_qk}/{w.d_v} {w.dtype} "
          f"causal={w.causal} seed={seed} fold_q={fold_q} rotated={rot(w.dtype, fold_q)}", flush=True)
    o, lse, ex = ops.prefill(dev(q), dev(k), dev(v), w.dtype, causal=w.causal, fold_q=fold_q)
    torch.cuda.synchronize()
    return q, k, v, o, lse, ex


SMALL = [
    Workload("tiny_mha_fp8", 1, 512, 2, 2, 128, 128, "fp8", "gauss"),
    Workload("ragged_gqa_fp8_outlier", 1, 777, 8, 2, 128, 128, "fp8", "outlier"),
    Workload("batch2_gqa_fp8", 2, 300, 4, 1, 128, 128, "fp8", "gauss"),
    # B * Hkv = 8: the XCD-aware work order (whole kv units per XCD) is used
    Workload("batch2_xcd_order_fp8", 2, 200, 8, 4, 128, 128, "fp8", "outlier"),
    Workload("batch4_xcd_order_bf16", 4, 100, 4, 2, 128, 128, "bf16", "gauss"),
    Workload("single_row_fp8", 1, 1, 2, 2, 128, 128, "fp8", "gauss"),
    Workload("ragged_mla_fp8", 1, 333, 4, 4, 192, 128, "fp8", "mla"),
    # long enough for the FP8 MLA kernel's unchecked loop part (9 or more full
    # 64-key tiles; loop unrolled by the ring depth, one MFMA job of look-ahead)
    Workload("mla_fp8_unchecked_loop", 1, 700, 2, 2, 192, 128, "fp8", "mla"),
    Workload("ragged_gqa_bf16", 1, 333, 8, 2, 128, 128, "bf16", "gauss"),
    Workload("batch2_bf16", 2, 129, 2, 2, 128, 128, "bf16", "gauss"),
    Workload("ragged_mla_bf16", 1, 200, 2, 2, 192, 128, "bf16", "mla"),
    # the BF16 MLA kernel's unchecked loop part (32-key steps, 24-chunk K
    # swizzle) starts at 9 full tiles: one and several iterations of it,
    # causal and non-causal
    Workload("mla_bf16_unchecked_577", 1, 577, 2, 2, 192, 128, "bf16", "mla"),
    Workload("mla_bf16_unchecked_1087", 1, 1087, 4, 2, 192, 128, "bf16", "mla"),
    Workload("noncausal_mla_bf16_705", 1, 705, 2, 1, 192, 128, "bf16", "mla", causal=False),
    Workload("mla_fp8_gqa_1087", 1, 1087, 4, 2, 192, 128, "fp8", "mla"),
    Workload("noncausal_fp8", 1, 300, 4, 2, 128, 128, "fp8", "gauss", causal=False),
    Workload("noncausal_bf16", 1, 200, 2, 1, 128, 128, "bf16", "gauss", causal=False),
    Workload("noncausal_mla_fp8", 1, 150, 2, 2, 192, 128, "fp8", "mla", causal=False),
    # the FP8 MLA kernel's unchecked loop part without the causal mask
    Workload("noncausal_mla_fp8_700", 1, 700, 2, 2, 192, 128, "fp8", "mla", causal=False),
    # 16 query heads per kv head: one XCD unit spans 16 query heads
    Workload("gqa_group16_fp8", 1, 300, 16, 1, 128, 128, "fp8", "outlier"),
    Workload("gqa_group8_bf16", 2, 150, 16, 2, 128, 128, "bf16", "gauss"),
    # group sizes that are not powers of two, under the plain tile-major order
    # (B * Hkv = 2) and the XCD order (B * Hkv = 8)
    Workload("gqa_group6_fp8", 1, 1000, 12, 2, 128, 128, "fp8", "outlier"),
    Workload("mla_group3_fp8", 1, 600, 6, 2, 192, 128, "fp8", "mla"),
    Workload("xcd_order_group3_fp8", 1, 300, 24, 8, 128, 128, "fp8", "gauss"),
    Workload("xcd_order_group3_bf16", 1, 300, 24, 8, 128, 128, "bf16", "outlier"),
    # many short sequences: 64 x 130 tokens, a full and a 2-row query tile each
    Workload("batch64_short_fp8", 64, 130, 4, 2, 128, 128, "fp8", "gauss"),
    Workload("batch64_short_mla_bf16", 64, 130, 2, 2, 192, 128, "bf16", "mla"),
]


# FP8 cases run twice: with the folded query scale (the kernel's folded score
# form) and with the plain per-tensor scale (its fma form)
SMALL_RUNS = [(w, True) for w in SMALL] + [(w, False) for w in SMALL if w.dtype == "fp8"]


@pytest.mark.parametrize("w,fold_q", SMALL_RUNS,
                         ids=[w.name + ("" if f else "_plain_q") for w, f in SMALL_RUNS])
def test_small_full_oracle(w, fold_q):
    q, k, v, o, lse, ex = run_case(w, seed=1, fold_q=fold_q)
    ref = prefill_reference(q, k, v, w.dtype, causal=w.causal, fold_q=fold_q, hadamard=rot(w.dtype, fold_q))
    for name in ("q", "k", "v"):
        assert np.array_equal(codes_np(ex[name]), ref[name + "_codes"]), f"{name} codes differ"
    if w.dtype == "fp8":
        sc = ex["scales"].cpu().numpy()
        assert np.array_equal(sc, np.float32([ref["q_scale"], ref["k_scale"], ref["v_scale"]]))
    og = o.float().cpu().numpy().astype(np.float64)
    lg = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    check_o(og, ref["o"], w.dtype)
    lerr = float(np.max(np.abs(lg - ref["lse"])))
    print(f"  LSE max-abs {lerr:.3e}", flush=True)
    assert lerr <= LSE_TOL
    # a second launch is bit-identical
    o2, l2 = ops.attn_prefill_fwd(ex["q"], ex["k"], ex["v"], causal=w.causal, d_scales=ex["scales"])
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16)) and torch.equal(l2, lse)


ZERO_Q = [
    # (B, S, Hq, Hkv, d_qk): the first is a short single-kv-head case; the
    # others run the unchecked main loop (S = 1087: 16 full tiles), four query
    # heads per kv head, B * Hkv = 8 (the XCD-aware work order) and, with
    # d_qk = 192, the MLA kernels
    (1, 300, 2, 2, 128),
    (2, 1087, 16, 4, 128),
    (2, 1087, 16, 4, 192),
    # a grid large enough for 8-wave workgroups (33 x 32 >= 1,024 of them:
    # BF16, and FP8 at d_qk = 192), ragged: the last 256-row tile holds 77
    # rows
    (1, 8269, 32, 8, 128),
    (1, 8269, 32, 8, 192),
]


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
@pytest.mark.parametrize("shape", ZERO_Q, ids=["x".join(map(str, z)) for z in ZERO_Q])
def test_zero_query_gives_running_mean(dtype, shape):
    # Q = 0: every logit is 0, softmax weights are exactly 1/(i+1), so every
    # output element has a closed form: O[b,i,h] = mean_{j<=i} V[b,j,h/G]
    B, S, Hq, Hkv, dqk = shape
    w = Workload("zero_q", B, S, Hq, Hkv, dqk, 128, dtype, "gauss")
    q, k, v = make_inputs(w, seed=3)
    q[:] = 0
    print(f"case zero_q {dtype} B={B} S={S} Hq={Hq} Hkv={Hkv} d_qk={dqk}", flush=True)
    o, lse, ex = ops.prefill(dev(q), dev(k), dev(v), dtype)
    torch.cuda.synchronize()
    ref = prefill_reference(q, k, v, dtype, rows=[(0, 0, 0)])
    vd = np.asarray(ref["views"][2][:])  # dequantized V (float64) [B, S, Hkv, d_v]
    G = Hq // Hkv
    mean = np.cumsum(vd, axis=1) / np.arange(1, S + 1)[None, :, None, None]
    mean = np.repeat(mean, G, axis=2)  # query head h reads kv head h // G
    og = o.float().cpu().numpy()
    # bf16 output rounding (2^-9 relative) plus fp32 accumulation
    assert np.allclose(og, mean, rtol=2 ** -8, atol=1e-5 * np.abs(vd).max())
    assert np.allclose(lse.cpu().numpy(), np.log(np.arange(1, S + 1))[None, None, :], rtol=0, atol=1e-5)
    # row 0 sees key 0 only: O row 0 is V row 0 up to the bf16 rounding
    assert np.allclose(og[:, 0], np.repeat(vd[:, 0], G, axis=1), rtol=2 ** -8, atol=0)


# lse = NULL skips the LSE output only: O keeps every bit, in every kernel and
# P mode that takes an LSE
O_ONLY = [("fp8", 128, 0), ("fp8", 192, 0), ("bf16", 128, 0), ("bf16", 192, 0),
          ("fp8", 128, ops.ATTN_FLAG_P_BLOCK_SCALE),
          ("fp8", 192, ops.ATTN_FLAG_P_BLOCK_SCALE | ops.ATTN_FLAG_P_ROUNDED_SUM)]


@pytest.mark.parametrize("dtype,dqk,flags", O_ONLY, ids=[f"{t}_d{d}_flags{f}" for t, d, f in O_ONLY])
def test_output_without_lse_is_unchanged(dtype, dqk, flags):
    w = Workload("o_only", 1, 777, 4, 2, dqk, 128, dtype, "gauss")
    q, k, v = make_inputs(w, seed=9)
    print(f"case o_only {dtype} d_qk={dqk} flags={flags}", flush=True)
    o, lse, ex = ops.prefill(dev(q), dev(k), dev(v), dtype, flags=flags)
    o2, l2 = ops.attn_prefill_fwd(ex["q"], ex["k"], ex["v"], d_scales=ex["scales"], flags=flags, return_lse=False)
    torch.cuda.synchronize()
    assert l2 is None and lse is not None
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16))


def test_host_and_device_scales_agree_bitwise():
    w = Workload("scales", 1, 260, 4, 2, 128, 128, "fp8", "gauss")
    q, k, v = make_inputs(w, seed=5)
    o1, l1, ex = ops.prefill(dev(q), dev(k), dev(v), "fp8")
    sc = ex["scales"].cpu().numpy()
    o2, l2 = ops.attn_prefill_fwd(ex["q"], ex["k"], ex["v"], float(sc[0]), float(sc[1]), float(sc[2]))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_quantizer_bf16_input_and_tail():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(1000 * 37 + 5) * 3).astype(np.float32)  # length not a multiple of 8
    xb = torch.from_numpy(x).to(torch.bfloat16)
    from oracle import quantize_fp8_per_tensor
    for t in (torch.from_numpy(x), xb):
        codes, scale = ops.attn_quantize_fp8(t.to("cuda"))
        rc, rs = quantize_fp8_per_tensor(t.float().numpy())
        assert np.array_equal(codes.cpu().numpy(), rc)
        assert scale.cpu().numpy()[0] == rs
    zc, zs = ops.attn_quantize_fp8(torch.zeros(100, device="cuda"))
    assert zs.item() == 1.0 and not zc.any().item()


def test_determinism_7200_launches():
    # the pages report bit-identical outputs over 7,200 launches
    w = WORKLOADS["tiny_mha_fp8"]
    q, k, v = make_inputs(w, seed=11)
    o0, l0, ex = ops.prefill(dev(q), dev(k), dev(v), "fp8")
    o = torch.empty_like(o0)
    lse = torch.empty_like(l0)
    diff = torch.zeros((), dtype=torch.int64, device="cuda")
    for _ in range(7200):
        ops.attn_prefill_fwd(ex["q"], ex["k"], ex["v"], out=o, lse=lse, d_scales=ex["scales"])
        diff += (o.view(torch.int16) != o0.view(torch.int16)).sum() + (lse != l0).sum()
    torch.cuda.synchronize()
    assert diff.item() == 0


# ---------------------------------------------------------------- full-size workloads, sampled rows

def sample_rows(w: Workload, rng: np.random.Generator, n_heads: int = 6):
    heads = sorted(set([0, w.Hq - 1] + list(rng.choice(w.Hq, min(n_heads, w.Hq), replace=False))))
    pos = [0, 1, 63, 64, 127, 128, 255, 256, w.S // 2, w.S - 129, w.S - 128, w.S - 2, w.S - 1]
    rows = []
    for h in heads:
        extra = rng.integers(0, w.S, 3)
        for i in sorted(set([p for p in pos if 0 <= p < w.S] + list(extra))):
            rows.append((int(rng.integers(0, w.B)), int(h), int(i)))
    return rows


# BF16 and FP8 d_qk = 192 (exact P) run 8-wave workgroups (256 query rows)
# from 8,192 tokens when that grid has at least 1,024 of them, 4-wave ones
# otherwise: these lengths with 32 query heads are past the switch (33 to 34
# tiles of 256 rows per head) and put every ragged tail of a 256-row tile and
# of a key step (64 keys; 32 for BF16 d_qk = 192) through the 8-wave kernels
# (d_qk = 192: a K tile of one and a half load instructions per lane)
EIGHT_WAVE_S = [8193, 8223, 8225, 8257, 8447, 8640]
EIGHT_WAVE_KINDS = [("bf16", 128, True, "gauss"), ("bf16", 192, True, "mla"), ("fp8", 192, True, "mla"),
                    ("fp8", 192, False, "mla")]


def _sampled_rows_check(w, seed, fold_q, n_heads=4):
    q, k, v, o, lse, ex = run_case(w, seed=seed, fold_q=fold_q)
    rows = sample_rows(w, np.random.default_rng(seed), n_heads=n_heads)
    ref = prefill_reference(q, k, v, w.dtype, causal=w.causal, rows=rows, fold_q=fold_q,
                            hadamard=rot(w.dtype, fold_q))
    bi = torch.tensor([r[0] for r in rows]); hi = torch.tensor([r[1] for r in rows])
    ii = torch.tensor([r[2] for r in rows])
    og = o[bi, ii, hi].float().cpu().numpy().astype(np.float64)
    lg = lse[bi, hi, ii].cpu().numpy().astype(np.float64)
    err, _ = check_o(og, ref["o_rows"], w.dtype, f"S={w.S} {len(rows)} rows: ")
    lerr = float(np.max(np.abs(lg - ref["lse_rows"])))
    print(f"  LSE max-abs {lerr:.3e}", flush=True)
    assert lerr <= LSE_TOL, (w.S, lerr)
    o2, l2 = ops.attn_prefill_fwd(ex["q"], ex["k"], ex["v"], causal=w.causal, d_scales=ex["scales"])
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16)) and torch.equal(l2, lse)
    return rows, err, lerr


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("dtype,dqk,fold_q,dist", EIGHT_WAVE_KINDS,
                         ids=[f"{t}_d{d}" + ("" if f else "_plain_q") for t, d, f, _ in EIGHT_WAVE_KINDS])
def test_eight_wave_workgroups_sampled_rows(dtype, dqk, fold_q, dist, causal):
    worst = (0.0, 0.0)
    for S in EIGHT_WAVE_S if causal else EIGHT_WAVE_S[-1:]:
        w = Workload(f"{dtype}_d{dqk}_w8_{S}", 1, S, 32, 8, dqk, 128, dtype, dist, causal=causal)
        assert S >= 8192 and w.B * w.Hq * -(-S // 256) >= 1024
        _, err, lerr = _sampled_rows_check(w, S, fold_q)
        worst = (max(worst[0], err), max(worst[1], lerr))
    print(f"  worst: O rel-L2 {worst[0]:.3e}  LSE max-abs {worst[1]:.3e}", flush=True)


# the 8-wave kernels under both work orders: two sequences with B * Hkv = 8
# (whole kv units per XCD) and G = 6 query heads per kv head with B * Hkv = 6
# (plain tile-major order)
EIGHT_WAVE_ORDERS = [Workload("bf16_w8_batch2_xcd_order", 2, 8200, 16, 4, 128, 128, "bf16", "gauss"),
                     Workload("bf16_w8_group6_plain_order", 1, 8300, 36, 6, 128, 128, "bf16", "outlier"),
                     Workload("bf16_mla_w8_batch2_xcd_order", 2, 8200, 16, 4, 192, 128, "bf16", "mla"),
                     Workload("fp8_mla_w8_batch2_xcd_order", 2, 8200, 16, 4, 192, 128, "fp8", "mla"),
                     Workload("fp8_mla_w8_group6_plain_order", 1, 8300, 36, 6, 192, 128, "fp8", "mla")]


@pytest.mark.parametrize("w", EIGHT_WAVE_ORDERS, ids=[w.name for w in EIGHT_WAVE_ORDERS])
def test_eight_wave_work_orders_sampled_rows(w):
    assert w.S >= 8192 and w.B * w.Hq * -(-w.S // 256) >= 1024
    rows, _, _ = _sampled_rows_check(w, w.S, True)
    assert len({r[0] for r in rows}) == w.B


# seeded random shapes past the 8-wave switch: batch 1-2, 1-8 kv heads with
# 1-8 query heads each, 8,192-9,299 tokens (any ragged tail), causal or not,
# through every 8-wave kernel
def _eight_wave_draw(n: int, seed: int = 31):
    rng = np.random.default_rng(seed)
    kinds = [("bf16", 128, True, "gauss"), ("bf16", 128, True, "outlier"), ("bf16", 192, True, "mla"),
             ("fp8", 192, True, "mla"), ("fp8", 192, False, "mla")]
    cases = []
    for i in range(n):
        dtype, dqk, fold_q, dist = kinds[int(rng.integers(len(kinds)))]
        while True:
            B, Hkv = int(rng.integers(1, 3)), int(rng.integers(1, 9))
            G, S = int(rng.choice([1, 2, 3, 4, 6, 8])), int(rng.integers(8192, 9300))
            if B * G * Hkv * -(-S // 256) >= 1024 and B * G * Hkv <= 64:
                break
        causal = bool(rng.random() < 0.8)
        w = Workload(f"w8rand{i}_{dtype}_d{dqk}_B{B}_S{S}_G{G}x{Hkv}", B, S, G * Hkv, Hkv, dqk, 128, dtype, dist,
                     causal=causal)
        cases.append((w, fold_q, 5000 + i))
    return cases


EIGHT_WAVE_RANDOM = _eight_wave_draw(12)


@pytest.mark.parametrize("case", EIGHT_WAVE_RANDOM,
                         ids=[c[0].name + ("" if c[0].causal else "_noncausal") + ("" if c[1] else "_plain_q")
                              for c in EIGHT_WAVE_RANDOM])
def test_eight_wave_random_shapes_sampled_rows(case):
    w, fold_q, seed = case
    assert w.S >= 8192 and w.B * w.Hq * -(-w.S // 256) >= 1024
    _sampled_rows_check(w, seed, fold_q, n_heads=3)


# every workload with the pipeline's folded query scale; the FP8 layers also
# with the plain per-tensor absmax scale of the configs (the kernel's fma form)
FULL_RUNS = [(n, True) for n in WORKLOADS] + [(n, False) for n in WORKLOADS
                                              if WORKLOADS[n].dtype == "fp8" and n != "tiny_mha_fp8"]


@pytest.mark.parametrize("name,fold_q", FULL_RUNS, ids=[n + ("" if f else "_plain_q") for n, f in FULL_RUNS])
def test_full_size_sampled_rows(name, fold_q):
    w = WORKLOADS[name]
    q, k, v, o, lse, ex = run_case(w, seed=0, fold_q=fold_q)
    rng = np.random.default_rng(12345)
    rows = sample_rows(w, rng)
    ref = prefill_reference(q, k, v, w.dtype, rows=rows, fold_q=fold_q, hadamard=rot(w.dtype, fold_q))
    if w.dtype == "fp8":
        sc = ex["scales"].cpu().numpy()
        assert np.array_equal(sc, np.float32([ref["q_scale"], ref["k_scale"], ref["v_scale"]]))
    # codes of the sampled heads' slices, bit-exact
    heads = sorted(set(h for _, h, _ in rows))
    G = w.Hq // w.Hkv
    for h in heads[:3]:
        assert np.array_equal(codes_np(ex["q"][0, :, h]), ref["views"][0].codes((0, slice(None), h)))
        assert np.array_equal(codes_np(ex["k"][0, :, h // G]), ref["views"][1].codes((0, slice(None), h // G)))
        assert np.array_equal(codes_np(ex["v"][0, :, h // G]), ref["views"][2].codes((0, slice(None), h // G)))
    bi = torch.tensor([r[0] for r in rows]); hi = torch.tensor([r[1] for r in rows])
    ii = torch.tensor([r[2] for r in rows])
    og = o[bi, ii, hi].float().cpu().numpy().astype(np.float64)
    lg = lse[bi, hi, ii].cpu().numpy().astype(np.float64)
    check_o(og, ref["o_rows"], w.dtype, f"{len(rows)} rows: ")
    lerr = float(np.max(np.abs(lg - ref["lse_rows"])))
    print(f"  LSE max-abs {lerr:.3e}", flush=True)
    assert lerr <= LSE_TOL
    # 50 more launches of the attention kernel alone are bit-identical
    h0 = hashlib.sha256(o.view(torch.int16).cpu().numpy().tobytes() + lse.cpu().numpy().tobytes()).hexdigest()
    o2 = torch.empty_like(o); l2 = torch.empty_like(lse)
    bad = torch.zeros((), dtype=torch.int64, device="cuda")
    for _ in range(50):
        ops.attn_prefill_fwd(ex["q"], ex["k"], ex["v"], out=o2, lse=l2, d_scales=ex["scales"])
        bad += (o2.view(torch.int16) != o.view(torch.int16)).sum() + (l2 != lse).sum()
    torch.cuda.synchronize()
    assert bad.item() == 0, h0


# ---------------------------------------------------------------- tile-boundary sweep and exact-path stress

BOUNDARY_S = [63, 64, 65, 127, 128, 129, 191, 192, 193, 255, 256, 257, 320, 449,
              # the main loop's unchecked part (whole iterations of full tiles
              # inside the sequence) starts at 9 full 64-key tiles: these run 0, 1
              # and 2 such iterations with every length of the checked remainder
              511, 512, 513, 575, 576, 577, 640, 705, 769, 831, 1024, 1087]


@pytest.mark.parametrize("dtype,fold_q", [("fp8", True), ("fp8", False), ("bf16", True)],
                         ids=["fp8", "fp8_plain_q", "bf16"])
def test_sequence_lengths_around_tile_boundaries(dtype, fold_q):
    # 64-key steps, 128-row workgroups, a main loop unrolled by the ring depth
    # (4): these lengths give every tile count mod 4 and every ragged tail, in
    # both parts of the main loop
    worst = (0.0, 0.0, 0.0)
    for S in BOUNDARY_S:
        w = Workload(f"boundary_{S}", 1, S, 4, 2, 128, 128, dtype, "gauss")
        q, k, v, o, lse, ex = run_case(w, seed=S, fold_q=fold_q)
        ref = prefill_reference(q, k, v, dtype, fold_q=fold_q, hadamard=rot(dtype, fold_q))
        err, row = check_o(o.float().cpu().numpy().astype(np.float64), ref["o"], dtype, f"S={S}: ")
        lerr = float(np.max(np.abs(lse.cpu().numpy().astype(np.float64) - ref["lse"])))
        worst = (max(worst[0], err), max(worst[1], row), max(worst[2], lerr))
        assert lerr <= LSE_TOL, (S, lerr)
    print(f"  worst over {len(BOUNDARY_S)} lengths: O rel-L2 {worst[0]:.3e}  row {worst[1]:.3e}  "
          f"LSE max-abs {worst[2]:.3e}", flush=True)


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_noncausal_through_the_unchecked_loop(dtype):
    # non-causal rows walk every key tile, so these lengths also run the main
    # loop's unchecked part, then a ragged checked remainder
    for S in (577, 705, 1087):
        w = Workload(f"noncausal_{S}", 1, S, 4, 2, 128, 128, dtype, "gauss", causal=False)
        q, k, v, o, lse, ex = run_case(w, seed=S)
        ref = prefill_reference(q, k, v, dtype, causal=False, fold_q=True, hadamard=rot(dtype, True))
        check_o(o.float().cpu().numpy().astype(np.float64), ref["o"], dtype, f"S={S}: ")
        lerr = float(np.max(np.abs(lse.cpu().numpy().astype(np.float64) - ref["lse"])))
        print(f"  S={S}: LSE max-abs {lerr:.3e}", flush=True)
        assert lerr <= LSE_TOL, (S, lerr)


RISING = [("fp8", 128, True), ("fp8", 128, False), ("bf16", 128, True),
          ("fp8", 192, True), ("fp8", 192, False), ("bf16", 192, True)]


@pytest.mark.parametrize("dtype,dqk,fold_q", RISING,
                         ids=[f"{t}_d{d}" + ("" if f else "_plain_q") for t, d, f in RISING])
def test_running_max_grows_every_tile(dtype, dqk, fold_q):
    # scores rise with the key index (k_j = (0.5 + 2j/S) * u, q_i = 4 u for a
    # random unit-scale u), so each new tile holds the row's largest score
    # and the exact-maximum path (running-max update, O and l rescale) runs
    # on nearly every step
    S, H = 700, 2
    rng = np.random.default_rng(21)
    u = rng.standard_normal(dqk).astype(np.float32)
    u /= np.float32(np.linalg.norm(u) / np.sqrt(128))
    ramp = (0.5 + 2.0 * np.arange(S, dtype=np.float32) / S)[None, :, None, None]
    k = np.ascontiguousarray(np.broadcast_to(ramp * u, (1, S, H, dqk))).astype(np.float32)
    k += 0.05 * rng.standard_normal(k.shape).astype(np.float32)
    q = np.ascontiguousarray(np.broadcast_to(4.0 * u, (1, S, H, dqk))).astype(np.float32)
    v = rng.standard_normal((1, S, H, 128)).astype(np.float32)
    print(f"case rising scores {dtype} S={S} d_qk={dqk} fold_q={fold_q}", flush=True)
    o, lse, ex = ops.prefill(dev(q), dev(k), dev(v), dtype, fold_q=fold_q)
    torch.cuda.synchronize()
    ref = prefill_reference(q, k, v, dtype, fold_q=fold_q, hadamard=rot(dtype, fold_q))
    check_o(o.float().cpu().numpy().astype(np.float64), ref["o"], dtype)
    lerr = float(np.max(np.abs(lse.cpu().numpy().astype(np.float64) - ref["lse"])))
    print(f"  LSE max-abs {lerr:.3e}", flush=True)
    assert lerr <= LSE_TOL
    o2, l2 = ops.attn_prefill_fwd(ex["q"], ex["k"], ex["v"], d_scales=ex["scales"] if dtype == "fp8" else None)
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16)) and torch.equal(l2, lse)


def test_long_context_64k_sampled_rows():
    # twice the pages' longest context: 1,024 key tiles and 512 query tiles per
    # head, past every 32-bit product of the 32K shape
    w = Workload("long_64k_fp8", 1, 65536, 8, 8, 128, 128, "fp8", "gauss")
    q, k, v, o, lse, ex = run_case(w, seed=5)
    rng = np.random.default_rng(64)
    rows = [(0, int(h), int(i)) for h in (0, 7) for i in sorted(set([0, 1, 32767, 32768, 65534, 65535]
                                                                     + list(rng.integers(0, w.S, 4))))]
    ref = prefill_reference(q, k, v, "fp8", rows=rows, fold_q=True, hadamard=True)
    sc = ex["scales"].cpu().numpy()
    assert np.array_equal(sc, np.float32([ref["q_scale"], ref["k_scale"], ref["v_scale"]]))
    bi = torch.tensor([r[0] for r in rows]); hi = torch.tensor([r[1] for r in rows])
    ii = torch.tensor([r[2] for r in rows])
    og = o[bi, ii, hi].float().cpu().numpy().astype(np.float64)
    lg = lse[bi, hi, ii].cpu().numpy().astype(np.float64)
    check_o(og, ref["o_rows"], "fp8", f"{len(rows)} rows: ")
    lerr = float(np.max(np.abs(lg - ref["lse_rows"])))
    print(f"  LSE max-abs {lerr:.3e}", flush=True)
    assert lerr <= LSE_TOL


@pytest.mark.parametrize("xdt", [torch.float32, torch.bfloat16])
def test_fused_input_step_matches_separate_calls(xdt):
    # one absmax and one encode launch over Q, K, V give the codes and scales
    # of three separate calls (K, V plain; Q folded with K's scale); MLA-like
    # shapes (K and V of different sizes), lengths that are not a multiple of
    # the 16-byte vector, an all-zero Q, and a one-element V
    rng = np.random.default_rng(31)
    cases = [((1, 333, 4, 192), (1, 333, 4, 192), (1, 333, 4, 128)),
             ((1, 1000 * 37 + 5,), (2, 3, 1, 7), (1, 1, 1, 1)),
             ((1, 65, 8, 128), (1, 65, 2, 128), (1, 65, 2, 128))]
    for n, (sq, sk, sv) in enumerate(cases):
        xs = [torch.from_numpy((rng.standard_normal(sh) * (1 + 3 * i)).astype(np.float32)).to("cuda").to(xdt)
              for i, sh in enumerate((sq, sk, sv))]
        if n == 2:
            xs[0].zero_()
        print(f"case fused input step {xdt} shapes {sq} {sk} {sv}", flush=True)
        sm = 1.0 / math.sqrt(sq[-1])
        (q8, k8, v8), sc = ops.attn_quantize_fp8_qkv(*xs, sm)
        k8s, ks = ops.attn_quantize_fp8(xs[1])
        v8s, vs = ops.attn_quantize_fp8(xs[2])
        q8s, qs = ops.attn_quantize_fp8(xs[0], k_scale=ks, softmax_scale=sm)
        torch.cuda.synchronize()
        assert torch.equal(q8, q8s) and torch.equal(k8, k8s) and torch.equal(v8, v8s)
        assert torch.equal(sc, torch.cat([qs, ks, vs]))
