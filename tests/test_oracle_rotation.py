"""Pins of the oracle's Hadamard rotation (oracle/rotation.py), CPU only.

Source: aicronaca.it, section "Perché l'FP8 non basta da solo" (a Hadamard
rotation of Q and K about halves the FP8 input quantization error). What pins
the module, none of which re-types its formulas:

* scipy.linalg.hadamard (a library routine) and the closed form
  H[i, j] = (-1)^popcount(i & j) for the matrices;
* H H^T = m I, and score invariance (q H)(k H)^T = b q.k^T;
* a pure-Python brute force with math.fsum for the rotated rows;
* a one-hot vector, whose rotation is a signed row of H (worked by hand);
* the folded-scale property: the stored query scale times k_scale,
  softmax_scale and log2(e) is a power of two;
* the page's claim itself: on heavy-tailed inputs whose large channels Q
  and K share, the end-to-end error against fp64 attention on the
  unquantized inputs drops to about half or less.

Each pin function takes the module, so the mutation tests at the end can run
the same pins against planted mistakes.
"""

import inspect
import math
import types

import numpy as np
import pytest
import scipy.linalg

import oracle.rotation as rot_mod
from oracle import causal_attention, dequantize_fp8, e4m3fn_decode, encode_with_scale, per_tensor_scale, \
    per_tensor_scale_folded
from bf16_causal_prefill_fwd_amd.workloads import make_inputs

LOG2E = 1.4426950408889634


def _brute_rotate(x, b):
    """y[.., blk*b + j] = sum_i x[.., blk*b + i] * (-1)^popcount(i & j), by math.fsum."""
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1, x.shape[-1])
    out = np.empty_like(flat)
    for r in range(flat.shape[0]):
        for blk in range(flat.shape[1] // b):
            for j in range(b):
                out[r, blk * b + j] = math.fsum(
                    flat[r, blk * b + i] * (-1.0 if bin(i & j).count("1") & 1 else 1.0) for i in range(b))
    return out.reshape(x.shape)


def pin_matrices(mod):
    for m in (1, 2, 4, 8, 16, 32, 64, 128):
        h = mod.sylvester_hadamard(m)
        assert np.array_equal(h, scipy.linalg.hadamard(m))
        assert np.array_equal(h @ h.T, m * np.eye(m, dtype=np.int64))
    h = mod.sylvester_hadamard(128)
    i, j = np.meshgrid(np.arange(128), np.arange(128), indexing="ij")
    parity = np.vectorize(lambda a: bin(a).count("1") & 1)(i & j)
    assert np.array_equal(h, np.where(parity == 1, -1, 1))
    assert [mod.hadamard_block(d) for d in (128, 192, 64, 96, 256, 1)] == [128, 64, 64, 32, 128, 1]


def pin_rotation(mod):
    rng = np.random.default_rng(7)
    for d in (128, 192):
        x = rng.standard_normal((3, d)).astype(np.float32)
        y = mod.rotate_rows(x)
        yb = _brute_rotate(x, 128 if d == 128 else 64)
        assert np.allclose(y, yb, rtol=0, atol=1e-12 * np.abs(yb).max())
        # scores only scale by the block size
        q = rng.standard_normal((5, d)); k = rng.standard_normal((7, d))
        b = 128 if d == 128 else 64
        s_rot = mod.rotate_rows(q) @ mod.rotate_rows(k).T
        assert np.allclose(s_rot, b * (q @ k.T), rtol=1e-12, atol=1e-10)


def pin_one_hot(mod):
    # x = 5 e_3 (d = 128): y = 5 * row 3 of H = +-5, absmax 5, plain scale fp32(5/448),
    # every code +-448 (0x7E / 0xFE) with the signs of row 3: (-1)^popcount(3 & j)
    x = np.zeros((1, 1, 1, 128), dtype=np.float32)
    x[0, 0, 0, 3] = 5.0
    codes, scale = mod.hadamard_quantize(x)
    assert scale == np.float32(np.float32(5.0) / np.float32(448.0))
    signs = np.array([bin(3 & j).count("1") & 1 for j in range(128)])
    assert np.array_equal(codes.reshape(-1), np.where(signs == 1, 0xFE, 0x7E).astype(np.uint8))
    # all-zero tensor: scale 1.0, all codes 0, as in the unrotated quantizer
    z = np.zeros((2, 3, 1, 192), dtype=np.float32)
    codes, scale = mod.hadamard_quantize(z)
    assert scale == np.float32(1.0) and not codes.any()


def pin_scales(mod):
    rng = np.random.default_rng(11)
    for d in (128, 192):
        b = 128 if d == 128 else 64
        q = rng.standard_normal((1, 33, 2, d)).astype(np.float32)
        k = rng.standard_normal((1, 33, 1, d)).astype(np.float32)
        sm = 1.0 / math.sqrt(d)
        kc, ks = mod.hadamard_quantize(k)
        # key: plain absmax/448 of the rotated tensor (absmax from the brute force)
        a = np.float32(np.abs(_brute_rotate(k, b)).max())
        assert ks == np.float32(a / np.float32(448.0))
        qc, qs = mod.hadamard_quantize(q, k_scale=ks, softmax_scale=sm)
        # folded: code scale * ks * sm * log2e a power of two, within absmax/448 .. 2x;
        # the stored scale is the code scale / b
        code_scale = np.float32(float(qs) * b)
        c = float(code_scale) * float(ks) * sm * LOG2E
        f, _ = math.frexp(c)
        assert abs(f - 0.5) < 1e-6 or abs(f - 1.0) < 1e-6
        aq = float(np.abs(_brute_rotate(q, b)).max())
        assert aq / 448.0 <= float(code_scale) * (1 + 1e-6) and float(code_scale) <= 2 * aq / 448.0 * (1 + 1e-6)
        # dequantized products approximate the unrotated q.k (input quantization error only)
        qd = dequantize_fp8(qc, qs).reshape(-1, d); kd = dequantize_fp8(kc, ks).reshape(-1, d)
        s_true = q.reshape(-1, d).astype(np.float64) @ k.reshape(-1, d).astype(np.float64).T
        err = np.linalg.norm(qd @ kd.T - s_true) / np.linalg.norm(s_true)
        assert err < 0.08
        # codes: y * (1/code_scale) in float64, to float32, then the nearest e4m3
        # value (ties to even), read off the format's value table on the
        # brute-force rotation
        y = _brute_rotate(q, b)
        t = (y * (1.0 / float(code_scale))).astype(np.float32).astype(np.float64)
        assert np.array_equal(qc, _nearest_code(t))


def _nearest_code(t):
    """Nearest e4m3fn code by exhaustive search over the 254 finite codes, ties to even mantissa."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = e4m3fn_decode(codes)
    flat = t.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for n, x in enumerate(flat):
        d = np.abs(vals - x)
        pick = list(codes[np.flatnonzero(d == d.min())])
        if len(pick) > 1:
            # ties: the even code (last mantissa bit clear); +0 / -0 follow the sign of x
            pick = [c for c in pick if (c & 1) == 0]
        if len(pick) > 1:
            pick = [c for c in pick if bool(c & 0x80) == bool(np.signbit(x))]
        out[n] = pick[0]
    return out.reshape(t.shape)


def pin_halves_error(mod):
    # the page's claim, on heavy-tailed inputs whose 4 large channels (x8) are
    # shared by Q and K (with independent channels an FP8 cast gains nothing:
    # its relative rounding error does not depend on the per-tensor scale)
    q, k, v = make_inputs("gqa_fp8_outlier_16k", seed=3, S=384, Hq=4, Hkv=2, dist="outlier_shared")
    sm = 1.0 / math.sqrt(128)
    O, _ = causal_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64))
    ks, vs = per_tensor_scale(k), per_tensor_scale(v)
    qs = per_tensor_scale_folded(q, ks, sm)
    vd = dequantize_fp8(encode_with_scale(v, vs), vs)
    O1, _ = causal_attention(dequantize_fp8(encode_with_scale(q, qs), qs),
                             dequantize_fp8(encode_with_scale(k, ks), ks), vd)
    kc, ks2 = mod.hadamard_quantize(k)
    qc, qs2 = mod.hadamard_quantize(q, k_scale=ks2, softmax_scale=sm)
    O2, _ = causal_attention(dequantize_fp8(qc, qs2), dequantize_fp8(kc, ks2), vd)
    e1 = np.linalg.norm(O1 - O) / np.linalg.norm(O)
    e2 = np.linalg.norm(O2 - O) / np.linalg.norm(O)
    assert e2 < 0.6 * e1, (e1, e2)


PINS = [pin_matrices, pin_rotation, pin_one_hot, pin_scales, pin_halves_error]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(rot_mod)


# ---- planted mistakes: each must break at least one pin
MUTANTS = {
    "sign_flip_block": ("h = np.block([[h, h], [h, -h]])", "h = np.block([[h, -h], [h, h]])"),
    "block_always_128": ("return min(d & -d, 128)", "return 128 if d % 128 == 0 else 64 if d % 64 == 0 else d & -d and 128"),
    "block_not_capped": ("return min(d & -d, 128)", "return d & -d"),
    "no_query_division": ("return s, np.float32(float(s) / b)", "return s, s"),
    "transposed_blocks": ("return (blocks @ h).reshape(x.shape)", "return (blocks @ h.T[::-1]).reshape(x.shape)"),
    "absmax_unrotated": ("y = rotate_rows(flat[r0:r0 + chunk_rows])", "y = np.asarray(flat[r0:r0 + chunk_rows], np.float64)"),
    "encode_unrotated": ("y = rotate_rows(x)\n    r = 1.0", "y = np.asarray(x, np.float64)\n    r = 1.0"),
    "encode_divides_by_b": ("r = 1.0 / float(np.float32(code_scale))", "r = 1.0 / float(np.float32(code_scale)) / 2"),
    "plain_scale_for_query": ("return per_tensor_scale_folded(one, k_scale, softmax_scale)", "return per_tensor_scale(one)"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = inspect.getsource(rot_mod)
    assert src.count(old) == 1, name
    mod = types.ModuleType("oracle._rot_mutant_" + name)
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "<mutant %s>" % name, "exec"), mod.__dict__)
    return mod


def _all_pins_pass(mod) -> bool:
    for pin in PINS:
        try:
            pin(mod)
        except Exception:
            return False
    return True


def test_unmutated_copy_passes():
    src = inspect.getsource(rot_mod)
    mod = types.ModuleType("oracle._rot_identity")
    mod.__package__ = "oracle"
    exec(compile(src, "<identity>", "exec"), mod.__dict__)
    assert _all_pins_pass(mod)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_caught(name):
    assert not _all_pins_pass(_mutant(name)), name


def test_prefill_reference_rotated_views():
    # the whole-path reference with the rotation: the same codes and scales as
    # hadamard_quantize, and selected rows equal to the full computation
    q, k, v = make_inputs("gqa_fp8_outlier_16k", seed=0, S=300, Hq=4, Hkv=2, dist="outlier_shared")
    from oracle import prefill_reference
    r = prefill_reference(q, k, v, "fp8", hadamard=True)
    kc, ks = rot_mod.hadamard_quantize(k)
    qc, qs = rot_mod.hadamard_quantize(q, k_scale=ks, softmax_scale=1.0 / math.sqrt(128))
    assert np.array_equal(r["q_codes"], qc) and np.array_equal(r["k_codes"], kc)
    assert r["q_scale"] == qs and r["k_scale"] == ks
    rows = [(0, 1, 5), (0, 3, 299), (0, 0, 0)]
    rr = prefill_reference(q, k, v, "fp8", hadamard=True, rows=rows)
    for n, (b, h, i) in enumerate(rows):
        assert np.allclose(rr["o_rows"][n], r["o"][b, i, h], rtol=0, atol=1e-13)
        assert abs(rr["lse_rows"][n] - r["lse"][b, h, i]) < 1e-12
    with pytest.raises(ValueError):
        prefill_reference(q, k, v, "bf16", hadamard=True)
