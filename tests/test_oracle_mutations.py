"""Plant plausible mistakes in the oracle (on the CPU) and check the pins catch them.

Each mutant is the oracle's attention module with one textual change (a
dropped term, a wrong sign or index, an off-by-one mask, a swapped operand).
The pins are re-run against the mutant; at least one must fail.
"""

import inspect
import math
import types

import numpy as np
import pytest
from scipy.special import softmax as scipy_softmax

import oracle.attention as attn_mod
from tests.test_oracle import brute_force

MUTANTS = {
    "scale_1_over_d": ("1.0 / math.sqrt(dqk) if softmax_scale is None", "1.0 / dqk if softmax_scale is None"),
    "mask_hides_diagonal": ("ends = rows + 1 if causal", "ends = rows if causal"),
    "mask_shows_next_key": ("ends = rows + 1 if causal", "ends = np.minimum(rows + 2, S) if causal"),
    "exp_sign_flipped": ("p = np.exp(s - m[:, None])", "p = np.exp(m[:, None] - s)"),
    "lse_drops_max": ("return o, m + np.log(l)", "return o, np.log(l)"),
    "lse_log2": ("return o, m + np.log(l)", "return o, m + np.log2(l)"),
    "no_normalisation": ("o = (p @ V[:n]) / l[:, None]", "o = (p @ V[:n])"),
    "gqa_modulo_mapping": ("g = h // G\n            K = np.ascontiguousarray", "g = h % Hkv\n            K = np.ascontiguousarray"),
    "k_used_for_v": ("o = (p @ V[:n])", "o = (p @ K[:n, :V.shape[1]])"),
    "transposed_logits": ("s = (qrows @ K[:n].T) * scale", "s = (K[:n] @ qrows.T).T[:, ::-1] * scale"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = inspect.getsource(attn_mod)
    assert src.count(old) >= 1, name
    src = src.replace(old, new)
    mod = types.ModuleType("oracle._mutant_" + name)
    mod.__package__ = "oracle"
    exec(compile(src, "<mutant %s>" % name, "exec"), mod.__dict__)
    return mod


def _pins_pass(mod) -> bool:
    try:
        rng = np.random.default_rng(1)
        q = rng.standard_normal((1, 17, 4, 16)); k = rng.standard_normal((1, 17, 2, 16))
        v = rng.standard_normal((1, 17, 2, 8))
        O, L = mod.causal_attention(q, k, v)
        Ob, Lb = brute_force(q, k, v)
        if not (np.allclose(O, Ob, atol=1e-12) and np.allclose(L, Lb, atol=1e-12)):
            return False
        # hand-worked two rows
        q = np.zeros((1, 2, 1, 4)); k = np.zeros((1, 2, 1, 4)); v = np.zeros((1, 2, 1, 4))
        q[0, 1, 0, 0] = 2.0; k[0, 0, 0, 0] = 1.0
        v[0, 0, 0] = [1.0, 0.0, 3.0, -1.0]; v[0, 1, 0] = [0.0, 1.0, 5.0, 1.0]
        O, L = mod.causal_attention(q, k, v)
        e = math.e
        if abs(L[0, 0, 1] - math.log(1 + e)) > 1e-14:
            return False
        if not np.allclose(O[0, 1, 0], (e * v[0, 0, 0] + v[0, 1, 0]) / (e + 1), atol=1e-14):
            return False
        # unmasked rows vs scipy softmax
        q = rng.standard_normal((1, 12, 1, 16)); k = rng.standard_normal((1, 12, 1, 16))
        v = rng.standard_normal((1, 12, 1, 8))
        On, _ = mod.causal_attention(q, k, v, causal=False)
        P = scipy_softmax(q[0, :, 0] @ k[0, :, 0].T / 4.0, axis=1)
        return bool(np.allclose(On[0, :, 0], P @ v[0, :, 0], atol=1e-13))
    except Exception:
        return False


def test_unmutated_oracle_passes_pins():
    assert _pins_pass(attn_mod)
    assert _pins_pass(_identity())


def _identity():
    src = inspect.getsource(attn_mod)
    mod = types.ModuleType("oracle._mutant_identity")
    mod.__package__ = "oracle"
    exec(compile(src, "<identity>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    assert not _pins_pass(_mutant(name)), f"mutant {name} survived the pins"


# ----------------------------------------------------------------- folded query scale

import oracle.formats as fmt_mod
from tests.test_oracle import test_folded_scale_by_search_and_bounds

FOLD_MUTANTS = {
    "rounds_down": ("j = e - 1 if f == 0.5 else e", "j = e - 1"),
    "drops_log2e": ("np.float64(np.float32(softmax_scale))) * LOG2E",
                    "np.float64(np.float32(softmax_scale)))"),
    "natural_log_base": ("np.float64(np.float32(softmax_scale))) * LOG2E",
                         "np.float64(np.float32(softmax_scale))) / LOG2E"),
    "half_range": ("t = (amax / E4M3_MAX) * g", "t = (amax / (E4M3_MAX / 2)) * g"),
    "plain_scale_kept": ("return np.float32(math.ldexp(1.0, j) / g)", "return np.float32(amax / E4M3_MAX)"),
}


@pytest.mark.parametrize("name", sorted(FOLD_MUTANTS))
def test_pins_catch_folded_scale_mutant(name, monkeypatch):
    old, new = FOLD_MUTANTS[name]
    src = inspect.getsource(fmt_mod)
    assert src.count(old) == 1, name
    mod = types.ModuleType("oracle._fold_mutant_" + name)
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "<mutant %s>" % name, "exec"), mod.__dict__)
    import tests.test_oracle as pins
    monkeypatch.setattr(pins, "per_tensor_scale_folded", mod.per_tensor_scale_folded)
    with pytest.raises(AssertionError):
        test_folded_scale_by_search_and_bounds()
