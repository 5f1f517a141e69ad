"""Seeded synthetic inputs for the causal prefill attention workloads.

This module only draws random numbers: it holds none of the attention or
quantization arithmetic, so the HIP path and the CPU oracle can both consume
its output. Every tensor is float32 in the flash_attn_func layout
[B, S, H, d].

Distributions:

* ``gauss``   -- Q, K, V ~ N(0, 1).
* ``outlier`` -- V ~ N(0, 1); Q and K ~ N(0, 1) with 4 channels per head
  multiplied by 8. The 4 channels are drawn independently for each tensor
  and each head. This stands in for the captured Mistral-7B / Qwen3-8B
  layers the pages measure on, whose weights are not available.
* ``outlier_shared`` -- as ``outlier``, but the 4 channels are drawn once per
  kv head and scaled in K's head and in each query head of its group, so
  the large channels of Q and K coincide, as in real activations whose
  outlier features sit in fixed channels. Then a few products dominate each
  score. This is the case a Hadamard rotation of Q and K is for.
* ``mla``     -- V ~ N(0, 1); Q and K ~ N(0, 1) on the 128 no-rope dims and
  N(0, 2) (std sqrt 2) on dims 128..191, the rope part of the
  DeepSeek-V2-Lite-shaped 192/128 head.

Generator: numpy PCG64 via ``default_rng([seed, tensor_index])``, tensor
index 0/1/2 for Q/K/V; outlier channels come from the same generator after
the tensor's values (``outlier``) or, shared, from ``default_rng([seed, 3])``
with one draw per kv head (``outlier_shared``).
"""

from __future__ import annotations

from dataclasses import dataclass, asdict

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S: int
    Hq: int
    Hkv: int
    d_qk: int
    d_v: int
    dtype: str        # "fp8" or "bf16"
    dist: str         # "gauss", "outlier", "outlier_shared" or "mla"
    causal: bool = True

    def as_dict(self):
        return asdict(self)

    @property
    def causal_flops(self) -> float:
        """Algorithmic causal FLOPs: 2 matmuls over the causal half.

        2 * B * Hq * (S^2 / 2) * (d_qk + d_v) = B * Hq * S^2 * (d_qk + d_v).
        """
        return float(self.B) * self.Hq * float(self.S) ** 2 * (self.d_qk + self.d_v)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_mha_fp8", B=1, S=512, Hq=2, Hkv=2, d_qk=128, d_v=128, dtype="fp8", dist="gauss"),
        Workload("gqa_fp8_outlier_16k", B=1, S=16384, Hq=32, Hkv=8, d_qk=128, d_v=128, dtype="fp8",
                 dist="outlier"),
        Workload("gqa_bf16_16k", B=1, S=16384, Hq=32, Hkv=8, d_qk=128, d_v=128, dtype="bf16", dist="gauss"),
        Workload("mha_fp8_32k", B=1, S=32768, Hq=32, Hkv=32, d_qk=128, d_v=128, dtype="fp8", dist="gauss"),
        Workload("mla_fp8_16k", B=1, S=16384, Hq=16, Hkv=16, d_qk=192, d_v=128, dtype="fp8", dist="mla"),
    ]
}


def _draw(seed: int, index: int, shape, dist: str, role: str) -> np.ndarray:
    rng = np.random.default_rng([seed, index])
    x = rng.standard_normal(shape, dtype=np.float32)
    if dist == "outlier" and role in ("q", "k"):
        d = shape[3]
        for h in range(shape[2]):
            ch = rng.choice(d, 4, replace=False)
            x[:, :, h, ch] *= np.float32(8.0)
    elif dist == "mla" and role in ("q", "k"):
        if shape[3] > 128:
            x[:, :, :, 128:] *= np.float32(np.sqrt(2.0))
    return x


def make_inputs(w: Workload | str, seed: int = 0, **overrides):
    """Draw (q, k, v) float32 arrays for a workload (fields may be overridden)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    if overrides:
        w = Workload(**{**w.as_dict(), **overrides})
    q = _draw(seed, 0, (w.B, w.S, w.Hq, w.d_qk), w.dist, "q")
    k = _draw(seed, 1, (w.B, w.S, w.Hkv, w.d_qk), w.dist, "k")
    v = _draw(seed, 2, (w.B, w.S, w.Hkv, w.d_v), w.dist, "v")
    if w.dist == "outlier_shared":
        rng = np.random.default_rng([seed, 3])
        G = w.Hq // w.Hkv
        for g in range(w.Hkv):
            ch = rng.choice(w.d_qk, 4, replace=False)
            k[:, :, g, ch] *= np.float32(8.0)
            for h in range(g * G, (g + 1) * G):
                q[:, :, h, ch] *= np.float32(8.0)
    return q, k, v
