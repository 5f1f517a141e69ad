"""CPU fp64 oracle for the causal prefill attention forward pass.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library (no kernels, headers, tables or helpers), and it does not import the
product package.

Sources (the three news pages on Zyphra's ZYFA kernels, cited by site and
section):

* Le Fil IA (lefilia.fr), "Zyphra ZYFA : FlashAttention en FP8 pour l'AMD
  MI355X" -- summary paragraph (causal prefill forward, FP8 and BF16, head dim
  128 and the MLA 192/128 shape) and the context paragraph (e4m3 codes grow by
  8 per doubling; only QK^T and PV are matrix products, the softmax runs on
  the vector unit).
* aicronaca.it, sections "Che cosa ha annunciato Zyphra" (causal prefill,
  flash_attn_func drop-in) and "Perché l'FP8 non basta da solo".
* ai4bro.com, section "TL;DR" (causal forward prefill attention in FP8 e4m3
  and BF16).

Modules:

* ``formats``   -- OCP e4m3fn and bfloat16 encoders/decoders written from the
  format definitions, the per-tensor absmax quantizer and its folded query
  scale.
* ``attention`` -- exact causal softmax attention in float64 on dequantized
  inputs: O and the natural-log log-sum-exp, for whole tensors or for
  selected rows.
* ``rotation``  -- the Hadamard rotation of Q and K ahead of the FP8 cast
  (aicronaca.it, section "Perché l'FP8 non basta da solo").

Parity status: every function here is pinned by ``tests/test_oracle.py``
(format tables against torch's casts and the pages' +8-per-doubling fact;
attention against brute force, closed forms and invariants) and
``tests/test_oracle_rotation.py`` (Hadamard matrices against scipy and the
closed form, rotation against a brute force, a hand-worked one-hot case,
score invariance and the page's error claim).
"""

from .formats import (
    E4M3_MAX,
    e4m3fn_decode,
    e4m3fn_encode,
    bf16_decode,
    bf16_encode,
    quantize_fp8_per_tensor,
    per_tensor_scale,
    per_tensor_scale_folded,
    encode_with_scale,
    dequantize_fp8,
)
from .attention import (
    causal_attention,
    attention_rows,
    prefill_reference,
)

__all__ = [
    "E4M3_MAX",
    "e4m3fn_decode",
    "e4m3fn_encode",
    "bf16_decode",
    "bf16_encode",
    "quantize_fp8_per_tensor",
    "per_tensor_scale",
    "per_tensor_scale_folded",
    "encode_with_scale",
    "dequantize_fp8",
    "causal_attention",
    "attention_rows",
    "prefill_reference",
]
